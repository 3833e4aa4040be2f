// The long-range decode step of one (sequence, head) as a device function,
// shared by the decode and chunked-prefill kernels and the fused attention
// decode kernel (FreeSolo, Sec. 3.3 "Inference"; App. C "Bounded cache",
// Eq. 15).  The record layout and its helpers live here too.
#pragma once

#include "fsl_internal.h"

#include <climits>

namespace fsl {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kS = 32;          // tokens per cell
constexpr int kB = 128;         // tokens per query block
constexpr int kCpb = kB / kS;   // cells per block
constexpr int kKmax = 8;

template <typename T>
__device__ __forceinline__ float elem_to_f32(T x);
template <>
__device__ __forceinline__ float elem_to_f32<uint16_t>(uint16_t x) { return bf16_bits_to_f32(x); }
template <>
__device__ __forceinline__ float elem_to_f32<float>(float x) { return x; }

// n contiguous elements (n * sizeof(T) a multiple of 16 bytes, 16-byte aligned) -> fp32.
template <typename T, int n>
__device__ __forceinline__ void load_row_f32(const T *__restrict__ p, float (&x)[n])
{
    constexpr int EPC = 16 / (int)sizeof(T);
    static_assert(n % EPC == 0, "16-byte chunks");
#pragma unroll
    for (int c = 0; c < n / EPC; ++c) {
        const u32x4 w = *reinterpret_cast<const u32x4 *>(p + c * EPC);
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[c * 8 + 2 * e] = bf16_bits_to_f32(w[e] & 0xffffu);
                x[c * 8 + 2 * e + 1] = bf16_bits_to_f32(w[e] >> 16);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                x[c * 4 + e] = __uint_as_float(w[e]);
        }
    }
}

// Order-preserving integer images of the two rankings (a larger key ranks first):
//   TopP by (norm desc, id asc): norm_key;
//   top-K by (score desc, id asc): rank_key of the fp32 score above
//   127 - (position in A) -- exact, since positions in A follow cell ids.

// Number of keys in k[0 .. n8) (n8 a multiple of 8, entries past the live ones
// zero) that are larger than `mine`: the rank of `mine` among distinct keys.
__device__ __forceinline__ int count_greater(const uint64_t *k, int n8, uint64_t mine)
{
    int r = 0;
#pragma unroll 4
    for (int x = 0; x < n8; x += 8) {
        uint64_t v[8];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const u32x4 w = *reinterpret_cast<const u32x4 *>(k + x + e);
            v[e] = ((uint64_t)w[1] << 32) | w[0];
            v[e + 1] = ((uint64_t)w[3] << 32) | w[2];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
            r += v[e] > mine ? 1 : 0;
    }
    return r;
}

struct Record {
    StateMeta *meta;
    int32_t *ridx, *cell, *flags;
    float *a, *kbar;
    char *k, *v;
};

__device__ __forceinline__ Record record_at(char *state, const StateLayout &L, int64_t bh)
{
    char *rec = state + kStateHeaderBytes + bh * L.rec_bytes;
    Record R;
    R.meta = reinterpret_cast<StateMeta *>(rec);
    R.ridx = reinterpret_cast<int32_t *>(rec + L.off_ridx);
    R.cell = reinterpret_cast<int32_t *>(rec + L.off_cell);
    R.flags = reinterpret_cast<int32_t *>(rec + L.off_flags);
    R.a = reinterpret_cast<float *>(rec + L.off_a);
    R.kbar = reinterpret_cast<float *>(rec + L.off_kbar);
    R.k = rec + L.off_k;
    R.v = rec + L.off_v;
    return R;
}

// ------------------------------------------------------------------------
// One decode step.  Latency, not bandwidth, bounds a step: one workgroup per
// (sequence, head) moves ~100 KB through a chain of dependent phases.  So the
// loads the step can know of at entry -- the slot tables, the token, the gain
// and every slot's mean key -- are issued at once, with no branch between the
// loads and their first use (a divergent branch makes the compiler wait for a
// load inside it).  Right after the first barrier each wave requests the keys
// and values of the cell it read at the previous step: the record keeps that
// slot per wave as a hint.  Queries of one head keep choosing the same
// high-norm cells in the same order, so the hint is usually right and the
// gather overlaps the scoring instead of following it.  The prefetched rows
// are used only if the hinted slot is selected again at the same rank, and the
// rows of a selected cell never change (only the cell being filled is written,
// and it is not in A), so no result depends on the hint.  Ranks (Eq. 15 merge,
// top-K) are counted over 64-bit integer keys in LDS; the top-K is taken per
// wave first and then over the waves' candidates.  Each selected cell's
// softmax partials are kept apart by rank, and wave 0 combines them in rank
// order, so outputs are bitwise the same whichever wave read which cell.
//
// CHUNK: the same steps for n_tok consecutive tokens of every record in one
// launch (a chunk of a prompt prefilled into the state, App. C "Bounded cache":
// the bounded cache is prefilled in fixed-size chunks with the retention update
// at every block boundary).  Token tau of record bh is row bh * n_tok + tau of
// q, k_new, v_new, out and sel; the steps run in order, so the results are
// those of n_tok single steps.
//
// FUSED (the fused attention decode kernel, whose other waves run the local
// branch): one step whose output stays in LDS (s_olr, rounded to T as the
// standalone step would store it; NaN for a foreign state).  The step's four
// waves then meet at barriers of their own (waves_barrier on the LDS counter
// s_bar) instead of the workgroup's, so the other waves are never held by
// them, and a foreign state does not end the waves early.
enum : int { kDecodeStep = 0, kDecodeChunk = 1, kDecodeFused = 2 };

// A barrier of `waves` waves of a workgroup, on an LDS counter that starts at 0
// (set before a workgroup barrier) and that only these waves advance: each
// wave adds one and waits until the counter reaches `target` (waves times the
// number of such barriers passed so far, this one included).  Every one of the
// waves passes the same barriers, so every wait ends.  LDS operations complete
// in order, so the release (all earlier LDS accesses of the wave done) and the
// acquire make the waves' LDS writes before the barrier visible after it.
__device__ __forceinline__ void waves_barrier(uint32_t *ctr, uint32_t target)
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (__lane_id() == 0)
        __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target)
        __builtin_amdgcn_s_sleep(1);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

template <typename T, int D, int MODE>
__device__ __forceinline__ void decode_step_body(char *__restrict__ state, const StateLayout &L,
                                                 const StateHeader &expect, const HeadConsts &hc,
                                                 const T *__restrict__ q, const T *__restrict__ k_new,
                                                 const T *__restrict__ v_new, const float *__restrict__ gain,
                                                 T *__restrict__ out, int32_t *__restrict__ sel, int H, int K, int P,
                                                 int W, float eps, int n_tok, float *__restrict__ s_olr,
                                                 uint32_t *s_bar)
{
    constexpr bool CHUNK = MODE == kDecodeChunk;
    constexpr bool FUSED = MODE == kDecodeFused;
    uint32_t bar_target = 0;
    auto step_sync = [&]() { // the step's waves only when fused, else the workgroup
        if constexpr (FUSED) {
            bar_target += kWaves;
            waves_barrier(s_bar, bar_target);
        } else {
            __syncthreads();
        }
    };
    constexpr int EPC = 16 / (int)sizeof(T); // elements per 16-byte chunk
    constexpr int CPR = D / EPC;             // chunks per row
    constexpr int RG = kWave / CPR;          // value rows per load step
    constexpr int VR = kS / RG;              // value chunks per lane
    constexpr int HALF = D / 2;              // key features per lane (two lanes per token)
    constexpr int KC = HALF / EPC;           // key chunks per lane
    constexpr int FPT = D / 2;               // mean-key features per thread while scoring
    constexpr int NCAND = kWaves * kKmax;    // the waves' top-K candidates
    constexpr int SPW = kWave / 2;           // slots scored per wave (two threads per slot)
    // a cell is prefetched when a lane's share of it fits in 64 registers
    constexpr bool kPrefetch = KC + VR <= 16;
    static_assert(kWaves == kStateHints, "one prefetch hint per wave");
    static_assert(SPW * kWaves == kMaxSlots, "every slot has two scoring threads");
    static_assert(kThreads % kMaxSlots == 0 && kThreads % D == 0, "threads cover the slots and features evenly");

    __shared__ int32_t s_cell[kMaxSlots], s_flags[kMaxSlots], s_ridx[kMaxSlots];
    __shared__ __attribute__((aligned(16))) int32_t s_kc[kMaxSlots]; // kept cell ids (merge), read 4 at a time
    __shared__ float s_a[kMaxSlots];
    __shared__ __attribute__((aligned(16))) uint64_t s_key[kMaxSlots]; // merge keys, then score keys, by slot
    __shared__ __attribute__((aligned(16))) uint64_t s_cand[NCAND];   // per wave: its K best score keys
    __shared__ int32_t s_pos_slot[kMaxSlots];                         // slot of each position in A
    __shared__ int32_t s_selw[kWaves][kKmax];                         // per wave: the selected slots by rank
    __shared__ float s_q[D];
    __shared__ __attribute__((aligned(16))) T s_qt[D]; // q as given (bf16 pairs feed dot2)
    __shared__ T s_knew[D];
    __shared__ T s_vnew[D];
    __shared__ float s_upart[kKmax][RG * D]; // per selected cell (by rank) and value-row group: partial P.V
    __shared__ float s_m[kKmax], s_z[kKmax];
    __shared__ double s_colsum[kWaves][D];
    __shared__ double s_rowmax[kWaves];
    __shared__ int32_t s_wcnt[kWaves];
    static_assert(kWaves == 4, "the kept-cell count adds four wave counts");

    const int64_t bh = blockIdx.x;
    const int h = (int)(bh % H);
    const int t = threadIdx.x, lane = t & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(t / kWave); // wave-uniform, kept in a scalar register
    const Record R = record_at(state, L, bh); // in bounds: the host checked the buffer size
    T *sk = reinterpret_cast<T *>(R.k);
    T *sv = reinterpret_cast<T *>(R.v);
    const int vrow0 = lane / CPR, vch = lane % CPR;
    const int steps = CHUNK ? n_tok : 1;
  for (int step = 0; step < steps; ++step) {
    const int64_t tok = CHUNK ? bh * (int64_t)n_tok + step : bh; // this step's row of q, k_new, v_new, out, sel
    T *o_row = FUSED ? nullptr : out + tok * D; // the fused kernel keeps the output in s_olr

    // ---- (a) entry: all loads first (clamped indices, no branches), then their uses ----
    // Threads t and t + 128 (t + D) load and store the same slot (feature), so the
    // LDS stores need no branch for the compiler to sink the loads into.
    constexpr int FPL = D / kWave; // output features per lane of wave 0
    const int td = t & (D - 1);
    float g_in[FPL]; // gain of the output features of lane (t % 64); first: its branch must precede the others
#pragma unroll
    for (int j = 0; j < FPL; ++j)
        g_in[j] = gain ? gain[(int64_t)h * D + FPL * lane + j] : 1.0f;
    const StateHeader hv = *reinterpret_cast<const StateHeader *>(state);
    const StateMeta mv = *R.meta;
    const int tt = t & (kMaxSlots - 1);
    const bool t_in = tt < L.S;
    const int ts = t_in ? tt : 0; // L.S >= 1
    const int32_t cell_in = R.cell[ts], flags_in = R.flags[ts], ridx_in = R.ridx[ts];
    const float a_in = R.a[ts];
    const T q_in = q[tok * D + td], k_in = k_new[tok * D + td], v_in = v_new[tok * D + td];
    const int my_slot = t >> 1, my_part = t & 1;
    const int ks = my_slot < L.S ? my_slot : 0;
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);
    u32x4 kbraw[FPT / 4];
#pragma unroll
    for (int c = 0; c < FPT / 4; ++c)
        kbraw[c] = *reinterpret_cast<const u32x4 *>(R.kbar + (int64_t)ks * D + my_part * FPT + 4 * c);
    int my_hint = mv.hint[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w)
        my_hint = wave == w ? mv.hint[w] : my_hint;
    my_hint = kPrefetch && my_hint >= 0 && my_hint < L.S ? my_hint : -1;
    u32x4 kraw[KC], vraw[VR];
    const int bad = (int)(hv.magic != kStateMagic) | (int)(hv.version != kStateVersion) |
                    (int)(hv.batch != expect.batch) | (int)(hv.H != expect.H) | (int)(hv.d != D) |
                    (int)(hv.dtype != expect.dtype) | (int)(hv.P != P) | (int)(hv.W != W) |
                    (int)(hv.n_slots != L.S) | (int)(hv.rec_bytes != L.rec_bytes);
    if (!FUSED && bad) { // not a state of this shape: flag the outputs, leave the state alone
        for (int s2 = step; s2 < steps; ++s2) {
            const int64_t tk = CHUNK ? bh * (int64_t)n_tok + s2 : bh;
            if (t < D) {
                if constexpr (sizeof(T) == 2)
                    out[tk * D + t] = (T)0x7fc0u; // bf16 quiet NaN
                else
                    out[tk * D + t] = __uint_as_float(0x7fc00000u);
            }
            if (sel && t < K)
                sel[tk * K + t] = -1;
        }
        return; // the header is the same for every thread: the whole workgroup leaves
    }
    s_cell[tt] = t_in ? cell_in : -1;
    s_flags[tt] = t_in ? flags_in : 0;
    s_a[tt] = t_in ? a_in : 0.0f;
    s_ridx[tt] = t_in ? ridx_in : -1;
    s_pos_slot[tt] = 0;
    if (t < NCAND) {
        s_cand[t] = 0;                 // empty candidates rank last
        s_selw[t / kKmax][t % kKmax] = 0; // slot 0 for any rank a corrupted state leaves unlisted
    }
    {
        const float qf = elem_to_f32<T>(q_in);
        s_q[td] = qf;
        s_qt[td] = q_in;
        s_knew[td] = k_in;
        s_vnew[td] = v_in;
    }
    const int64_t i = mv.pos;
    int n_ret = mv.n_ret < 0 ? 0 : (mv.n_ret > L.S ? L.S : mv.n_ret);
    int cur = mv.cur_slot;
    step_sync();
    // The cell prefetch goes out only now: issued with the loads above, it delayed
    // them (and the barrier) by the whole step's traffic; from here it overlaps
    // the scoring and top-K.
    if constexpr (kPrefetch) { // slot 0 stands in for a missing hint: the read is wasted, never used
        const int ps = my_hint >= 0 ? my_hint : 0;
        const T *kc = sk + (int64_t)ps * kS * D + (int64_t)(lane >> 1) * D + (lane & 1) * HALF;
        const T *vc = sv + (int64_t)ps * kS * D + (int64_t)vrow0 * D + vch * EPC;
#pragma unroll
        for (int x = 0; x < KC; ++x)
            kraw[x] = *reinterpret_cast<const u32x4 *>(kc + x * EPC);
#pragma unroll
        for (int x = 0; x < VR; ++x)
            vraw[x] = *reinterpret_cast<const u32x4 *>(vc + (int64_t)RG * x * D);
    }

    const int64_t beta = i / kB;
    const int r = (int)(i % kS);
    const int64_t c_new = i / kS;

    // ---- (1) block boundary: Eq. 15 merge, then A = TopP u Recent_W ----
    const bool keep_state = !(FUSED && bad); // a foreign state is never written (elsewhere it has returned)
    const bool merge = keep_state && i % kB == 0 && i > 0;
    if (merge) {
        const int64_t d_lo = (beta - 1) * kCpb, d_hi = beta * kCpb;
        const int64_t rec_lo = d_hi > W ? d_hi - W : 0;
        const int S8 = (L.S + 7) & ~7;
        int32_t c = -1;
        bool cand = false;
        uint64_t my = 0;
        if (t < kMaxSlots) {
            c = s_cell[t];
            cand = c >= 0 && ((s_flags[t] & kFlagTop) || (c >= d_lo && c < d_hi));
            my = cand ? norm_key(s_a[t], c) : 0;
            s_key[t] = my;
        }
        step_sync();
        // rank among TopP(C) u D by (a desc, id asc)
        const bool top = cand && count_greater(s_key, S8, my) < P;
        const bool keep = c >= 0 && (top || (c >= rec_lo && c < d_hi));
        if (t < kMaxSlots) {
            s_flags[t] = top ? kFlagTop : 0;
            s_cell[t] = keep ? c : -1;
            s_kc[t] = keep ? c : INT_MAX;
        }
        step_sync();
        int pos = -1;
        if (keep) { // position in A: kept cells with a smaller id
            pos = 0;
            for (int u = 0; u < S8; u += 4) {
                const u32x4 w = *reinterpret_cast<const u32x4 *>(&s_kc[u]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    pos += (int32_t)w[e] < c ? 1 : 0;
            }
        }
        if (t < kMaxSlots)
            s_ridx[t] = pos;
        if constexpr (FUSED) { // |A|: the kept cells, counted per wave, summed after the step's barrier
            const uint64_t kept = __ballot(keep);
            if (lane == 0)
                s_wcnt[wave] = __popcll(kept);
            step_sync();
            n_ret = (s_wcnt[0] + s_wcnt[1]) + (s_wcnt[2] + s_wcnt[3]);
        } else {
            n_ret = __syncthreads_count(keep);
        }
        if (t < L.S) {
            R.cell[t] = s_cell[t];
            R.flags[t] = s_flags[t];
            R.ridx[t] = pos;
        }
        if (t == 0)
            R.meta->n_ret = n_ret;
    }

    // ---- (2) append the token; a new cell takes the lowest free slot ----
    if (keep_state && r == 0) {
        const uint64_t f0 = __ballot(lane < L.S && s_cell[lane] < 0);
        const uint64_t f1 = __ballot(lane + kWave < L.S && s_cell[lane + kWave] < 0);
        cur = f0 ? __ffsll((unsigned long long)f0) - 1 : (f1 ? kWave + __ffsll((unsigned long long)f1) - 1 : -1);
        if (t == 0 && cur >= 0) {
            R.cell[cur] = (int32_t)c_new;
            R.flags[cur] = 0;
            R.ridx[cur] = -1;
            R.meta->cur_slot = cur;
        }
    }
    const bool can_append = keep_state && cur >= 0 && cur < L.S; // false only for a corrupted state
    if (can_append && t < D) {
        sk[((int64_t)cur * kS + r) * D + t] = s_knew[t];
        sv[((int64_t)cur * kS + r) * D + t] = s_vnew[t];
    }
    const bool complete = r == kS - 1 && can_append;
    if (complete) {
        // Eq. 5 for the completed cell: rows 0..s-2 from the slot, row s-1 from this token
        constexpr int FP = D / 8;
        const int row = t >> 3, part = t & 7;
        float x[FP];
        if (row == kS - 1) {
#pragma unroll
            for (int e = 0; e < FP; ++e)
                x[e] = elem_to_f32<T>(s_knew[part * FP + e]);
        } else {
            load_row_f32<T, FP>(sk + ((int64_t)cur * kS + row) * D + part * FP, x);
        }
        double col[FP];
        double sq = 0.0;
#pragma unroll
        for (int e = 0; e < FP; ++e) {
            col[e] = (double)x[e];
            sq += col[e] * col[e];
        }
        sq += shfl_xor_d(sq, 1);
        sq += shfl_xor_d(sq, 2);
        sq += shfl_xor_d(sq, 4);
        double mx = sq;
#pragma unroll
        for (int m = 8; m < kWave; m <<= 1)
            mx = fmax(mx, shfl_xor_d(mx, m));
#pragma unroll
        for (int e = 0; e < FP; ++e) {
#pragma unroll
            for (int m = 8; m < kWave; m <<= 1)
                col[e] += shfl_xor_d(col[e], m);
        }
        if (lane < 8) {
#pragma unroll
            for (int e = 0; e < FP; ++e)
                s_colsum[wave][part * FP + e] = col[e];
        }
        if (lane == 0)
            s_rowmax[wave] = mx;
        step_sync();
        if (t < D)
            R.kbar[(int64_t)cur * D + t] =
                (float)(((s_colsum[0][t] + s_colsum[1][t]) + (s_colsum[2][t] + s_colsum[3][t])) * (1.0 / 32.0));
        if (t == 0)
            R.a[cur] = (float)sqrt(fmax(fmax(s_rowmax[0], s_rowmax[1]), fmax(s_rowmax[2], s_rowmax[3])));
    }

    // ---- (3) Eq. 7 over A, in fp32 as the prefill scores; each wave keeps the K best of its slots ----
    const int ri = s_ridx[my_slot]; // my_slot < kMaxSlots; -1 past L.S
    const bool scored = ri >= 0 && ri < n_ret;
    float part4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < FPT / 4; ++c) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            part4[e] = fmaf(s_q[my_part * FPT + 4 * c + e], __uint_as_float(kbraw[c][e]), part4[e]);
    }
    float dot = (part4[0] + part4[1]) + (part4[2] + part4[3]);
    dot += dpp_f<0xB1>(dot); // the slot's other half (lanes 2j, 2j + 1)
    uint64_t key = 0;
    if (scored && my_part == 0) {
        const int32_t c = s_cell[my_slot];
        // (i - p_c) / (2 sigma_h) with i - p_c exact below 2^24; erf rounds to 1 in fp32 from 4 on
        const float x = (float)(i - ((int64_t)c * kS + kS / 2)) * hc.inv_two_sigma[h];
        const float g = x < 4.0f ? erff(x) : 1.0f;
        const float score = fmaf(hc.lambda[h] * s_a[my_slot], g, dot * inv_sqrt_d);
        key = rank_key(score, 127u - (uint32_t)ri); // ties: the smaller position in A (the smaller id) first
        s_pos_slot[ri] = my_slot;
    }
    if (my_part == 0)
        s_key[my_slot] = key;
    // the wave reads back only what its own lanes wrote: a wave-level barrier orders it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (key != 0) {
        const int rk = count_greater(s_key + wave * SPW, SPW, key);
        if (rk < K)
            s_cand[wave * kKmax + rk] = key;
    }
    step_sync();

    // ---- top-K over the candidates (score desc, id asc), taken by every wave ----
    // Each wave lists the selected slots by rank in its own LDS row, then reads it back.
    {
        const uint64_t ck = lane < NCAND ? s_cand[lane] : 0;
        const int grank = ck != 0 ? count_greater(s_cand, NCAND, ck) : NCAND;
        if (grank < K) {
            const int sl = s_pos_slot[127 - (int)((uint32_t)ck & 0x7fu)];
            s_selw[wave][grank] = sl >= 0 && sl < L.S ? sl : 0;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int nT = n_ret < K ? n_ret : K;
    // wave w reads out ranks w and w + 4; the slot at rank w is its next hint
    const int rk0 = wave, rk1 = wave + kWaves;
    const int slot0 = __builtin_amdgcn_readfirstlane(rk0 < nT ? s_selw[wave][rk0] : -1);
    const int slot1 = __builtin_amdgcn_readfirstlane(rk1 < nT ? s_selw[wave][rk1] : -1);
    const int32_t sel_cell = t < nT ? s_cell[s_selw[0][t < kKmax ? t : 0]] : -1; // for lanes t < K of wave 0

    // ---- (b) readout (Eq. 9): one cell per pass, its softmax partials stored by rank ----
    auto read_cell = [&](int rk, int slot, bool have) {
        if (!have) {
            const T *kc = sk + (int64_t)slot * kS * D + (int64_t)(lane >> 1) * D + (lane & 1) * HALF;
            const T *vc = sv + (int64_t)slot * kS * D + (int64_t)vrow0 * D + vch * EPC;
#pragma unroll
            for (int x = 0; x < KC; ++x)
                kraw[x] = *reinterpret_cast<const u32x4 *>(kc + x * EPC);
#pragma unroll
            for (int x = 0; x < VR; ++x)
                vraw[x] = *reinterpret_cast<const u32x4 *>(vc + (int64_t)RG * x * D);
        }
        float lp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int x = 0; x < KC; ++x) {
            if constexpr (sizeof(T) == 2) {
                const u32x4 qw = *reinterpret_cast<const u32x4 *>(&s_qt[(lane & 1) * HALF + x * EPC]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t qe = qw[e], ke = kraw[x][e]; // named copies: a bit_cast of an element in place reads element 0
                    lp[e] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qe),
                                                            __builtin_bit_cast(bf16x2, ke), lp[e], false);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    lp[e] = fmaf(s_q[(lane & 1) * HALF + x * EPC + e], __uint_as_float(kraw[x][e]), lp[e]);
            }
        }
        float l = (lp[0] + lp[1]) + (lp[2] + lp[3]);
        l = (l + dpp_f<0xB1>(l)) * inv_sqrt_d; // logit of token lane / 2, on both lanes of the pair
        const float mx = wave_max_f(l);
        const float p = expf(l - mx);
        const float z = wave_sum_f((lane & 1) ? 0.0f : p);
        float acc[EPC];
#pragma unroll
        for (int e = 0; e < EPC; ++e)
            acc[e] = 0.0f;
#pragma unroll
        for (int x = 0; x < VR; ++x) {
            const float pr = __shfl(p, 2 * (vrow0 + RG * x), kWave);
            if constexpr (sizeof(T) == 2) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[2 * e] = fmaf(pr, bf16_bits_to_f32(vraw[x][e] & 0xffffu), acc[2 * e]);
                    acc[2 * e + 1] = fmaf(pr, bf16_bits_to_f32(vraw[x][e] >> 16), acc[2 * e + 1]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[e] = fmaf(pr, __uint_as_float(vraw[x][e]), acc[e]);
            }
        }
#pragma unroll
        for (int e = 0; e < EPC; ++e)
            s_upart[rk][vrow0 * D + vch * EPC + e] = acc[e];
        if (lane == 0) {
            s_m[rk] = mx;
            s_z[rk] = z;
        }
    };
    if (slot0 >= 0)
        read_cell(rk0, slot0, slot0 == my_hint);
    if (slot1 >= 0)
        read_cell(rk1, slot1, false);
    if (kPrefetch && keep_state && lane == 0)
        R.meta->hint[wave] = slot0;
    step_sync();

    // ---- wave 0: combine the cells in rank order, normalise, RMSNorm over d (Eq. 17), write ----
    if (MODE == kDecodeStep && wave != 0)
        return;
    if (wave == 0) {
    float u[FPL];
#pragma unroll
    for (int j = 0; j < FPL; ++j)
        u[j] = 0.0f;
    if (nT > 0) {
        float M = s_m[0];
#pragma unroll
        for (int q8 = 1; q8 < kKmax; ++q8)
            M = q8 < nT ? fmaxf(M, s_m[q8]) : M;
        float Z = 0.0f, U[FPL];
#pragma unroll
        for (int j = 0; j < FPL; ++j)
            U[j] = 0.0f;
#pragma unroll
        for (int q8 = 0; q8 < kKmax; ++q8) {
            if (q8 < nT) {
                const float f = expf(s_m[q8] - M);
                Z = fmaf(s_z[q8], f, Z);
#pragma unroll
                for (int j = 0; j < FPL; ++j) {
                    float uw = 0.0f;
#pragma unroll
                    for (int g = 0; g < RG; ++g)
                        uw += s_upart[q8][g * D + FPL * lane + j];
                    U[j] = fmaf(uw, f, U[j]);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < FPL; ++j)
            u[j] = U[j] / Z;
    }
    float sq = 0.0f;
#pragma unroll
    for (int j = 0; j < FPL; ++j)
        sq = fmaf(u[j], u[j], sq);
    const float rs = 1.0f / sqrtf(wave_sum_f(sq) / (float)D + eps);
#pragma unroll
    for (int j = 0; j < FPL; ++j) {
        const float y = nT > 0 ? g_in[j] * u[j] * rs : 0.0f;
        if constexpr (FUSED) { // the output as the standalone step would store it, or NaN for a foreign state
            const float yr = sizeof(T) == 2 ? bf16_bits_to_f32(f32_to_bf16_bits(y)) : y;
            s_olr[FPL * lane + j] = bad ? __uint_as_float(0x7fc00000u) : yr;
        } else if constexpr (sizeof(T) == 2) {
            o_row[FPL * lane + j] = (T)f32_to_bf16_bits(y);
        } else {
            o_row[FPL * lane + j] = y;
        }
    }
    if (sel && t < K)
        sel[tok * K + t] = keep_state ? sel_cell : -1;
    if (keep_state && t == 0)
        R.meta->pos = i + 1;
    }
    if constexpr (CHUNK)
        __syncthreads(); // the next step reads what this one wrote to the record
  }
}

} // namespace
} // namespace fsl
