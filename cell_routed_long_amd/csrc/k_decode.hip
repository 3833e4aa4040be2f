// Streaming decode of the FS-L long-range branch (FreeSolo, Sec. 3.3
// "Inference"; App. C "Bounded cache", Eq. 15).
//
// Per (sequence, head) the state keeps only the cells FS-L can still read: the
// retained set A of the current query block (at most P + W cells) and the
// B/s cells of the block being filled, each in a fixed-size slot holding its
// raw keys and values, fp32 mean key and norm.  One step, for a token at
// position i, is one launch with one workgroup per (sequence, head):
//   (1) i a block start (i % B == 0, i > 0): the B/s cells that just became
//       eligible (D) are merged into TopP by rank among TopP(C) u D (Eq. 15:
//       TopP(C u D) = TopP(TopP(C) u D)); A = TopP u Recent_W; every slot whose
//       cell is in neither is freed (a discarded cell can never re-enter TopP);
//   (2) the token's key and value are written into its cell's slot (a free
//       slot is taken when a cell starts); when the token completes the cell,
//       its mean key and largest key norm (Eq. 5) are formed in fp64 and
//       rounded once, exactly as the prefill summary kernel does;
//   (3) q is scored against A in fp64 (Eq. 7), its top-K cells are chosen by
//       rank (score desc, id asc), and the readout (Eq. 9) with RMSNorm
//       (Eq. 17) runs over their tokens: each wave gathers one selected cell
//       and keeps a running softmax (max, sum, weighted values) that the waves
//       combine at the end, so the readout needs a single barrier.
// All branching on the position happens on the device, so a step can be
// captured in a HIP graph.  The prefill builds the state directly from its
// exit blocks (state_build_kernel), so no merge chain is replayed.
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
//   TopP by (norm desc, id asc): the fp32 norm's bits (made monotone) above the
//   complemented id -- exact;
//   top-K by (score desc, id asc): the fp64 score's bits made monotone, with the
//   lowest 7 bits replaced by 127 - (position in A).  Positions in A follow cell
//   ids, so scores within 2^-45 (relative) of each other count as tied and go to
//   the smaller id; the numerical error of any score is far larger than that.
__device__ __forceinline__ uint64_t norm_key(float a, int32_t cell)
{
    uint32_t u = __float_as_uint(a);
    u = (u >> 31) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)(0x7fffffff - cell);
}
__device__ __forceinline__ uint64_t score_key(double sc, int pos)
{
    uint64_t u = (uint64_t)__double_as_longlong(sc);
    u = (u >> 63) ? ~u : (u | 0x8000000000000000ull);
    return (u & ~(uint64_t)0x7f) | (uint64_t)(127 - pos);
}

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
// State from a prefill of N tokens: the query block of the last prompt token
// is beta = (N - 1) / B.  Its retained set is A_beta = {c < nav : c leaves
// TopP after beta} u Recent_W, nav = |C_beta|; the cells of block beta itself
// (the last one possibly partial) are pending.  Retained cells take slots
// 0..|A|-1 in ascending id order, pending cells the next ones.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void state_build_kernel(char *__restrict__ state, StateLayout L,
                                                               StateHeader hdr, const T *__restrict__ k,
                                                               const T *__restrict__ v,
                                                               const float *__restrict__ kbar,
                                                               const float *__restrict__ a,
                                                               const int32_t *__restrict__ death, int64_t N,
                                                               int64_t M, int W)
{
    __shared__ int32_t s_cell[kMaxSlots];
    __shared__ int32_t s_flags[kMaxSlots];
    __shared__ int32_t s_wcnt[kWaves];
    __shared__ int32_t s_count;

    const int64_t bh = blockIdx.x;
    const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
    if (bh == 0 && t == 0)
        *reinterpret_cast<StateHeader *>(state) = hdr;
    const Record R = record_at(state, L, bh);
    const int32_t *dh = M > 0 ? death + bh * M : nullptr;
    const int64_t beta = (N - 1) / kB;
    const int64_t nav = beta * kCpb < M ? beta * kCpb : M;
    const int64_t recent0 = nav > W ? nav - W : 0;

    for (int x = t; x < kMaxSlots; x += kThreads) {
        s_cell[x] = -1;
        s_flags[x] = 0;
    }
    if (t == 0)
        s_count = 0;
    __syncthreads();
    // non-recent cells still in TopP(C_beta), ascending: block-wide compaction
    for (int64_t base = 0; base < recent0; base += kThreads) {
        const int64_t c = base + t;
        const bool keep = c < recent0 && dh[c] > beta;
        const uint64_t m = __ballot(keep);
        if (lane == 0)
            s_wcnt[wave] = __popcll(m);
        __syncthreads();
        int off = s_count;
        for (int w = 0; w < wave; ++w)
            off += s_wcnt[w];
        const int pos = off + __popcll(m & ((1ull << lane) - 1ull));
        if (keep && pos < L.S) {
            s_cell[pos] = (int32_t)c;
            s_flags[pos] = kFlagTop;
        }
        __syncthreads();
        if (t == 0) {
            int tot = 0;
            for (int w = 0; w < kWaves; ++w)
                tot += s_wcnt[w];
            s_count += tot;
        }
        __syncthreads();
    }
    const int n_old = s_count < L.S ? s_count : L.S;
    const int n_rec = (int)(nav - recent0);
    const int64_t p0 = beta * kCpb, p1 = (N + kS - 1) / kS;
    const int n_pend = (int)(p1 - p0);
    const int n_A = n_old + n_rec;
    // the host sizes S = P + W + B/s, so n_A + n_pend <= S always holds
    for (int x = t; x < n_rec; x += kThreads) {
        const int64_t c = recent0 + x;
        if (n_old + x < L.S) {
            s_cell[n_old + x] = (int32_t)c;
            s_flags[n_old + x] = dh[c] > beta ? kFlagTop : 0;
        }
    }
    for (int x = t; x < n_pend; x += kThreads)
        if (n_A + x < L.S)
            s_cell[n_A + x] = (int32_t)(p0 + x);
    __syncthreads();

    for (int x = t; x < L.S; x += kThreads) {
        const int32_t c = s_cell[x];
        R.cell[x] = c;
        R.flags[x] = s_flags[x];
        R.a[x] = (c >= 0 && c < M) ? a[bh * M + c] : 0.0f;
        R.ridx[x] = x < n_A ? x : -1;
    }
    if (t == 0) {
        R.meta->pos = N;
        R.meta->n_ret = n_A;
        R.meta->cur_slot = (N % kS) != 0 ? n_A + n_pend - 1 : -1;
    }
    for (int e = t; e < L.S * D; e += kThreads) {
        const int x = e / D, f = e % D;
        const int32_t c = s_cell[x];
        R.kbar[e] = (c >= 0 && c < M) ? kbar[(bh * M + c) * D + f] : 0.0f;
    }
    // raw keys and values of every occupied slot, 16-byte chunks
    constexpr int CPR = D * (int)sizeof(T) / 16;
    T *sk = reinterpret_cast<T *>(R.k);
    T *sv = reinterpret_cast<T *>(R.v);
    for (int e = t; e < L.S * kS * CPR; e += kThreads) {
        const int x = e / (kS * CPR);
        const int rem = e % (kS * CPR);
        const int row = rem / CPR, ch = rem % CPR;
        const int32_t c = s_cell[x];
        if (c < 0)
            continue;
        const int64_t j = (int64_t)c * kS + row;
        if (j >= N)
            continue;
        const int64_t src = (bh * N + j) * D;
        const int64_t dst = ((int64_t)x * kS + row) * D;
        reinterpret_cast<u32x4 *>(sk + dst)[ch] = reinterpret_cast<const u32x4 *>(k + src)[ch];
        reinterpret_cast<u32x4 *>(sv + dst)[ch] = reinterpret_cast<const u32x4 *>(v + src)[ch];
    }
}

// ------------------------------------------------------------------------
// One decode step.  Latency, not bandwidth, bounds a step (one workgroup per
// (sequence, head) moves ~100 KB), so the kernel is laid out as two memory
// round trips with no dependent loads in between: (a) the header, position,
// slot tables, token and every slot's mean key, all issued at entry (while
// scoring, thread t owns half t & 1 of slot t >> 1); (b) the selected cells'
// keys and values.  Ranks (Eq. 15 merge, top-K) are counted by every thread
// at once over 64-bit integer keys in LDS; reductions run on the DPP network.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void decode_step_kernel(char *__restrict__ state, StateLayout L,
                                                               StateHeader expect, HeadConsts hc,
                                                               const T *__restrict__ q,
                                                               const T *__restrict__ k_new,
                                                               const T *__restrict__ v_new,
                                                               const float *__restrict__ gain,
                                                               T *__restrict__ out, int32_t *__restrict__ sel,
                                                               int H, int K, int P, int W, float eps)
{
    constexpr int EPC = 16 / (int)sizeof(T); // elements per 16-byte chunk
    constexpr int CPR = D / EPC;             // chunks per row
    constexpr int RG = kWave / CPR;          // value rows per load step
    constexpr int VR = kS / RG;              // value loads per lane
    constexpr int HALF = D / 2;              // key features per lane (two lanes per token)
    constexpr int FPT = D / 2;               // mean-key features per thread while scoring

    __shared__ int32_t s_cell[kMaxSlots], s_flags[kMaxSlots], s_ridx[kMaxSlots];
    __shared__ __attribute__((aligned(16))) int32_t s_kc[kMaxSlots]; // kept cell ids (merge), read 4 at a time
    __shared__ float s_a[kMaxSlots];
    __shared__ __attribute__((aligned(16))) uint64_t s_key[kMaxSlots]; // ranking keys (merge, then top-K)
    __shared__ int32_t s_rc[kMaxSlots];   // cell ids, by position in A
    __shared__ int32_t s_rslot[kMaxSlots];
    __shared__ float s_q[D];
    __shared__ T s_knew[D];
    __shared__ T s_vnew[D];
    __shared__ int32_t s_sel_slot[kKmax], s_sel_cell[kKmax];
    __shared__ float s_upart[kWaves][RG * D]; // per wave and value-row group: partial P.V
    __shared__ float s_m[kWaves], s_z[kWaves];
    __shared__ double s_colsum[kWaves][D];
    __shared__ double s_rowmax[kWaves];
    __shared__ float s_red[kWaves];
    __shared__ int32_t s_int[2];

    const int64_t bh = blockIdx.x;
    const int h = (int)(bh % H);
    const int t = threadIdx.x, lane = t & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(t / kWave); // wave-uniform, kept in a scalar register
    T *o_row = out + bh * D;
    const Record R = record_at(state, L, bh); // in bounds: the host checked the buffer size
    T *sk = reinterpret_cast<T *>(R.k);
    T *sv = reinterpret_cast<T *>(R.v);

    // ---- (a) entry loads: header, position, slot tables, token, mean keys ----
    const StateHeader hv = *reinterpret_cast<const StateHeader *>(state);
    const StateMeta mv = *R.meta;
    if (t < kMaxSlots) {
        const bool in = t < L.S;
        s_cell[t] = in ? R.cell[t] : -1;
        s_flags[t] = in ? R.flags[t] : 0;
        s_a[t] = in ? R.a[t] : 0.0f;
        s_ridx[t] = in ? R.ridx[t] : -1;
    }
    if (t < D) {
        s_q[t] = elem_to_f32<T>(q[bh * D + t]);
        s_knew[t] = k_new[bh * D + t];
        s_vnew[t] = v_new[bh * D + t];
    }
    const int my_slot = t >> 1, my_part = t & 1;
    float kb[FPT];
    if (my_slot < L.S) {
        load_row_f32<float, FPT>(R.kbar + (int64_t)my_slot * D + my_part * FPT, kb);
    } else {
#pragma unroll
        for (int e = 0; e < FPT; ++e)
            kb[e] = 0.0f;
    }
    const int bad = (int)(hv.magic != kStateMagic) | (int)(hv.version != kStateVersion) |
                    (int)(hv.batch != expect.batch) | (int)(hv.H != expect.H) | (int)(hv.d != D) |
                    (int)(hv.dtype != expect.dtype) | (int)(hv.P != P) | (int)(hv.W != W) |
                    (int)(hv.n_slots != L.S) | (int)(hv.rec_bytes != L.rec_bytes);
    if (bad) { // not a state of this shape: flag the output, leave the state alone
        if (t < D) {
            if constexpr (sizeof(T) == 2)
                o_row[t] = (T)0x7fc0u; // bf16 quiet NaN
            else
                o_row[t] = __uint_as_float(0x7fc00000u);
        }
        if (sel && t < K)
            sel[bh * K + t] = -1;
        return;
    }
    const int64_t i = mv.pos;
    int n_ret = mv.n_ret < 0 ? 0 : (mv.n_ret > L.S ? L.S : mv.n_ret);
    int cur = mv.cur_slot;
    __syncthreads();

    const int64_t beta = i / kB;
    const int r = (int)(i % kS);
    const int64_t c_new = i / kS;

    // ---- (1) block boundary: Eq. 15 merge, then A = TopP u Recent_W ----
    if (i % kB == 0 && i > 0) {
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
        __syncthreads();
        // rank among TopP(C) u D by (a desc, id asc)
        const bool top = cand && count_greater(s_key, S8, my) < P;
        const bool keep = c >= 0 && (top || (c >= rec_lo && c < d_hi));
        if (t < kMaxSlots) {
            s_flags[t] = top ? kFlagTop : 0;
            s_cell[t] = keep ? c : -1;
            s_kc[t] = keep ? c : INT_MAX;
        }
        __syncthreads();
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
        n_ret = __syncthreads_count(keep);
        if (t < L.S) {
            R.cell[t] = s_cell[t];
            R.flags[t] = s_flags[t];
            R.ridx[t] = pos;
        }
        if (t == 0)
            R.meta->n_ret = n_ret;
    }

    // ---- (2) append the token; a new cell takes the lowest free slot ----
    if (r == 0) {
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
    const bool can_append = cur >= 0 && cur < L.S; // false only for a corrupted state
    if (can_append && t < D) {
        sk[((int64_t)cur * kS + r) * D + t] = s_knew[t];
        sv[((int64_t)cur * kS + r) * D + t] = s_vnew[t];
    }
    if (r == kS - 1 && can_append) {
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
        __syncthreads();
        if (t < D)
            R.kbar[(int64_t)cur * D + t] =
                (float)(((s_colsum[0][t] + s_colsum[1][t]) + (s_colsum[2][t] + s_colsum[3][t])) * (1.0 / 32.0));
        if (t == 0)
            R.a[cur] = (float)sqrt(fmax(fmax(s_rowmax[0], s_rowmax[1]), fmax(s_rowmax[2], s_rowmax[3])));
    }

    // ---- (3) Eq. 7 over A in fp64 ----
    const int ri = my_slot < L.S ? s_ridx[my_slot] : -1;
    const bool scored = ri >= 0 && ri < n_ret;
    double dot = 0.0;
    if (scored) {
        double part4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int e = 0; e < FPT; ++e)
            part4[e & 3] = fma((double)s_q[my_part * FPT + e], (double)kb[e], part4[e & 3]);
        dot = (part4[0] + part4[1]) + (part4[2] + part4[3]);
    }
    dot += shfl_xor_d(dot, 1);
    if (scored && my_part == 0) {
        const int32_t c = s_cell[my_slot];
        const double delta = (double)i - ((double)c + 0.5) * kS;
        // erf rounds to exactly 1 in fp64 from 6 on (erfc(6) < 2^-54): skip the series there
        const double x = delta / (2.0 * (double)hc.sigma[h]);
        const double g = x >= 6.0 ? 1.0 : erf(x);
        s_key[ri] = score_key(dot / sqrt((double)D) + (double)hc.lambda[h] * (double)s_a[my_slot] * g, ri);
        s_rc[ri] = c;
        s_rslot[ri] = my_slot;
    }
    const int n8 = (n_ret + 7) & ~7;
    if (t >= n_ret && t < n8)
        s_key[t] = 0; // padding ranks last
    if (t < kKmax) { // every rank below min(K, |A|) is written below; slot 0 keeps reads in bounds regardless
        s_sel_slot[t] = 0;
        s_sel_cell[t] = -1;
    }
    __syncthreads();

    // ---- top-K by rank (score desc, id asc) ----
    if (t < n_ret) {
        const int rank = count_greater(s_key, n8, s_key[t]);
        if (rank < K) {
            const int slot = s_rslot[t];
            s_sel_slot[rank] = slot >= 0 && slot < L.S ? slot : 0;
            s_sel_cell[rank] = s_rc[t];
        }
    }
    const int nT = n_ret < K ? n_ret : K;
    __syncthreads();

    // ---- (b) readout: wave w gathers selections w, w + 4 with a running softmax ----
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);
    const int vrow0 = lane / CPR, vch = lane % CPR;
    float m_w = -INFINITY, z_w = 0.0f;
    float acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e)
        acc[e] = 0.0f;
    for (int j = wave; j < nT; j += kWaves) {
        const int slot = s_sel_slot[j];
        const T *kc = sk + (int64_t)slot * kS * D;
        const T *vc = sv + (int64_t)slot * kS * D;
        u32x4 vraw[VR];
#pragma unroll
        for (int x = 0; x < VR; ++x)
            vraw[x] = *reinterpret_cast<const u32x4 *>(vc + (int64_t)(vrow0 + RG * x) * D + vch * EPC);
        float kr[HALF];
        load_row_f32<T, HALF>(kc + (int64_t)(lane >> 1) * D + (lane & 1) * HALF, kr);
        float lp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int e = 0; e < HALF; ++e)
            lp[e & 3] = fmaf(s_q[(lane & 1) * HALF + e], kr[e], lp[e & 3]);
        float l = (lp[0] + lp[1]) + (lp[2] + lp[3]);
        l = (l + dpp_f<0xB1>(l)) * inv_sqrt_d; // logit of token lane / 2, on both lanes of the pair
        const float m_new = fmaxf(m_w, wave_max_f(l));
        const float scale = expf(m_w - m_new); // 0 on the wave's first cell
        const float p = expf(l - m_new);
        z_w = z_w * scale + wave_sum_f((lane & 1) ? 0.0f : p);
#pragma unroll
        for (int e = 0; e < EPC; ++e)
            acc[e] *= scale;
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
        m_w = m_new;
    }
#pragma unroll
    for (int e = 0; e < EPC; ++e)
        s_upart[wave][vrow0 * D + vch * EPC + e] = acc[e];
    if (lane == 0) {
        s_m[wave] = m_w;
        s_z[wave] = z_w;
    }
    __syncthreads();

    // ---- combine the waves and row groups, normalise, RMSNorm over d (Eq. 17), write ----
    float u = 0.0f;
    if (t < D && nT > 0) {
        float M = s_m[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            M = fmaxf(M, s_m[w]);
        float Z = 0.0f, U = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = s_m[w] == -INFINITY ? 0.0f : expf(s_m[w] - M);
            float uw = 0.0f;
#pragma unroll
            for (int g = 0; g < RG; ++g)
                uw += s_upart[w][g * D + t];
            Z = fmaf(s_z[w], f, Z);
            U = fmaf(uw, f, U);
        }
        u = U / Z;
    }
    const float sq = wave_sum_f(t < D ? u * u : 0.0f);
    if (lane == 0)
        s_red[wave] = sq;
    __syncthreads();
    float ms = 0.0f;
#pragma unroll
    for (int w = 0; w < (D + kWave - 1) / kWave; ++w)
        ms += s_red[w];
    const float rs = 1.0f / sqrtf(ms / (float)D + eps);
    if (t < D) {
        const float gv = gain ? gain[(int64_t)h * D + t] : 1.0f;
        const float y = nT > 0 ? gv * u * rs : 0.0f;
        if constexpr (sizeof(T) == 2)
            o_row[t] = (T)f32_to_bf16_bits(y);
        else
            o_row[t] = y;
    }
    if (sel && t < K)
        sel[bh * K + t] = t < nT ? s_sel_cell[t] : -1;
    if (t == 0)
        R.meta->pos = i + 1;
}

template <typename T, int D>
hipError_t build_t(const Geometry &g, const StateLayout &L, const StateHeader &hdr, void *state, const void *k,
                   const void *v, const float *kbar, const float *a, const int32_t *death, hipStream_t st)
{
    hipLaunchKernelGGL((state_build_kernel<T, D>), dim3((unsigned)g.bh), dim3(kThreads), 0, st,
                       static_cast<char *>(state), L, hdr, static_cast<const T *>(k), static_cast<const T *>(v),
                       kbar, a, death, g.N, g.M, g.W);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t step_t(int32_t bh, int32_t H, int32_t K, int32_t P, int32_t W, float eps, const StateLayout &L,
                  const StateHeader &expect, const HeadConsts &hc, void *state, const void *q, const void *k_new,
                  const void *v_new, const float *gain, void *out, int32_t *sel, hipStream_t st)
{
    hipLaunchKernelGGL((decode_step_kernel<T, D>), dim3((unsigned)bh), dim3(kThreads), 0, st,
                       static_cast<char *>(state), L, expect, hc, static_cast<const T *>(q),
                       static_cast<const T *>(k_new), static_cast<const T *>(v_new), gain, static_cast<T *>(out),
                       sel, H, K, P, W, eps);
    return hipGetLastError();
}

} // namespace

hipError_t launch_state_build(const Geometry &g, const StateLayout &L, const StateHeader &hdr, void *state,
                              const void *k, const void *v, const float *kbar, const float *a,
                              const int32_t *death, hipStream_t st)
{
    if (g.bf16)
        return g.d == 64 ? build_t<uint16_t, 64>(g, L, hdr, state, k, v, kbar, a, death, st)
                         : build_t<uint16_t, 128>(g, L, hdr, state, k, v, kbar, a, death, st);
    return g.d == 64 ? build_t<float, 64>(g, L, hdr, state, k, v, kbar, a, death, st)
                     : build_t<float, 128>(g, L, hdr, state, k, v, kbar, a, death, st);
}

hipError_t launch_decode_step(int32_t bh, int32_t H, int32_t d, int32_t bf16, int32_t K, int32_t P, int32_t W,
                              float eps, const StateLayout &L, const StateHeader &expect, const HeadConsts &hc,
                              void *state, const void *q, const void *k_new, const void *v_new,
                              const float *gain, void *out, int32_t *sel, hipStream_t st)
{
    if (bf16)
        return d == 64 ? step_t<uint16_t, 64>(bh, H, K, P, W, eps, L, expect, hc, state, q, k_new, v_new, gain, out,
                                              sel, st)
                       : step_t<uint16_t, 128>(bh, H, K, P, W, eps, L, expect, hc, state, q, k_new, v_new, gain,
                                               out, sel, st);
    return d == 64 ? step_t<float, 64>(bh, H, K, P, W, eps, L, expect, hc, state, q, k_new, v_new, gain, out, sel,
                                       st)
                   : step_t<float, 128>(bh, H, K, P, W, eps, L, expect, hc, state, q, k_new, v_new, gain, out, sel,
                                        st);
}

} // namespace fsl
