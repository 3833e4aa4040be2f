// Chunked prefill into a decode state, one query block at a time (FreeSolo,
// App. C "Bounded cache": the bounded cache is prefilled in fixed-size chunks
// with the retention update at every block boundary; Sec. 3.3 "Inference": the
// prefill and decode are one causal operator), for bf16 tensors.
//
// The queries of one 128-query block all read the same retained set A_beta
// (Eq. 6 makes the block's own cells unavailable to it), so a chunk need not
// be walked token by token: one workgroup per (sequence, head) takes the
// chunk's blocks in order and, for each,
//   (1) at a block start, merges the B/s cells that just became eligible into
//       TopP (Eq. 15) and forms A = TopP u Recent_W, as the decode step does;
//   (2) routes and reads out all of the block's queries in the chunk at once,
//       with the arithmetic of the fused prefill kernel: the retained mean keys
//       (fp32 in the state, split into the same bf16 hi/mid/lo parts the
//       summary pass writes) scored on the matrix cores, each query's top-K
//       in registers, the block's union of selected cells gathered from the
//       state's slots and applied on the matrix cores with the running
//       softmax, RMSNorm.  Tiles, unions and products come in the same order
//       as there, so every output row and selection is bitwise the whole
//       prompt's prefill's;
//   (3) appends the block's tokens to the state: a cell starting in the block
//       takes the lowest free slot, its rows are copied in, and a completed
//       cell gets its mean key and largest key norm (Eq. 5) in fp64, rounded
//       once, with the decode step's order of operations.
// Cells never straddle blocks, so every row a completed cell needs is either
// in the chunk or was written by an earlier launch.  A chunk may start and end
// anywhere; only the queries inside it are computed and written.
#include "decode_lr.h"
#include "readout_math.h"

#include <cfloat>
#include <type_traits>

namespace fsl {
namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));

template <int D>
struct alignas(16) ChunkSmem {
    static constexpr int kStride = D + 8;   // bf16 elements per row (16-byte pad against bank conflicts)
    static constexpr int kStrideVR = D + 16; // bf16 elements per V row
    union {
        struct { // readout: one cell
            uint16_t k[32][kStride];
            uint16_t v[32][kStrideVR];
        };
        uint16_t tile[128][kStride]; // epilogue: the block's output tile
        uint16_t crow[kCpb][32][D]; // appending: the rows of the block's completed cells
    };
    // per position in A (padded to whole tiles): lambda a_c, the cell centre relative to
    // the block start, the low half of the ranking key (-1 past |A|), the slot
    float prior[kMaxSlots], pc[kMaxSlots];
    int32_t id[kMaxSlots], pslot[kMaxSlots];
};

// The mean key's bf16 hi, mid and lo parts of every slot, kept in LDS for the whole
// launch: slot x, part p at (3 x + p) * (D + 8).
template <int D>
constexpr int kPartStride = D + 8;

// The summary pass's split of two fp32 mean-key features: hi, mid, lo (24 mantissa bits in all).
__device__ __forceinline__ void split3(float m0, float m1, uint32_t &hi, uint32_t &mid, uint32_t &lo)
{
    hi = cvt_pk_bf16(m0, m1);
    const float r0 = m0 - bf16_bits_to_f32(hi & 0xffffu), r1 = m1 - bf16_bits_to_f32(hi >> 16);
    mid = cvt_pk_bf16(r0, r1);
    const float s0 = r0 - bf16_bits_to_f32(mid & 0xffffu), s1 = r1 - bf16_bits_to_f32(mid >> 16);
    lo = cvt_pk_bf16(s0, s1);
}

template <int D, int KT>
__global__ __launch_bounds__(kThreads) void chunk_block_kernel(char *__restrict__ state, StateLayout L,
                                                               StateHeader expect, HeadConsts hc,
                                                               const uint16_t *__restrict__ q,
                                                               const uint16_t *__restrict__ kin,
                                                               const uint16_t *__restrict__ vin,
                                                               const float *__restrict__ gain,
                                                               uint16_t *__restrict__ out, int32_t *__restrict__ sel,
                                                               int H, int P, int W, float eps, int64_t n)
{
    __shared__ ChunkSmem<D> sm;
    __shared__ int32_t s_cell[kMaxSlots], s_flags[kMaxSlots], s_ridx[kMaxSlots];
    __shared__ __attribute__((aligned(16))) int32_t s_kc[kMaxSlots];
    __shared__ float s_a[kMaxSlots];
    __shared__ __attribute__((aligned(16))) uint64_t s_key[kMaxSlots];
    __shared__ int32_t s_Acell[kMaxSlots], s_Aslot[kMaxSlots]; // A by position (ascending cell id)
    __shared__ int32_t sel_s[128][KT];                          // selections as positions in A
    __shared__ int32_t ulist[128 * KT];
    __shared__ uint32_t bitmap[kMaxSlots / 32];
    __shared__ int32_t n_u, s_cur, s_newslot[kCpb];
    __shared__ double s_rowmax[kCpb][kWaves];
    __shared__ __attribute__((aligned(16))) uint16_t s_kbs[kMaxSlots * 3 * kPartStride<D>]; // the slots' parts
    // the tile bound: every slot's |kbar| (and by scoring row), and per 32-row tile the
    // largest lambda a_c and |kbar_c| (infinite where a value is not finite)
    __shared__ float s_kn[kMaxSlots], s_knr[kMaxSlots], s_tpr[kMaxSlots / 32], s_tkn[kMaxSlots / 32];

    constexpr int KC = D / 16;   // k-steps of the bf16 matrix products
    constexpr int PS = kPartStride<D>;
    constexpr int CPR = D / 8;   // 16-byte chunks per row
    const int64_t bh = blockIdx.x;
    const int h = (int)(bh % H);
    const int t = threadIdx.x;
    const int wave = t / kWave;
    const int lane = t & (kWave - 1);
    const int half = lane >> 5;
    const int col = lane & 31;
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    const float inv2s = hc.inv_two_sigma[h];
    const float lam = hc.lambda[h];

    const Record R = record_at(state, L, bh); // in bounds: the host checked the buffer size
    uint16_t *sk = reinterpret_cast<uint16_t *>(R.k);
    uint16_t *sv = reinterpret_cast<uint16_t *>(R.v);
    const StateHeader hv = *reinterpret_cast<const StateHeader *>(state);
    const StateMeta mv = *R.meta;
    const int bad = (int)(hv.magic != kStateMagic) | (int)(hv.version != kStateVersion) |
                    (int)(hv.batch != expect.batch) | (int)(hv.H != expect.H) | (int)(hv.d != D) |
                    (int)(hv.dtype != expect.dtype) | (int)(hv.P != P) | (int)(hv.W != W) |
                    (int)(hv.n_slots != L.S) | (int)(hv.rec_bytes != L.rec_bytes);
    if (bad) { // not a state of this shape: flag the outputs, leave the state alone
        for (int64_t e = t; e < n * D; e += kThreads)
            out[bh * n * D + e] = (uint16_t)0x7fc0u; // bf16 quiet NaN
        if (sel)
            for (int64_t e = t; e < n * KT; e += kThreads)
                sel[bh * n * KT + e] = -1;
        return; // the header is the same for every thread: the whole workgroup leaves
    }
    for (int x = t; x < kMaxSlots; x += kThreads) {
        const bool in = x < L.S;
        s_cell[x] = in ? R.cell[x] : -1;
        s_flags[x] = in ? R.flags[x] : 0;
        s_ridx[x] = in ? R.ridx[x] : -1;
        s_a[x] = in ? R.a[x] : 0.0f;
    }
    // every slot's mean key, split once (slots without a summary yet hold stale values,
    // overwritten when their cell completes and unread before)
    for (int e = t; e < L.S * (D / 2); e += kThreads) {
        const int x = e / (D / 2), f = 2 * (e % (D / 2));
        const u32x2 m = *reinterpret_cast<const u32x2 *>(R.kbar + (int64_t)x * D + f);
        uint32_t hi, mid, lo;
        split3(__uint_as_float(m[0]), __uint_as_float(m[1]), hi, mid, lo);
        *reinterpret_cast<uint32_t *>(s_kbs + (3 * x + 0) * PS + f) = hi;
        *reinterpret_cast<uint32_t *>(s_kbs + (3 * x + 1) * PS + f) = mid;
        *reinterpret_cast<uint32_t *>(s_kbs + (3 * x + 2) * PS + f) = lo;
    }
    if (t < L.S) { // the slot's |kbar| (slots without a summary yet: stale, unread until it completes)
        float ss = 0.0f;
        for (int f = 0; f < D; f += 4) {
            const u32x4 m4 = *reinterpret_cast<const u32x4 *>(R.kbar + (int64_t)t * D + f);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ss = fmaf(__uint_as_float(m4[e]), __uint_as_float(m4[e]), ss);
        }
        s_kn[t] = sqrtf(ss);
    }
    const int64_t i0 = mv.pos;
    int n_ret = mv.n_ret < 0 ? 0 : (mv.n_ret > L.S ? L.S : mv.n_ret);
    int cur = mv.cur_slot;
    __syncthreads();

    for (int64_t seg = i0; seg < i0 + n;) {
        const int64_t beta = seg / kB;
        const int64_t q0 = beta * kB;
        const int64_t seg_end = q0 + kB < i0 + n ? q0 + kB : i0 + n;

        // ---- (1) block start: Eq. 15 merge, then A = TopP u Recent_W (the decode step's) ----
        if (seg % kB == 0 && seg > 0) {
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
            const bool top = cand && count_greater(s_key, S8, my) < P;
            const bool keep = c >= 0 && (top || (c >= rec_lo && c < d_hi));
            if (t < kMaxSlots) {
                s_flags[t] = top ? kFlagTop : 0;
                s_cell[t] = keep ? c : -1;
                s_kc[t] = keep ? c : INT_MAX;
            }
            __syncthreads();
            int pos = -1;
            if (keep) {
                pos = 0;
                for (int u = 0; u < S8; u += 4) {
                    const u32x4 w4 = *reinterpret_cast<const u32x4 *>(&s_kc[u]);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        pos += (int32_t)w4[e] < c ? 1 : 0;
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

        // ---- (2) the block's queries in the chunk: routing and readout ----
        if (t < kMaxSlots) {
            const int ri = s_ridx[t];
            if (t < L.S && ri >= 0 && ri < n_ret) {
                s_Acell[ri] = s_cell[t];
                s_Aslot[ri] = t;
            }
        }
        __syncthreads();
        const int nA = n_ret;
        const int64_t qi = q0 + wave * 32 + col; // this lane's query position
        const bool q_ok = qi >= seg && qi < seg_end;
        const float qrel = (float)(qi - q0); // positions relative to the block start: exact
        bf16x8 qf[KC]; // requested here: the loads are in flight while A is ordered below
        {
            const uint16_t *qrow = q + (bh * n + ((q_ok ? qi : seg) - i0)) * D;
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
                qf[kc] = as_bf16x8(*reinterpret_cast<const u32x4 *>(qrow + kc * 16 + half * 8));
        }
        // Scoring takes A in priority order (a_c desc, id asc: the order of the prefill's
        // retained lists), so that the first tile holds the largest priors and the tile
        // bound below can pass over the rest.  A row keeps its position in A (ascending
        // id) as the low half of its ranking key, so selections, the union and the readout
        // are exactly those of scoring in position order (a score does not depend on the
        // tile its row sits in).
        if (t < kMaxSlots)
            s_key[t] = t < nA ? norm_key(s_a[s_Aslot[t]], s_Acell[t]) : 0ull;
        __syncthreads();
        if (t < kMaxSlots) { // position t of A, or a padding row of the last tile
            const bool in = t < nA;
            const int slot = in ? s_Aslot[t] : 0;
            const int row = in ? count_greater(s_key, (nA + 7) & ~7, s_key[t]) : t; // its priority rank
            sm.prior[row] = in ? lam * s_a[slot] : 0.0f;
            // (padding rows sit far before the block: they never call for erf)
            sm.pc[row] = in ? (float)((int64_t)s_Acell[t] * kS + kS / 2 - q0) : -1.0e9f;
            sm.id[row] = in ? 0x7fffffff - t : -1;
            sm.pslot[row] = slot;
            s_knr[row] = in ? s_kn[slot] : 0.0f;
        }
        __syncthreads();
        if (t < kMaxSlots) { // per 32-row tile: the largest lambda a_c and |kbar_c|
            float pr = sm.prior[t], kn = s_knr[t];
            pr = pr <= FLT_MAX ? pr : INFINITY; // NaN or infinite: the tile is never passed over
            kn = kn <= FLT_MAX ? kn : INFINITY;
#pragma unroll
            for (int o = 1; o < 32; o <<= 1) {
                pr = fmaxf(pr, shfl_xor_f(pr, o));
                kn = fmaxf(kn, shfl_xor_f(kn, o));
            }
            if ((t & 31) == 0) {
                s_tpr[t >> 5] = pr;
                s_tkn[t >> 5] = kn;
            }
        }
        __syncthreads();
        uint64_t kl[KT]; // this lane's best keys so far
#pragma unroll
        for (int j = 0; j < KT; ++j)
            kl[j] = 0;
        // Tile bound, per wave: every score in a tile is at most
        //   max_c (lambda a_c) + max_i |q_i| max_c |kbar_c| / sqrt(d)
        // (lambda a_c >= 0 and 0 < g <= 1 for every available cell, Cauchy-Schwarz on the
        // content term), widened for rounding.  Once it falls below the smallest K-th best
        // key of the wave's queries so far, no cell of the tile can enter any of their
        // top-K lists and the wave passes over the tile: the selections are those of
        // scoring every tile.  The first tile is always scored.
        float qn_w;
        {
            float ss = 0.0f;
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const u32x4 w4 = __builtin_bit_cast(u32x4, qf[kc]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // the element goes through a named copy: hipcc miscompiles a bit cast
                    // of a vector element taken in place (it reads element 0)
                    const uint32_t we = w4[e];
                    const bf16x2 x2 = __builtin_bit_cast(bf16x2, we);
                    ss = __builtin_amdgcn_fdot2_f32_bf16(x2, x2, ss, false);
                }
            }
            ss += shfl_xor_f(ss, 32); // the partner lane holds the other half of the features
            // + 2^-100: covers subnormal elements, should the dot product flush them
            const float qn = q_ok ? sqrtf(ss) * (1.0f + 0x1p-10f) + 0x1p-100f : 0.0f;
            const bool badq = __ballot(!(qn <= FLT_MAX)) != 0ull;
            qn_w = badq ? INFINITY : wave_max_f(qn);
        }
        uint32_t tau_w = 0; // the wave's smallest K-th best key (high word) so far
        for (int t0 = 0; t0 < nA; t0 += 32) {
            if (t0 > 0) {
                const float ub = (s_tpr[t0 >> 5] + qn_w * s_tkn[t0 >> 5] * inv_sqrt_d * (1.0f + 0x1p-10f)) *
                                 (1.0f + 0x1p-10f);
                // ub >= 0: its ranking key's high word is its bits with the sign bit set
                if (ub <= FLT_MAX && (__float_as_uint(ub) | 0x80000000u) < tau_w)
                    continue; // wave-uniform
            }
            const uint16_t *kbrow = s_kbs + 3 * sm.pslot[t0 + col] * PS; // the tile row this lane's operand reads
            f32x16 acc;
            f32x16 acc3[3];
#pragma unroll
            for (int sp = 0; sp < 3; ++sp)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc3[sp][r] = 0.0f;
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
#pragma unroll
                for (int sp = 2; sp >= 0; --sp) {
                    const u32x4 w4 = *reinterpret_cast<const u32x4 *>(kbrow + sp * PS + kc * 16 + half * 8);
                    acc3[sp] = mfma_bf16(as_bf16x8(w4), qf[kc], acc3[sp]);
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[r] = (acc3[2][r] + acc3[1][r]) + acc3[0][r];
            float prv[16], pcv[16];
            int idv[16]; // low key halves; -1 on padding rows
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int r0 = t0 + 8 * g + 4 * half;
                const u32x4 vp = *reinterpret_cast<const u32x4 *>(&sm.prior[r0]);
                const u32x4 vc = *reinterpret_cast<const u32x4 *>(&sm.pc[r0]);
                const u32x4 vi = *reinterpret_cast<const u32x4 *>(&sm.id[r0]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    prv[4 * g + e] = __uint_as_float(vp[e]);
                    pcv[4 * g + e] = __uint_as_float(vc[e]);
                    idv[4 * g + e] = (int)vi[e];
                }
            }
            // erf only below 4 (from there on it rounds to 1 in fp32, and fmaf(prior,
            // 1, content) == prior + content)
            float pcmax = pcv[0];
#pragma unroll
            for (int r = 1; r < 16; ++r)
                pcmax = fmaxf(pcmax, pcv[r]);
            const bool need_erf = __ballot(q_ok && (qrel - pcmax) * inv2s < 4.0f) != 0ull;
            uint64_t key[16];
            if (need_erf) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float g = 1.0f;
                    const float x = (qrel - pcv[r]) * inv2s; // (i - p_c) / (2 sigma_h), i - p_c exact
                    if (x < 4.0f)
                        g = erff(x);
                    const float score = fmaf(prv[r], g, acc[r] * inv_sqrt_d);
                    key[r] = (q_ok && idv[r] >= 0) ? rank_key(score, (uint32_t)idv[r]) : 0;
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float score = fmaf(prv[r], 1.0f, acc[r] * inv_sqrt_d);
                    key[r] = (q_ok && idv[r] >= 0) ? rank_key(score, (uint32_t)idv[r]) : 0;
                }
            }
            take_tile_keys<KT>(kl, key, t0 == 0);
            tau_w = wave_min_u32(q_ok ? (uint32_t)(kl[KT - 1] >> 32) : 0xffffffffu);
        }
        { // merge with the partner lane (same query, other 16 rows of every tile)
            uint64_t pk[KT];
#pragma unroll
            for (int j = 0; j < KT; ++j)
                pk[j] = ((uint64_t)(uint32_t)shfl_xor_i((int)(kl[j] >> 32), 32) << 32) |
                        (uint32_t)shfl_xor_i((int)(uint32_t)kl[j], 32);
#pragma unroll
            for (int j = 0; j < KT; ++j)
                insert_key<KT>(kl, pk[j]);
        }

        // selections (positions in A) to LDS and, as cell ids, to global; their union in A's order
        int my_sel[KT];
#pragma unroll
        for (int j = 0; j < KT; ++j)
            my_sel[j] = (q_ok && kl[j]) ? 0x7fffffff - (int32_t)(uint32_t)kl[j] : -1;
        if (t < kMaxSlots / 32)
            bitmap[t] = 0u;
        if (half == 0) {
#pragma unroll
            for (int j = 0; j < KT; ++j)
                sel_s[wave * 32 + col][j] = my_sel[j];
            if (sel && q_ok) {
                int32_t *dst = sel + (bh * n + (qi - i0)) * KT;
#pragma unroll
                for (int j = 0; j < KT; ++j)
                    dst[j] = my_sel[j] >= 0 ? s_Acell[my_sel[j]] : -1;
            }
        }
        __syncthreads();
        for (int x = t; x < 128 * KT; x += kThreads) {
            const int32_t c = sel_s[x / KT][x % KT];
            if (c >= 0)
                atomicOr(&bitmap[c >> 5], 1u << (c & 31));
        }
        __syncthreads();
        if (t == 0) {
            int tot = 0;
            for (int w = 0; w < kMaxSlots / 32; ++w) {
                uint32_t b = bitmap[w];
                while (b) {
                    ulist[tot++] = w * 32 + __ffs(b) - 1;
                    b &= b - 1u;
                }
            }
            n_u = tot;
        }
        __syncthreads();
        const int nU = n_u;

        // readout (Eq. 9): one gathered cell at a time, next one in flight
        constexpr int KCH = (32 * CPR) / kThreads; // K chunks per thread: 1 or 2
        u32x4 pk[KCH], pv[KCH];
        auto fetch = [&](int pos) {
            const int64_t base = (int64_t)s_Aslot[pos] * kS * D;
#pragma unroll
            for (int u = 0; u < KCH; ++u) {
                const int ch = t + u * kThreads;
                const int64_t off = base + (ch / CPR) * D + (ch % CPR) * 8;
                pk[u] = *reinterpret_cast<const u32x4 *>(sk + off);
                pv[u] = *reinterpret_cast<const u32x4 *>(sv + off);
            }
        };
        if (nU > 0)
            fetch(ulist[0]);
        constexpr int DT = D / 32; // feature tiles of the output
        f32x16 o_acc[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                o_acc[dt][r] = 0.0f;
        float m_run = -INFINITY, l_run = 0.0f; // m_run in the exp2 domain
        for (int x = 0; x < nU; ++x) {
            const int pos = ulist[x];
            __syncthreads();
#pragma unroll
            for (int u = 0; u < KCH; ++u) {
                const int ch = t + u * kThreads;
                *reinterpret_cast<u32x4 *>(&sm.k[ch / CPR][(ch % CPR) * 8]) = pk[u];
                *reinterpret_cast<u32x4 *>(&sm.v[ch / CPR][(ch % CPR) * 8]) = pv[u];
            }
            __syncthreads();
            if (x + 1 < nU)
                fetch(ulist[x + 1]);
            bool mine = false;
#pragma unroll
            for (int j = 0; j < KT; ++j)
                mine |= my_sel[j] == pos;
            if (__ballot(mine) == 0ull)
                continue; // no query of this wave reads the cell
            f32x16 acc;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[r] = 0.0f;
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const u32x4 w4 = *reinterpret_cast<const u32x4 *>(&sm.k[col][kc * 16 + half * 8]);
                acc = mfma_bf16(as_bf16x8(w4), qf[kc], acc);
            }
            float p[16];
            const float alpha = softmax_cell(acc, mine, scale_log2, m_run, l_run, p);
            if (__ballot(alpha != 1.0f)) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        o_acc[dt][r] *= alpha;
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 bh, bl;
                split_bf16x8(&p[8 * kk], bh, bl);
                bf16x8 av[DT];
                const int r0 = 16 * kk + 4 * half + ((lane & 15) >> 2);
                const int c0 = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4i16 *)&sm.v[r0][dt * 32 + c0]);
                    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4i16 *)&sm.v[r0 + 8][dt * 32 + c0]);
                    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                    av[dt] = as_bf16x8(u32x4{l2[0], l2[1], h2[0], h2[1]});
                }
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    o_acc[dt] = mfma_bf16(av[dt], bl, o_acc[dt]);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    o_acc[dt] = mfma_bf16(av[dt], bh, o_acc[dt]);
            }
        }

        // the block's key and value rows for the state, requested now so that they arrive
        // while the output goes out; stored into their slots below
        constexpr int kIt = (kB * CPR) / kThreads;
        u32x4 rk[kIt], rv[kIt];
#pragma unroll
        for (int u = 0; u < kIt; ++u) {
            const int e = t + u * kThreads;
            const int64_t tok = seg + e / CPR < seg_end ? seg + e / CPR : seg_end - 1;
            const int64_t src = (bh * n + (tok - i0)) * D + (e % CPR) * 8;
            rk[u] = *reinterpret_cast<const u32x4 *>(kin + src);
            rv[u] = *reinterpret_cast<const u32x4 *>(vin + src);
        }
        // normalise, RMSNorm over d (Eq. 17), the chunk's rows out through LDS
        const float c = rms_factor<DT>(o_acc, l_run, eps);
        __syncthreads(); // the last cell's LDS reads are done: the tile area takes the output
        {
            const float *gh = gain ? gain + (int64_t)h * D : nullptr;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const int d0 = dt * 32 + 8 * rg + 4 * half;
                    float y[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        y[e] = o_acc[dt][4 * rg + e] * c;
                        if (gh)
                            y[e] = l_run > 0.0f ? y[e] * gh[d0 + e] : 0.0f;
                    }
                    *reinterpret_cast<u32x2 *>(&sm.tile[wave * 32 + col][d0]) =
                        u32x2{cvt_pk_bf16(y[0], y[1]), cvt_pk_bf16(y[2], y[3])};
                }
        }
        __syncthreads();
        {
            const int r_lo = (int)(seg - q0), r_hi = (int)(seg_end - q0);
            for (int e = t; e < (r_hi - r_lo) * CPR; e += kThreads) {
                const int r = r_lo + e / CPR, c8 = (e % CPR) * 8;
                *reinterpret_cast<u32x4 *>(out + (bh * n + (q0 + r - i0)) * D + c8) =
                    *reinterpret_cast<const u32x4 *>(&sm.tile[r][c8]);
            }
        }

        // ---- (3) the block's tokens in the chunk enter the state ----
        const int cur_before = cur;
        const int64_t c_first = (seg + kS - 1) / kS; // cells that start inside [seg, seg_end)
        const int n_new = (int)((seg_end - 1) / kS - c_first + 1);
        if (wave == 0) {
            // the k-th cell that starts here takes the k-th lowest free slot: the slot the
            // decode step gives it (nothing frees a slot between two block starts)
            const uint64_t f0 = __ballot(lane < L.S && s_cell[lane] < 0);
            const uint64_t f1 = __ballot(lane + kWave < L.S && s_cell[lane + kWave] < 0);
            int slot = -1;
            if (lane < n_new) {
                uint64_t m0 = f0, m1 = f1;
                for (int j = 0; j < lane; ++j) { // drop the lane lowest free slots
                    if (m0)
                        m0 &= m0 - 1u;
                    else
                        m1 &= m1 - 1u;
                }
                slot = m0 ? __ffsll((unsigned long long)m0) - 1
                          : (m1 ? kWave + __ffsll((unsigned long long)m1) - 1 : -1);
                s_newslot[lane] = slot;
                if (slot >= 0) {
                    const int32_t cc = (int32_t)(c_first + lane);
                    s_cell[slot] = cc;
                    s_flags[slot] = 0;
                    s_ridx[slot] = -1;
                    R.cell[slot] = cc;
                    R.flags[slot] = 0;
                    R.ridx[slot] = -1;
                }
            }
            const uint64_t got = __ballot(slot >= 0);
            if (lane == 0)
                s_cur = got ? __builtin_amdgcn_readlane(slot, 63 - __clzll((long long)got)) : cur_before;
        }
        __syncthreads();
        cur = s_cur;
        auto slot_of = [&](int64_t cell) { // -1 when the state had no free slot (a corrupted state)
            return cell >= c_first ? s_newslot[(int)(cell - c_first)] : cur_before;
        };
        { // the rows (requested before the output tile, above): the stores
#pragma unroll
            for (int u = 0; u < kIt; ++u) {
                const int e = t + u * kThreads;
                const int64_t tok = seg + e / CPR;
                const int slot = tok < seg_end ? slot_of(tok / kS) : -1;
                if (slot >= 0 && slot < L.S) {
                    const int64_t dst = ((int64_t)slot * kS + tok % kS) * D + (e % CPR) * 8;
                    *reinterpret_cast<u32x4 *>(sk + dst) = rk[u];
                    *reinterpret_cast<u32x4 *>(sv + dst) = rv[u];
                }
            }
        }
        // cells completed in this block: Eq. 5 with the decode step's operations and order,
        // every cell's rows requested first
        {
            constexpr int FP = D / 8;
            const int row = t >> 3, part = t & 7;
            int64_t cdone[kCpb];
            int n_done = 0;
            for (int64_t cc = seg / kS; cc * kS + kS - 1 < seg_end; ++cc)
                if ((cc + 1) * kS - 1 >= seg)
                    cdone[n_done++] = cc;
            float x[kCpb][FP];
#pragma unroll
            for (int j = 0; j < kCpb; ++j) {
                if (j < n_done) {
                    const int64_t tok = cdone[j] * kS + row;
                    const int slot = slot_of(cdone[j]);
                    const int ss = slot >= 0 && slot < L.S ? slot : 0; // in bounds; unused for a corrupted state
                    if (tok >= i0) // a row of this chunk
                        load_row_f32<uint16_t, FP>(kin + (bh * n + (tok - i0)) * D + part * FP, x[j]);
                    else // a row an earlier launch wrote
                        load_row_f32<uint16_t, FP>(sk + ((int64_t)ss * kS + row) * D + part * FP, x[j]);
                }
            }
            // the largest row norm: the decode step's fp64 sums over a row's parts and its order
#pragma unroll
            for (int j = 0; j < kCpb; ++j) {
                if (j < n_done) {
                    double sq = 0.0;
#pragma unroll
                    for (int e = 0; e < FP; ++e) {
                        const double v = (double)x[j][e];
                        sq += v * v;
                    }
                    sq += shfl_xor_d(sq, 1);
                    sq += shfl_xor_d(sq, 2);
                    sq += shfl_xor_d(sq, 4);
                    double mx = sq;
#pragma unroll
                    for (int m = 8; m < kWave; m <<= 1)
                        mx = fmax(mx, shfl_xor_d(mx, m));
                    if (lane == 0)
                        s_rowmax[j][wave] = mx;
                    // the row (exact bf16 values) for the column sums below
#pragma unroll
                    for (int e = 0; e < FP; ++e)
                        sm.crow[j][row][part * FP + e] = (uint16_t)(__float_as_uint(x[j][e]) >> 16);
                }
            }
            __syncthreads();
            // the mean key, one column per task, summed in the decode step's order: the
            // rows of each wave (8 w .. 8 w + 7) pairwise, then the four waves pairwise
            for (int task = t; task < n_done * D; task += kThreads) {
                const int j = task / D, f = task % D;
                const int slot = slot_of(cdone[j]);
                if (slot < 0 || slot >= L.S)
                    continue;
                double ws[kWaves];
#pragma unroll
                for (int w = 0; w < kWaves; ++w) {
                    double r[8];
#pragma unroll
                    for (int y = 0; y < 8; ++y)
                        r[y] = (double)bf16_bits_to_f32(sm.crow[j][8 * w + y][f]);
                    ws[w] = ((r[0] + r[1]) + (r[2] + r[3])) + ((r[4] + r[5]) + (r[6] + r[7]));
                }
                const float m = (float)(((ws[0] + ws[1]) + (ws[2] + ws[3])) * (1.0 / 32.0));
                R.kbar[(int64_t)slot * D + f] = m;
                uint32_t hi, mid, lo;
                split3(m, m, hi, mid, lo);
                s_kbs[(3 * slot + 0) * PS + f] = (uint16_t)(hi & 0xffffu);
                s_kbs[(3 * slot + 1) * PS + f] = (uint16_t)(mid & 0xffffu);
                s_kbs[(3 * slot + 2) * PS + f] = (uint16_t)(lo & 0xffffu);
            }
            if (t < n_done) {
                const int slot = slot_of(cdone[t]);
                if (slot >= 0 && slot < L.S) {
                    const float av = (float)sqrt(fmax(fmax(s_rowmax[t][0], s_rowmax[t][1]),
                                                      fmax(s_rowmax[t][2], s_rowmax[t][3])));
                    R.a[slot] = av;
                    s_a[slot] = av;
                }
            }
            __syncthreads();
            // the completed cells' |kbar|, one wave per cell, from its parts (hi + mid + lo =
            // the mean; the tile bound only needs it to about 2^-10)
            static_assert(kCpb <= kWaves, "a wave per completed cell");
            if (wave < n_done) {
                const int slot = slot_of(cdone[wave]);
                if (slot >= 0 && slot < L.S) {
                    float ss = 0.0f;
                    for (int f = lane; f < D; f += kWave) {
                        const float m = (bf16_bits_to_f32(s_kbs[(3 * slot + 0) * PS + f]) +
                                         bf16_bits_to_f32(s_kbs[(3 * slot + 1) * PS + f])) +
                                        bf16_bits_to_f32(s_kbs[(3 * slot + 2) * PS + f]);
                        ss = fmaf(m, m, ss);
                    }
#pragma unroll
                    for (int o = 1; o < kWave; o <<= 1)
                        ss += shfl_xor_f(ss, o);
                    if (lane == 0)
                        s_kn[slot] = sqrtf(ss);
                }
            }
            __syncthreads();
        }
        seg = seg_end;
    }
    if (t == 0) {
        R.meta->pos = i0 + n;
        R.meta->cur_slot = cur;
    }
}

template <int D>
hipError_t launch_d(int32_t bh, int32_t H, int32_t K, int32_t P, int32_t W, float eps, const StateLayout &L,
                    const StateHeader &expect, const HeadConsts &hc, void *state, const void *q, const void *k,
                    const void *v, const float *gain, void *out, int32_t *sel, int64_t n, hipStream_t st)
{
#define FSL_CHUNK_LAUNCH(KT)                                                                                          \
    hipLaunchKernelGGL((chunk_block_kernel<D, KT>), dim3((unsigned)bh), dim3(kThreads), 0, st,                        \
                       static_cast<char *>(state), L, expect, hc, static_cast<const uint16_t *>(q),                   \
                       static_cast<const uint16_t *>(k), static_cast<const uint16_t *>(v), gain,                      \
                       static_cast<uint16_t *>(out), sel, H, P, W, eps, n)
    switch (K) {
    case 1: FSL_CHUNK_LAUNCH(1); break;
    case 2: FSL_CHUNK_LAUNCH(2); break;
    case 3: FSL_CHUNK_LAUNCH(3); break;
    case 4: FSL_CHUNK_LAUNCH(4); break;
    case 5: FSL_CHUNK_LAUNCH(5); break;
    case 6: FSL_CHUNK_LAUNCH(6); break;
    case 7: FSL_CHUNK_LAUNCH(7); break;
    default: FSL_CHUNK_LAUNCH(8); break;
    }
#undef FSL_CHUNK_LAUNCH
    return hipGetLastError();
}

} // namespace

hipError_t launch_chunk_blocks(int32_t bh, int32_t H, int32_t d, int32_t K, int32_t P, int32_t W, float eps,
                               const StateLayout &L, const StateHeader &expect, const HeadConsts &hc, void *state,
                               const void *q, const void *k, const void *v, const float *gain, void *out,
                               int32_t *sel, int64_t n, hipStream_t st)
{
    return d == 64 ? launch_d<64>(bh, H, K, P, W, eps, L, expect, hc, state, q, k, v, gain, out, sel, n, st)
                   : launch_d<128>(bh, H, K, P, W, eps, L, expect, hc, state, q, k, v, gain, out, sel, n, st);
}

} // namespace fsl
