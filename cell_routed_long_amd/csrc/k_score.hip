// Block-level cell scoring and per-query top-K (FreeSolo, Sec. 3.3 "Cell scoring",
// Eq. 7, and "Per-query selection"):
//   r_ic = q_i . kbar_c / sqrt(d) + lambda_h a_c erf((i - p_c) / (2 sigma_h)),
//   T_i  = the min(K, |A_i|) best cells of A_i by (score desc, id asc).
//
// One workgroup (4 waves) per (sequence, head, 128-query block): the block's
// queries share the retained set A_beta (FS-L, listed in priority order) or the
// prefix C_beta (FS).  The retained mean keys are staged through LDS 32 cells at
// a time and each wave
// computes S^T = Kbar_tile . Q_wave^T on the matrix cores, so that a lane owns
// one query and 16 cells of the tile and keeps its running top-K in registers.
//
// Precision: selections must agree with an fp64 evaluation, so for bf16
// queries (exact in bf16) each fp32 mean key is split into three bf16 parts
// (hi + mid + lo carries all 24 mantissa bits) and three bf16 MFMA passes
// accumulate in fp32; fp32 queries use the fp32 MFMA directly.
#include "fsl_internal.h"

#include <climits>
#include <type_traits>

namespace fsl {
namespace {

constexpr int kThreads = 256;

template <typename T, int D>
struct ScoreSmem;

template <int D>
struct alignas(16) ScoreSmem<uint16_t, D> {
    static constexpr int kStride = D + 8; // bf16 elements per row (16-byte pad against bank conflicts)
    union {
        uint16_t kb[3][32][kStride];
        uint16_t tile[128][kStride]; // the block's q tile, read once at entry
    };
    float prior[32]; // lambda_h * a_c
    float pc[32];    // cell centre p_c
    int32_t id[32];
};

template <int D>
struct alignas(16) ScoreSmem<float, D> {
    static constexpr int kStride = D + 1;
    float kb[32][kStride];
    float prior[32];
    float pc[32];
    int32_t id[32];
};

template <typename T, int D, int KT, bool kPre>
__global__ __launch_bounds__(kThreads) void score_topk_kernel(
    const T *__restrict__ q, const float *__restrict__ kbar, const uint16_t *__restrict__ kbar_split,
    const float *__restrict__ a, const int32_t *__restrict__ retained, const int32_t *__restrict__ n_ret,
    int32_t *__restrict__ sel, int64_t N, int64_t M, int NB, int cap, int prune, int H, int cells_per_block, int s,
    HeadConsts hc)
{
    static_assert(!kPre || sizeof(T) == 2, "the split operands are for bf16 queries");
    __shared__ ScoreSmem<T, D> sm;
    constexpr bool kBf16 = sizeof(T) == 2;
    constexpr int PER = D / 8; // mean-key floats staged per thread and tile
    const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int beta = (int)(lb % (uint32_t)NB);
    const int64_t head = (int64_t)(lb / (uint32_t)NB);
    const int h = (int)(head % H);
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int half = lane >> 5;
    const int col = lane & 31;
    const int64_t qi = (int64_t)beta * 128 + wave * 32 + col; // this lane's query position
    const bool q_ok = qi < N;
    const float qpos = (float)qi; // exact: N <= 2^22
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);
    const float inv2s = hc.inv_two_sigma[h];
    const float lam = hc.lambda[h];

    int64_t n_avail = (int64_t)beta * cells_per_block;
    if (n_avail > M)
        n_avail = M;
    const int nA = prune ? n_ret[head * NB + beta] : (int)n_avail;
    const int32_t *A = prune ? retained + (head * NB + beta) * (int64_t)cap : nullptr;

    // staging role of this thread: row (cell of the tile) and feature part
    const int srow = threadIdx.x >> 3;
    const int spart = threadIdx.x & 7;
    constexpr int SCH = kPre ? PER / 8 : 1; // 16-byte chunks per part and thread (split input)
    float pre[kPre ? 1 : PER];
    u32x4 pre3[kPre ? 3 * SCH : 1];
    int pre_id;
    float pre_a;
    auto prefetch = [&](int t0) {
        const int x = t0 + srow;
        pre_id = x < nA ? (prune ? A[x] : x) : -1;
        pre_a = 0.0f;
        if (pre_id >= 0) {
            if constexpr (kPre) {
                const uint16_t *src = kbar_split + (head * M + pre_id) * 3 * D + spart * PER;
#pragma unroll
                for (int part = 0; part < 3; ++part)
#pragma unroll
                    for (int u = 0; u < SCH; ++u)
                        pre3[part * SCH + u] = *reinterpret_cast<const u32x4 *>(src + part * D + u * 8);
            } else {
                const float *src = kbar + (head * M + pre_id) * D + spart * PER;
#pragma unroll
                for (int e = 0; e < PER; e += 4) {
                    const u32x4 w = *reinterpret_cast<const u32x4 *>(src + e);
                    pre[e] = __uint_as_float(w[0]);
                    pre[e + 1] = __uint_as_float(w[1]);
                    pre[e + 2] = __uint_as_float(w[2]);
                    pre[e + 3] = __uint_as_float(w[3]);
                }
            }
            if (spart == 0)
                pre_a = a[head * M + pre_id];
        } else {
            if constexpr (kPre) {
#pragma unroll
                for (int u = 0; u < 3 * SCH; ++u)
                    pre3[u] = u32x4{0, 0, 0, 0};
            } else {
#pragma unroll
                for (int e = 0; e < PER; ++e)
                    pre[e] = 0.0f;
            }
        }
    };
    if (nA > 0)
        prefetch(0);

    // query fragments (B operand): column `col`, k values of group `half`
    constexpr int KC = kBf16 ? D / 16 : D / 2;
    using QFrag = typename std::conditional<kBf16, bf16x8, float>::type;
    QFrag qf[KC];
    if constexpr (kBf16) { // through LDS, coalesced; the tile area is reused for the mean keys below
        const int64_t q0 = (int64_t)beta * 128;
        tile_load_bf16<D, kThreads>(&sm.tile[0][0], sm.kStride, q + (head * N + q0) * D,
                                    (int)(N - q0 < 128 ? N - q0 : 128));
        __syncthreads();
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
            qf[kc] = as_bf16x8(*reinterpret_cast<const u32x4 *>(&sm.tile[wave * 32 + col][kc * 16 + half * 8]));
    } else {
        const T *qrow = q + (head * N + (q_ok ? qi : 0)) * D;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
            qf[kc] = q_ok ? qrow[kc * 2 + half] : 0.0f;
    }

    uint64_t kl[KT]; // this lane's best keys so far
#pragma unroll
    for (int j = 0; j < KT; ++j)
        kl[j] = 0;

    for (int t0 = 0; t0 < nA; t0 += 32) {
        __syncthreads();
        // ---- the prefetched 32 mean keys (and prior terms, ids) into LDS ----
        if (spart == 0) {
            sm.id[srow] = pre_id >= 0 ? 0x7fffffff - pre_id : -1;   // low half of the ranking key
            sm.prior[srow] = pre_id >= 0 ? lam * pre_a : 0.0f;
            sm.pc[srow] = pre_id >= 0 ? (float)pre_id * s + 0.5f * s : 0.0f;
        }
        if constexpr (kPre) {
#pragma unroll
            for (int part = 0; part < 3; ++part)
#pragma unroll
                for (int u = 0; u < SCH; ++u)
                    *reinterpret_cast<u32x4 *>(&sm.kb[part][srow][spart * PER + u * 8]) = pre3[part * SCH + u];
        } else if constexpr (kBf16) {
#pragma unroll
            for (int e = 0; e < PER; e += 2) {
                const float v0 = pre[e], v1 = pre[e + 1];
                const uint32_t hi2 = cvt_pk_bf16(v0, v1);
                const float r0 = v0 - bf16_bits_to_f32(hi2 & 0xffffu), r1 = v1 - bf16_bits_to_f32(hi2 >> 16);
                const uint32_t mid2 = cvt_pk_bf16(r0, r1);
                const float s0 = r0 - bf16_bits_to_f32(mid2 & 0xffffu), s1 = r1 - bf16_bits_to_f32(mid2 >> 16);
                const uint32_t lo2 = cvt_pk_bf16(s0, s1);
                const int c0 = spart * PER + e;
                *reinterpret_cast<uint32_t *>(&sm.kb[0][srow][c0]) = hi2;
                *reinterpret_cast<uint32_t *>(&sm.kb[1][srow][c0]) = mid2;
                *reinterpret_cast<uint32_t *>(&sm.kb[2][srow][c0]) = lo2;
            }
        } else {
#pragma unroll
            for (int e = 0; e < PER; ++e)
                sm.kb[srow][spart * PER + e] = pre[e];
        }
        __syncthreads();
        if (t0 + 32 < nA)
            prefetch(t0 + 32); // overlaps the matrix work below

        // ---- S^T[32 cells x 32 queries] on the matrix cores ----
        f32x16 acc;
        if constexpr (kBf16) {
            // three independent accumulators (lo, mid, hi parts) keep the matrix cores busy;
            // the parts are added smallest first
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
                    const u32x4 w = *reinterpret_cast<const u32x4 *>(&sm.kb[sp][col][kc * 16 + half * 8]);
                    acc3[sp] = mfma_bf16(as_bf16x8(w), qf[kc], acc3[sp]);
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[r] = (acc3[2][r] + acc3[1][r]) + acc3[0][r];
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[r] = 0.0f;
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
                acc = mfma_f32(sm.kb[col][kc * 2 + half], qf[kc], acc);
        }

        // ---- Eq. 7 and the running top-K of this lane's query ----
        // FS-L lists the retained cells in priority order (a desc), so the
        // first tile holds the largest prior terms and later cells mostly
        // fall below every query's K-th best: the insertion runs only when
        // some lane of the wave needs it.
        // this lane's 16 rows come in 4 runs of 4 consecutive rows: 12 vector LDS reads
        float prv[16], pcv[16];
        int idv[16]; // low key halves; -1 on padding rows
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int r0 = 8 * g + 4 * half;
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
        // 1, content) == prior + content); a wave takes the long path only if
        // one of its queries is that close to one of its cells
        float pcmax = pcv[0];
#pragma unroll
        for (int r = 1; r < 16; ++r)
            pcmax = fmaxf(pcmax, pcv[r]);
        const bool need_erf = __ballot(q_ok && (qpos - pcmax) * inv2s < 4.0f) != 0ull;
        uint64_t key[16];
        if (need_erf) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float g = 1.0f;
                const float x = (qpos - pcv[r]) * inv2s; // (i - p_c) / (2 sigma_h), i - p_c exact
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
    }

    // ---- merge with the partner lane (same query, other 16 rows) ----
    {
        uint64_t pk[KT]; // the partner's list as it was, before either lane inserts
#pragma unroll
        for (int j = 0; j < KT; ++j)
            pk[j] = ((uint64_t)(uint32_t)shfl_xor_i((int)(kl[j] >> 32), 32) << 32) |
                    (uint32_t)shfl_xor_i((int)(uint32_t)kl[j], 32);
#pragma unroll
        for (int j = 0; j < KT; ++j)
            insert_key<KT>(kl, pk[j]);
    }

    if (q_ok && half == 0) {
        int32_t *dst = sel + (head * N + qi) * KT;
#pragma unroll
        for (int j = 0; j < KT; ++j)
            dst[j] = kl[j] ? 0x7fffffff - (int32_t)(uint32_t)kl[j] : -1;
    }
}

template <typename T, int D, int KT>
hipError_t launch_k(const Geometry &g, const HeadConsts &hc, const void *q, const float *kbar,
                    const uint16_t *kbar_split, const float *a, const int32_t *retained, const int32_t *n_ret,
                    int32_t *sel, hipStream_t st)
{
    dim3 grid((unsigned)((int64_t)g.NB * g.bh)); // one linear range, renumbered per XCD in the kernel
    if constexpr (sizeof(T) == 2) {
        if (kbar_split) {
            hipLaunchKernelGGL((score_topk_kernel<T, D, KT, true>), grid, dim3(kThreads), 0, st,
                               static_cast<const T *>(q), kbar, kbar_split, a, retained, n_ret, sel, g.N, g.M, g.NB,
                               g.cap, g.prune, g.H, g.B / g.s, g.s, hc);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((score_topk_kernel<T, D, KT, false>), grid, dim3(kThreads), 0, st, static_cast<const T *>(q),
                       kbar, nullptr, a, retained, n_ret, sel, g.N, g.M, g.NB, g.cap, g.prune, g.H, g.B / g.s, g.s,
                       hc);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_t(const Geometry &g, const HeadConsts &hc, const void *q, const float *kbar,
                    const uint16_t *ks, const float *a, const int32_t *retained, const int32_t *n_ret, int32_t *sel,
                    hipStream_t st)
{
    switch (g.K) {
    case 1: return launch_k<T, D, 1>(g, hc, q, kbar, ks, a, retained, n_ret, sel, st);
    case 2: return launch_k<T, D, 2>(g, hc, q, kbar, ks, a, retained, n_ret, sel, st);
    case 3: return launch_k<T, D, 3>(g, hc, q, kbar, ks, a, retained, n_ret, sel, st);
    case 4: return launch_k<T, D, 4>(g, hc, q, kbar, ks, a, retained, n_ret, sel, st);
    case 5: return launch_k<T, D, 5>(g, hc, q, kbar, ks, a, retained, n_ret, sel, st);
    case 6: return launch_k<T, D, 6>(g, hc, q, kbar, ks, a, retained, n_ret, sel, st);
    case 7: return launch_k<T, D, 7>(g, hc, q, kbar, ks, a, retained, n_ret, sel, st);
    default: return launch_k<T, D, 8>(g, hc, q, kbar, ks, a, retained, n_ret, sel, st);
    }
}

} // namespace

hipError_t launch_score_topk(const Geometry &g, const HeadConsts &hc, const void *q, const float *kbar,
                             const uint16_t *kbar_split, const float *a, const int32_t *retained,
                             const int32_t *n_ret, int32_t *sel, hipStream_t st)
{
    if (g.bf16)
        return g.d == 64 ? launch_t<uint16_t, 64>(g, hc, q, kbar, kbar_split, a, retained, n_ret, sel, st)
                         : launch_t<uint16_t, 128>(g, hc, q, kbar, kbar_split, a, retained, n_ret, sel, st);
    return g.d == 64 ? launch_t<float, 64>(g, hc, q, kbar, nullptr, a, retained, n_ret, sel, st)
                     : launch_t<float, 128>(g, hc, q, kbar, nullptr, a, retained, n_ret, sel, st);
}

} // namespace fsl
