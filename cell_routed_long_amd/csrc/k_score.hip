// Block-level cell scoring and per-query top-K (FreeSolo, Sec. 3.3 "Cell scoring",
// Eq. 7, and "Per-query selection"):
//   r_ic = q_i . kbar_c / sqrt(d) + lambda_h a_c erf((i - p_c) / (2 sigma_h)),
//   T_i  = the min(K, |A_i|) best cells of A_i by (score desc, id asc).
//
// One workgroup (4 waves) per (sequence, head, 128-query block): the block's
// queries share the retained set A_beta (FS-L) or the prefix C_beta (FS).  The
// retained mean keys are staged through LDS 32 cells at a time and each wave
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
constexpr int kKmax = 8;

template <typename T, int D>
struct ScoreSmem;

template <int D>
struct alignas(16) ScoreSmem<uint16_t, D> {
    static constexpr int kStride = D + 8; // bf16 elements per row (16-byte pad against bank conflicts)
    uint16_t kb[3][32][kStride];
    float a[32];
    int32_t id[32];
};

template <int D>
struct alignas(16) ScoreSmem<float, D> {
    static constexpr int kStride = D + 1;
    float kb[32][kStride];
    float a[32];
    int32_t id[32];
};

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void score_topk_kernel(
    const T *__restrict__ q, const float *__restrict__ kbar, const float *__restrict__ a,
    const int32_t *__restrict__ retained, const int32_t *__restrict__ n_ret, int32_t *__restrict__ sel,
    int64_t N, int64_t M, int NB, int cap, int K, int prune, int H, int cells_per_block, int s,
    HeadConsts hc)
{
    __shared__ ScoreSmem<T, D> sm;
    const int beta = blockIdx.x;
    const int64_t head = blockIdx.y;
    const int h = (int)(head % H);
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int half = lane >> 5;
    const int col = lane & 31;
    const int64_t qi = (int64_t)beta * 128 + wave * 32 + col; // this lane's query position
    const bool q_ok = qi < N;
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);
    const float inv2s = hc.inv_two_sigma[h];
    const float lam = hc.lambda[h];

    int64_t n_avail = (int64_t)beta * cells_per_block;
    if (n_avail > M)
        n_avail = M;
    const int nA = prune ? n_ret[head * NB + beta] : (int)n_avail;
    const int32_t *A = prune ? retained + (head * NB + beta) * (int64_t)cap : nullptr;

    // query fragments (B operand): column `col`, k values of group `half`
    constexpr int KC = (sizeof(T) == 2) ? D / 16 : D / 2;
    using QFrag = typename std::conditional<sizeof(T) == 2, bf16x8, float>::type;
    QFrag qf[KC];
    {
        const T *qrow = q + (head * N + (q_ok ? qi : 0)) * D;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            if constexpr (sizeof(T) == 2) {
                u32x4 w = q_ok ? *reinterpret_cast<const u32x4 *>(qrow + kc * 16 + half * 8) : u32x4{0, 0, 0, 0};
                qf[kc] = as_bf16x8(w);
            } else {
                qf[kc] = q_ok ? qrow[kc * 2 + half] : 0.0f;
            }
        }
    }

    float tv[kKmax];
    int ti[kKmax];
#pragma unroll
    for (int j = 0; j < kKmax; ++j) {
        tv[j] = -INFINITY;
        ti[j] = INT_MAX;
    }

    for (int t0 = 0; t0 < nA; t0 += 32) {
        __syncthreads();
        // ---- stage 32 mean keys (and their norms and ids) in LDS ----
        {
            const int row = threadIdx.x >> 3;   // 32 rows, 8 threads per row
            const int part = threadIdx.x & 7;
            constexpr int PER = D / 8;          // floats per thread: 8 or 16
            const int x = t0 + row;
            const int cid = x < nA ? (prune ? A[x] : x) : -1;
            if (part == 0) {
                sm.id[row] = cid;
                sm.a[row] = cid >= 0 ? a[head * M + cid] : 0.0f;
            }
            float vals[PER];
            if (cid >= 0) {
                const float *src = kbar + (head * M + cid) * D + part * PER;
#pragma unroll
                for (int e = 0; e < PER; e += 4) {
                    const u32x4 w = *reinterpret_cast<const u32x4 *>(src + e);
                    vals[e] = __uint_as_float(w[0]);
                    vals[e + 1] = __uint_as_float(w[1]);
                    vals[e + 2] = __uint_as_float(w[2]);
                    vals[e + 3] = __uint_as_float(w[3]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < PER; ++e)
                    vals[e] = 0.0f;
            }
            if constexpr (sizeof(T) == 2) {
#pragma unroll
                for (int e = 0; e < PER; e += 2) {
                    uint32_t hi2 = 0, mid2 = 0, lo2 = 0;
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const float v0 = vals[e + u];
                        const uint32_t hb = f32_to_bf16_bits(v0);
                        const float r1 = v0 - bf16_bits_to_f32(hb);
                        const uint32_t mb = f32_to_bf16_bits(r1);
                        const float r2 = r1 - bf16_bits_to_f32(mb);
                        const uint32_t lb = f32_to_bf16_bits(r2);
                        hi2 |= hb << (16 * u);
                        mid2 |= mb << (16 * u);
                        lo2 |= lb << (16 * u);
                    }
                    const int c0 = part * PER + e;
                    *reinterpret_cast<uint32_t *>(&sm.kb[0][row][c0]) = hi2;
                    *reinterpret_cast<uint32_t *>(&sm.kb[1][row][c0]) = mid2;
                    *reinterpret_cast<uint32_t *>(&sm.kb[2][row][c0]) = lo2;
                }
            } else {
#pragma unroll
                for (int e = 0; e < PER; ++e)
                    sm.kb[row][part * PER + e] = vals[e];
            }
        }
        __syncthreads();

        // ---- S^T[32 cells x 32 queries] on the matrix cores ----
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[r] = 0.0f;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int sp = 2; sp >= 0; --sp) { // smallest parts first
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    const u32x4 w = *reinterpret_cast<const u32x4 *>(&sm.kb[sp][col][kc * 16 + half * 8]);
                    acc = mfma_bf16(as_bf16x8(w), qf[kc], acc);
                }
            }
        } else {
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
                acc = mfma_f32(sm.kb[col][kc * 2 + half], qf[kc], acc);
        }

        // ---- Eq. 7 and the running top-K of this lane's query ----
        if (q_ok) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = acc_row(r, half);
                const int cid = sm.id[row];
                if (cid >= 0) {
                    const float delta = (float)(qi - ((int64_t)cid * s + s / 2)); // i - p_c, exact integer
                    const float prior = lam * sm.a[row];
                    const float score = fmaf(prior, erff(delta * inv2s), acc[r] * inv_sqrt_d);
                    topk_insert<kKmax>(tv, ti, K, score, cid);
                }
            }
        }
    }

    // ---- merge with the partner lane (same query, other 16 rows) ----
    float pv[kKmax];
    int pi[kKmax];
#pragma unroll
    for (int j = 0; j < kKmax; ++j) {
        pv[j] = shfl_xor_f(tv[j], 32);
        pi[j] = shfl_xor_i(ti[j], 32);
    }
#pragma unroll
    for (int j = 0; j < kKmax; ++j)
        if (j < K && pi[j] != INT_MAX)
            topk_insert<kKmax>(tv, ti, K, pv[j], pi[j]);

    if (q_ok && half == 0) {
        int32_t *dst = sel + (head * N + qi) * K;
#pragma unroll
        for (int j = 0; j < kKmax; ++j)
            if (j < K)
                dst[j] = ti[j] == INT_MAX ? -1 : ti[j];
    }
}

template <typename T, int D>
hipError_t launch_t(const Geometry &g, const HeadConsts &hc, const void *q, const float *kbar, const float *a,
                    const int32_t *retained, const int32_t *n_ret, int32_t *sel, hipStream_t st)
{
    dim3 grid((unsigned)g.NB, (unsigned)g.bh);
    hipLaunchKernelGGL((score_topk_kernel<T, D>), grid, dim3(kThreads), 0, st, static_cast<const T *>(q), kbar, a,
                       retained, n_ret, sel, g.N, g.M, g.NB, g.cap, g.K, g.prune, g.H, g.B / g.s, g.s, hc);
    return hipGetLastError();
}

} // namespace

hipError_t launch_score_topk(const Geometry &g, const HeadConsts &hc, const void *q, const float *kbar,
                             const float *a, const int32_t *retained, const int32_t *n_ret, int32_t *sel,
                             hipStream_t st)
{
    if (g.bf16)
        return g.d == 64 ? launch_t<uint16_t, 64>(g, hc, q, kbar, a, retained, n_ret, sel, st)
                         : launch_t<uint16_t, 128>(g, hc, q, kbar, a, retained, n_ret, sel, st);
    return g.d == 64 ? launch_t<float, 64>(g, hc, q, kbar, a, retained, n_ret, sel, st)
                     : launch_t<float, 128>(g, hc, q, kbar, a, retained, n_ret, sel, st);
}

} // namespace fsl
