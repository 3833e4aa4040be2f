// Gather-readout with online softmax and fused RMSNorm (FreeSolo, Sec. 3.3
// "Token readout", Eq. 9; Sec. 2 Eq. 1; App. D.2 Eq. 17):
//   u_i = softmax(q_i k_j / sqrt(d), j in S_i) V_{S_i},   o_i = g * u_i / sqrt(|u_i|^2/d + eps),
// with o_i = 0 when S_i is empty.
//
// One workgroup (4 waves, 32 queries each) per (sequence, head, 128-query
// block).  The queries of a block pick their K cells from the same retained
// pool and mostly agree, so the workgroup first forms the union U of the cells
// its queries selected (an LDS bitmap over cell ids, compacted in id order),
// then gathers each cell of U once from HBM into LDS (K row-major, V
// transposed) and lets every wave apply it to its queries:
//   S^T[32 tokens x 32 queries] = K_cell . Q^T      (matrix cores)
//   online-softmax update of the queries that selected the cell
//   O^T[d x 32 queries] += V_cell^T . P^T          (matrix cores)
// A query that did not select the cell contributes p = 0, so each query's
// softmax runs over exactly its own S_i.  Each lane owns one query (and its
// partner lane the other half of the tokens / features), so the softmax
// statistics and the RMSNorm need one cross-lane exchange.
//
// Precision: q and k are exact in bf16 (fp32 products, fp32 accumulation);
// the probabilities are split into bf16 hi + lo parts for the P.V product so
// that the readout keeps ~16 mantissa bits before the final rounding.  fp32
// tensors use the fp32 MFMA.
#include "fsl_internal.h"

#include <type_traits>

namespace fsl {
namespace {

constexpr int kThreads = 256;
constexpr int kKmax = 8;

template <typename T, int D>
struct ReadoutSmem;

template <int D>
struct alignas(16) ReadoutSmem<uint16_t, D> {
    static constexpr int kStrideK = D + 8; // bf16 elements per K row
    static constexpr int kStrideV = 32 + 4; // bf16 elements per V^T row (72 bytes)
    uint16_t k[32][kStrideK];
    uint16_t vt[D][kStrideV];
};

template <int D>
struct alignas(16) ReadoutSmem<float, D> {
    static constexpr int kStride = D + 1;
    float k[32][kStride];
    float v[32][kStride];
};

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void readout_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                           const T *__restrict__ v,
                                                           const int32_t *__restrict__ sel,
                                                           const float *__restrict__ gain, T *__restrict__ out,
                                                           int64_t N, int64_t M, int H, int K, int s,
                                                           int cells_per_block, float eps)
{
    __shared__ ReadoutSmem<T, D> sm;
    __shared__ int32_t sel_s[128][kKmax];
    __shared__ int32_t ulist[128 * kKmax];
    __shared__ int32_t n_u;
    extern __shared__ uint32_t bitmap[]; // ceil(M / 32) words

    const int beta = blockIdx.x;
    const int64_t head = blockIdx.y;
    const int h = (int)(head % H);
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int half = lane >> 5;
    const int col = lane & 31;
    const int64_t q0 = (int64_t)beta * 128;
    const int64_t qi = q0 + wave * 32 + col;
    const bool q_ok = qi < N;
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);

    int64_t n_avail = (int64_t)beta * cells_per_block;
    if (n_avail > M)
        n_avail = M;
    const int n_words = (int)((n_avail + 31) / 32);

    // ---- selections of the block's queries, and their union ----
    for (int w = threadIdx.x; w < n_words; w += kThreads)
        bitmap[w] = 0u;
    for (int x = threadIdx.x; x < 128 * kKmax; x += kThreads) {
        const int r = x / kKmax, j = x % kKmax;
        int32_t c = -1;
        if (j < K && q0 + r < N)
            c = sel[(head * N + q0 + r) * K + j];
        if (c >= n_avail)
            c = -1; // not a cell of this block's prefix: ignore
        sel_s[r][j] = c;
    }
    __syncthreads();
    for (int x = threadIdx.x; x < 128 * kKmax; x += kThreads) {
        const int32_t c = sel_s[x / kKmax][x % kKmax];
        if (c >= 0)
            atomicOr(&bitmap[c >> 5], 1u << (c & 31));
    }
    __syncthreads();
    if (wave == 0) {
        int total = 0;
        for (int base = 0; base < n_words; base += kWave) {
            const int w = base + lane;
            const uint32_t bits = w < n_words ? bitmap[w] : 0u;
            const int cnt = __popc(bits);
            int incl = cnt;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const int y = __shfl_up(incl, o, kWave);
                if (lane >= o)
                    incl += y;
            }
            int pos = total + incl - cnt;
            uint32_t b = bits;
            while (b) {
                const int bit = __ffs(b) - 1;
                b &= b - 1u;
                if (pos < 128 * kKmax)
                    ulist[pos] = w * 32 + bit;
                ++pos;
            }
            total += __shfl(incl, kWave - 1, kWave);
        }
        if (lane == 0)
            n_u = total < 128 * kKmax ? total : 128 * kKmax;
    }
    __syncthreads();
    const int nU = n_u;

    int my_sel[kKmax];
#pragma unroll
    for (int j = 0; j < kKmax; ++j)
        my_sel[j] = sel_s[wave * 32 + col][j];

    // ---- query fragments ----
    constexpr bool kBf16 = sizeof(T) == 2;
    constexpr int KC = kBf16 ? D / 16 : D / 2;
    using QFrag = typename std::conditional<kBf16, bf16x8, float>::type;
    QFrag qf[KC];
    {
        const T *qrow = q + (head * N + (q_ok ? qi : 0)) * D;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            if constexpr (kBf16) {
                u32x4 w = q_ok ? *reinterpret_cast<const u32x4 *>(qrow + kc * 16 + half * 8) : u32x4{0, 0, 0, 0};
                qf[kc] = as_bf16x8(w);
            } else {
                qf[kc] = q_ok ? qrow[kc * 2 + half] : 0.0f;
            }
        }
    }

    constexpr int DT = D / 32; // feature tiles of the output
    f32x16 o_acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            o_acc[dt][r] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;

    for (int x = 0; x < nU; ++x) {
        const int cell = ulist[x];
        const T *kc_src = k + (head * N + (int64_t)cell * s) * D;
        const T *vc_src = v + (head * N + (int64_t)cell * s) * D;
        __syncthreads();
        // ---- gather the cell's 32 keys and values into LDS ----
        if constexpr (kBf16) {
            constexpr int CPR = D / 8; // 16-byte chunks per row
#pragma unroll
            for (int ch = threadIdx.x; ch < 32 * CPR; ch += kThreads) {
                const int row = ch / CPR, c8 = (ch % CPR) * 8;
                *reinterpret_cast<u32x4 *>(&sm.k[row][c8]) =
                    *reinterpret_cast<const u32x4 *>(kc_src + (int64_t)row * D + c8);
            }
            // V^T: thread -> (token pair, 8-feature chunk)
            const int tp = threadIdx.x & 15;
            for (int fc = threadIdx.x >> 4; fc < CPR; fc += kThreads / 16) {
                const u32x4 r0 = *reinterpret_cast<const u32x4 *>(vc_src + (int64_t)(2 * tp) * D + fc * 8);
                const u32x4 r1 = *reinterpret_cast<const u32x4 *>(vc_src + (int64_t)(2 * tp + 1) * D + fc * 8);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t a0 = (r0[e >> 1] >> (16 * (e & 1))) & 0xffffu;
                    const uint32_t a1 = (r1[e >> 1] >> (16 * (e & 1))) & 0xffffu;
                    *reinterpret_cast<uint32_t *>(&sm.vt[fc * 8 + e][2 * tp]) = a0 | (a1 << 16);
                }
            }
        } else {
            for (int e = threadIdx.x; e < 32 * D; e += kThreads) {
                const int row = e / D, f = e % D;
                sm.k[row][f] = kc_src[(int64_t)row * D + f];
                sm.v[row][f] = vc_src[(int64_t)row * D + f];
            }
        }
        __syncthreads();

        bool mine = false;
#pragma unroll
        for (int j = 0; j < kKmax; ++j)
            mine |= (j < K) && (my_sel[j] == cell);
        if (__ballot(mine) == 0ull)
            continue; // no query of this wave reads the cell

        // ---- logits S^T[32 tokens x 32 queries] ----
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[r] = 0.0f;
        if constexpr (kBf16) {
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const u32x4 w = *reinterpret_cast<const u32x4 *>(&sm.k[col][kc * 16 + half * 8]);
                acc = mfma_bf16(as_bf16x8(w), qf[kc], acc);
            }
        } else {
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
                acc = mfma_f32(sm.k[col][kc * 2 + half], qf[kc], acc);
        }

        // ---- online softmax over the query's own tokens ----
        float p[16];
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            p[r] = acc[r] * inv_sqrt_d;
            tmax = fmaxf(tmax, p[r]);
        }
        tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
        float alpha = 1.0f, psum = 0.0f;
        if (mine) {
            const float m_new = fmaxf(m_run, tmax);
            alpha = expf(m_run - m_new); // 0 on the first cell (m_run = -inf)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                p[r] = expf(p[r] - m_new);
                psum += p[r];
            }
            m_run = m_new;
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                p[r] = 0.0f;
        }
        psum += shfl_xor_f(psum, 32);
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                o_acc[dt][r] *= alpha;

        // ---- O^T[d x 32 queries] += V^T . P^T ----
        if constexpr (kBf16) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                u32x4 ph, pl;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float x0 = p[8 * kk + 2 * w], x1 = p[8 * kk + 2 * w + 1];
                    const uint32_t h0 = f32_to_bf16_bits(x0), h1 = f32_to_bf16_bits(x1);
                    ph[w] = h0 | (h1 << 16);
                    pl[w] = pack_bf16x2(x0 - bf16_bits_to_f32(h0), x1 - bf16_bits_to_f32(h1));
                }
                const bf16x8 bh = as_bf16x8(ph), bl = as_bf16x8(pl);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const int m = dt * 32 + col;
                    const u32x2 lo4 = *reinterpret_cast<const u32x2 *>(&sm.vt[m][16 * kk + 4 * half]);
                    const u32x2 hi4 = *reinterpret_cast<const u32x2 *>(&sm.vt[m][16 * kk + 8 + 4 * half]);
                    const bf16x8 av = as_bf16x8(u32x4{lo4[0], lo4[1], hi4[0], hi4[1]});
                    o_acc[dt] = mfma_bf16(av, bl, o_acc[dt]);
                    o_acc[dt] = mfma_bf16(av, bh, o_acc[dt]);
                }
            }
        } else {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    o_acc[dt] = mfma_f32(sm.v[acc_row(r, half)][dt * 32 + col], p[r], o_acc[dt]);
        }
    }

    // ---- normalise, RMSNorm over d, write ----
    const float inv_l = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    float ms = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float u = o_acc[dt][r] * inv_l;
            o_acc[dt][r] = u;
            ms += u * u;
        }
    ms += shfl_xor_f(ms, 32);
    const float rs = 1.0f / sqrtf(ms / (float)D + eps);
    if (q_ok) {
        T *dst = out + (head * N + qi) * D;
        const float *gh = gain ? gain + (int64_t)h * D : nullptr;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int d0 = dt * 32 + 8 * rg + 4 * half;
                float y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float gv = gh ? gh[d0 + e] : 1.0f;
                    y[e] = l_run > 0.0f ? gv * o_acc[dt][4 * rg + e] * rs : 0.0f;
                }
                if constexpr (kBf16) {
                    *reinterpret_cast<u32x2 *>(dst + d0) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
                } else {
                    *reinterpret_cast<u32x4 *>(dst + d0) = u32x4{__float_as_uint(y[0]), __float_as_uint(y[1]),
                                                                 __float_as_uint(y[2]), __float_as_uint(y[3])};
                }
            }
    }
}

template <typename T, int D>
hipError_t launch_t(const Geometry &g, const void *q, const void *k, const void *v, const int32_t *sel,
                    const float *gain, void *out, hipStream_t st)
{
    dim3 grid((unsigned)g.NB, (unsigned)g.bh);
    const size_t words = (size_t)((g.M + 31) / 32);
    const size_t dyn = (words > 0 ? words : 1) * sizeof(uint32_t);
    hipLaunchKernelGGL((readout_kernel<T, D>), grid, dim3(kThreads), dyn, st, static_cast<const T *>(q),
                       static_cast<const T *>(k), static_cast<const T *>(v), sel, gain, static_cast<T *>(out), g.N,
                       g.M, g.H, g.K, g.s, g.B / g.s, g.eps);
    return hipGetLastError();
}

} // namespace

hipError_t launch_readout(const Geometry &g, const void *q, const void *k, const void *v, const int32_t *sel,
                          const float *gain, void *out, hipStream_t st)
{
    if (g.bf16)
        return g.d == 64 ? launch_t<uint16_t, 64>(g, q, k, v, sel, gain, out, st)
                         : launch_t<uint16_t, 128>(g, q, k, v, sel, gain, out, st);
    return g.d == 64 ? launch_t<float, 64>(g, q, k, v, sel, gain, out, st)
                     : launch_t<float, 128>(g, q, k, v, sel, gain, out, st);
}

} // namespace fsl
