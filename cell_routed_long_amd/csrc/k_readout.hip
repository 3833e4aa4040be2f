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
// tensors use the fp32 MFMA.  The softmax runs in the exp2 domain with a lazy
// running max: it is raised only when a logit exceeds it by more than 16 (so
// every weight stays below 2^16 and the accumulators are rescaled rarely); the
// result is the same softmax up to rounding.  The next cell's keys and values
// are fetched into registers while the current cell is on the matrix cores.
#include "fsl_internal.h"
#include "readout_math.h"

#include <type_traits>

namespace fsl {
namespace {

constexpr int kThreads = 256;


template <typename T, int D>
struct ReadoutSmem;

template <int D>
struct alignas(16) ReadoutSmem<uint16_t, D> {
    static constexpr int kStrideK = D + 8; // bf16 elements per K row
    static constexpr int kStrideV = 32 + 8; // bf16 elements per V^T row (80 bytes: 16-byte aligned, conflict-free)
    static constexpr int kStrideT = D + 8; // bf16 elements per row of a 128-row query/output tile
    union {
        struct {
            uint16_t k[32][kStrideK];
            uint16_t vt[D][kStrideV];
        };
        uint16_t tile[128][kStrideT]; // the block's q tile at entry, its output tile at exit
    };
};

template <int D>
struct alignas(16) ReadoutSmem<float, D> {
    static constexpr int kStride = D + 1;
    float k[32][kStride];
    float v[32][kStride];
};

// bf16 with K <= 4: three workgroups per CU (168 VGPRs) hide more of each cell's memory
// latency; otherwise two
template <typename T, int D, int KT>
constexpr int kReadoutBlocksPerCU = (sizeof(T) == 2 && KT <= 4) ? 3 : 2;

template <typename T, int D, int KT>
__global__ __launch_bounds__(kThreads, (kReadoutBlocksPerCU<T, D, KT>)) void readout_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                           const T *__restrict__ v,
                                                           const int32_t *__restrict__ sel,
                                                           const float *__restrict__ gain, T *__restrict__ out,
                                                           int64_t N, int64_t M, int NB, int H, int s,
                                                           int cells_per_block, float eps)
{
    __shared__ ReadoutSmem<T, D> sm;
    __shared__ int32_t sel_s[128][KT];
    __shared__ int32_t ulist[128 * KT];
    __shared__ int32_t n_u;
    extern __shared__ uint32_t bitmap[]; // ceil(M / 32) words

    constexpr bool kBf16 = sizeof(T) == 2;
    const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int beta = (int)(lb % (uint32_t)NB);
    const int64_t head = (int64_t)(lb / (uint32_t)NB);
    const int h = (int)(head % H);
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int half = lane >> 5;
    const int col = lane & 31;
    const int64_t q0 = (int64_t)beta * 128;
    const int64_t qi = q0 + wave * 32 + col;
    const bool q_ok = qi < N;
    // logits in the exp2 domain: log2(e) / sqrt(d)
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);

    int64_t n_avail = (int64_t)beta * cells_per_block;
    if (n_avail > M)
        n_avail = M;
    const int n_words = (int)((n_avail + 31) / 32);

    // ---- selections of the block's queries, and their union ----
    for (int w = threadIdx.x; w < n_words; w += kThreads)
        bitmap[w] = 0u;
    for (int x = threadIdx.x; x < 128 * KT; x += kThreads) {
        const int r = x / KT, j = x % KT;
        int32_t c = -1;
        if (q0 + r < N)
            c = sel[(head * N + q0 + r) * KT + j];
        if (c >= n_avail)
            c = -1; // not a cell of this block's prefix: ignore
        sel_s[r][j] = c;
    }
    __syncthreads();
    for (int x = threadIdx.x; x < 128 * KT; x += kThreads) {
        const int32_t c = sel_s[x / KT][x % KT];
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
                if (pos < 128 * KT)
                    ulist[pos] = w * 32 + bit;
                ++pos;
            }
            total += __shfl(incl, kWave - 1, kWave);
        }
        if (lane == 0)
            n_u = total < 128 * KT ? total : 128 * KT;
    }
    __syncthreads();
    const int nU = n_u;

    int my_sel[KT];
#pragma unroll
    for (int j = 0; j < KT; ++j)
        my_sel[j] = sel_s[wave * 32 + col][j];

    // ---- query fragments (bf16: the tile comes in through LDS, coalesced) ----
    constexpr int KC = kBf16 ? D / 16 : D / 2;
    using QFrag = typename std::conditional<kBf16, bf16x8, float>::type;
    QFrag qf[KC];
    const int rows = (int)(N - q0 < 128 ? N - q0 : 128);
    if constexpr (kBf16) {
        tile_load_bf16<D, kThreads>(&sm.tile[0][0], sm.kStrideT, q + (head * N + q0) * D, rows);
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

    // ---- gather roles (bf16): K in 16-byte chunks, V^T by (token pair, 8-feature chunk) ----
    constexpr int CPR = D / 8;                   // 16-byte chunks per row
    constexpr int KCH = (32 * CPR) / kThreads;   // K chunks per thread: 1 or 2
    const int tp = threadIdx.x & 15;
    const int fc = threadIdx.x >> 4;             // V roles exist for fc < CPR
    u32x4 pk[KCH > 0 ? KCH : 1], pv0, pv1;
    auto fetch = [&](int cell) {
        const T *kc_src = k + (head * N + (int64_t)cell * s) * D;
        const T *vc_src = v + (head * N + (int64_t)cell * s) * D;
#pragma unroll
        for (int u = 0; u < KCH; ++u) {
            const int ch = threadIdx.x + u * kThreads;
            pk[u] = *reinterpret_cast<const u32x4 *>(kc_src + (int64_t)(ch / CPR) * D + (ch % CPR) * 8);
        }
        if (fc < CPR) {
            pv0 = *reinterpret_cast<const u32x4 *>(vc_src + (int64_t)(2 * tp) * D + fc * 8);
            pv1 = *reinterpret_cast<const u32x4 *>(vc_src + (int64_t)(2 * tp + 1) * D + fc * 8);
        }
    };
    if constexpr (kBf16) {
        if (nU > 0)
            fetch(ulist[0]);
    }

    constexpr int DT = D / 32; // feature tiles of the output
    f32x16 o_acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            o_acc[dt][r] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f; // m_run in the exp2 domain

    for (int x = 0; x < nU; ++x) {
        const int cell = ulist[x];
        __syncthreads();
        // ---- the cell's 32 keys and values into LDS ----
        if constexpr (kBf16) {
#pragma unroll
            for (int u = 0; u < KCH; ++u) {
                const int ch = threadIdx.x + u * kThreads;
                *reinterpret_cast<u32x4 *>(&sm.k[ch / CPR][(ch % CPR) * 8]) = pk[u];
            }
            if (fc < CPR) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t a0 = (pv0[e >> 1] >> (16 * (e & 1))) & 0xffffu;
                    const uint32_t a1 = (pv1[e >> 1] >> (16 * (e & 1))) & 0xffffu;
                    *reinterpret_cast<uint32_t *>(&sm.vt[fc * 8 + e][vt_pos(2 * tp)]) = a0 | (a1 << 16);
                }
            }
        } else {
            const T *kc_src = k + (head * N + (int64_t)cell * s) * D;
            const T *vc_src = v + (head * N + (int64_t)cell * s) * D;
            for (int e = threadIdx.x; e < 32 * D; e += kThreads) {
                const int row = e / D, f = e % D;
                sm.k[row][f] = kc_src[(int64_t)row * D + f];
                sm.v[row][f] = vc_src[(int64_t)row * D + f];
            }
        }
        __syncthreads();
        if constexpr (kBf16) {
            if (x + 1 < nU)
                fetch(ulist[x + 1]); // overlaps the matrix work below
        }

        bool mine = false;
#pragma unroll
        for (int j = 0; j < KT; ++j)
            mine |= my_sel[j] == cell;
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

        // ---- online softmax over the query's own tokens (exp2 domain) ----
        float p[16];
        const float alpha = softmax_cell(acc, mine, scale_log2, m_run, l_run, p);
        if (__ballot(alpha != 1.0f)) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    o_acc[dt][r] *= alpha;
        }

        // ---- O^T[d x 32 queries] += V^T . P^T ----
        if constexpr (kBf16) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 bh, bl;
                split_bf16x8(&p[8 * kk], bh, bl);
                // two feature tiles at a time (fewer registers live): lo parts of both, then
                // hi parts, so no product waits on the one just before it
                constexpr int DP = DT < 2 ? DT : 2;
#pragma unroll
                for (int d0 = 0; d0 < DT; d0 += DP) {
                    bf16x8 av[DP];
#pragma unroll
                    for (int j = 0; j < DP; ++j)
                        av[j] = as_bf16x8(*reinterpret_cast<const u32x4 *>(&sm.vt[(d0 + j) * 32 + col][16 * kk + 8 * half]));
#pragma unroll
                    for (int j = 0; j < DP; ++j)
                        o_acc[d0 + j] = mfma_bf16(av[j], bl, o_acc[d0 + j]);
#pragma unroll
                    for (int j = 0; j < DP; ++j)
                        o_acc[d0 + j] = mfma_bf16(av[j], bh, o_acc[d0 + j]);
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
    const float c = rms_factor<DT>(o_acc, l_run, eps); // y = c * o, times the gain
    const float *gh = gain + (int64_t)h * D;
    // y = g * u * rs for the four features d0..d0+3 (g = 1 without a gain vector;
    // the test is uniform, so each copy below is straight-line code)
    auto rms4 = [&](float (&y)[4], int dt, int rg, int d0, auto with_gain) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            y[e] = o_acc[dt][4 * rg + e] * c;
            if constexpr (decltype(with_gain)::value)
                y[e] = l_run > 0.0f ? y[e] * gh[d0 + e] : 0.0f;
        }
    };
    if constexpr (kBf16) {
        __syncthreads(); // the last cell's LDS reads are done: the tile area takes the output
        auto emit = [&](auto with_gain) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const int d0 = dt * 32 + 8 * rg + 4 * half;
                    float y[4];
                    rms4(y, dt, rg, d0, with_gain);
                    *reinterpret_cast<u32x2 *>(&sm.tile[wave * 32 + col][d0]) =
                        u32x2{cvt_pk_bf16(y[0], y[1]), cvt_pk_bf16(y[2], y[3])};
                }
        };
        if (gain)
            emit(std::true_type{});
        else
            emit(std::false_type{});
        __syncthreads();
        tile_store_bf16<D, kThreads>(reinterpret_cast<uint16_t *>(out) + (head * N + q0) * D, &sm.tile[0][0],
                                     sm.kStrideT, rows);
    } else if (q_ok) {
        T *dst = out + (head * N + qi) * D;
        auto emit = [&](auto with_gain) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const int d0 = dt * 32 + 8 * rg + 4 * half;
                    float y[4];
                    rms4(y, dt, rg, d0, with_gain);
                    *reinterpret_cast<u32x4 *>(dst + d0) = u32x4{__float_as_uint(y[0]), __float_as_uint(y[1]),
                                                                 __float_as_uint(y[2]), __float_as_uint(y[3])};
                }
        };
        if (gain)
            emit(std::true_type{});
        else
            emit(std::false_type{});
    }
}

template <typename T, int D, int KT>
hipError_t launch_k(const Geometry &g, const void *q, const void *k, const void *v, const int32_t *sel,
                    const float *gain, void *out, hipStream_t st)
{
    dim3 grid((unsigned)((int64_t)g.NB * g.bh)); // one linear range, renumbered per XCD in the kernel
    const size_t words = (size_t)((g.M + 31) / 32);
    const size_t dyn = (words > 0 ? words : 1) * sizeof(uint32_t);
    hipLaunchKernelGGL((readout_kernel<T, D, KT>), grid, dim3(kThreads), dyn, st, static_cast<const T *>(q),
                       static_cast<const T *>(k), static_cast<const T *>(v), sel, gain, static_cast<T *>(out), g.N,
                       g.M, g.NB, g.H, g.s, g.B / g.s, g.eps);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_t(const Geometry &g, const void *q, const void *k, const void *v, const int32_t *sel,
                    const float *gain, void *out, hipStream_t st)
{
    switch (g.K) {
    case 1: return launch_k<T, D, 1>(g, q, k, v, sel, gain, out, st);
    case 2: return launch_k<T, D, 2>(g, q, k, v, sel, gain, out, st);
    case 3: return launch_k<T, D, 3>(g, q, k, v, sel, gain, out, st);
    case 4: return launch_k<T, D, 4>(g, q, k, v, sel, gain, out, st);
    case 5: return launch_k<T, D, 5>(g, q, k, v, sel, gain, out, st);
    case 6: return launch_k<T, D, 6>(g, q, k, v, sel, gain, out, st);
    case 7: return launch_k<T, D, 7>(g, q, k, v, sel, gain, out, st);
    default: return launch_k<T, D, 8>(g, q, k, v, sel, gain, out, st);
    }
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
