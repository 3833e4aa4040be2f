// Cell summaries (FreeSolo, Sec. 3.3 "Cells", Eq. 5): for every complete cell,
// the mean key kbar_c and the largest key norm a_c over its s = 32 tokens.
//
// One wave per cell streams the cell's 32 x d keys once with 16-byte loads
// (a cell is one contiguous 4-16 KB span, so a wave's loads are fully
// coalesced).  Lane l always reads the same 16-byte feature group of every
// row it touches, so the column sums need only a final cross-lane reduction,
// and each row's squared norm is reduced across the lanes that share the row.
// Sums and squared norms accumulate in fp64 (exact for bf16 keys) and are
// rounded once to fp32.  Optionally the fp32 mean is also written as three
// bf16 parts (hi, mid, lo), the operands the block scorer feeds to the bf16
// matrix cores, so that the split is done once per cell instead of once per
// query block, and its Euclidean norm (fp64, rounded once), which bounds the
// content term of every score of the cell (|q . kbar| <= |q| |kbar|).
// HBM-bound: the kernel reads each key exactly once, with streaming
// (non-temporal) loads, so the keys do not displace from the caches the cells
// and mean keys the routing and readout kernel gathers next.
#include "fsl_internal.h"

namespace fsl {
namespace {

template <typename T, int D>
__global__ __launch_bounds__(256, 5) void cell_summaries_kernel(const T *__restrict__ k, float *__restrict__ kbar,
                                                             float *__restrict__ a,
                                                             uint16_t *__restrict__ kbar_split,
                                                             float *__restrict__ kbar_norm,
                                                             double *__restrict__ kbar64, double *__restrict__ a64,
                                                             int64_t N, int64_t M, int64_t total_cells)
{
    constexpr int EPC = 16 / (int)sizeof(T); // elements per 16-byte chunk
    constexpr int R = D / EPC;               // chunks per key row: 8, 16 or 32
    constexpr int CHUNKS = 32 * R;           // chunks per cell (s = 32)
    constexpr int PER_LANE = CHUNKS / kWave; // 4, 8 or 16
    constexpr int ROWS_STEP = kWave / R;     // rows advanced per load step
    static_assert(kWave % R == 0, "feature groups must tile the wave");

    const int lane = threadIdx.x & (kWave - 1);
    const int64_t cell = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
    if (cell >= total_cells)
        return; // whole wave exits together

    const int64_t seq_head = cell / M;
    const int64_t c = cell - seq_head * M;
    const T *base = k + (seq_head * N + c * 32) * D;
    const int group = lane % R;   // feature group of this lane
    const int row0 = lane / R;    // first row of this lane

    u32x4 buf[PER_LANE];
#pragma unroll
    for (int t = 0; t < PER_LANE; ++t)
        buf[t] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(base + (int64_t)(row0 + t * ROWS_STEP) * D + group * EPC));

    double colsum[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e)
        colsum[e] = 0.0;
    double best = 0.0;

#pragma unroll
    for (int t = 0; t < PER_LANE; ++t) {
        double vals[EPC];
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                vals[2 * w] = (double)bf16_bits_to_f32(buf[t][w] & 0xffffu);
                vals[2 * w + 1] = (double)bf16_bits_to_f32(buf[t][w] >> 16);
            }
        } else {
#pragma unroll
            for (int w = 0; w < 4; ++w)
                vals[w] = (double)__uint_as_float(buf[t][w]);
        }
        double sq = 0.0;
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
            colsum[e] += vals[e];
            sq += vals[e] * vals[e];
        }
        // squared norm of the row: reduce over the R lanes sharing it
#pragma unroll
        for (int m = 1; m < R; m <<= 1)
            sq += shfl_xor_d(sq, m);
        best = fmax(best, sq);
    }
    // column sums: reduce over the lanes that share this feature group
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
#pragma unroll
        for (int m = R; m < kWave; m <<= 1)
            colsum[e] += shfl_xor_d(colsum[e], m);
    }
#pragma unroll
    for (int m = R; m < kWave; m <<= 1)
        best = fmax(best, shfl_xor_d(best, m));

    float m[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e)
        m[e] = (float)(colsum[e] * (1.0 / 32.0));
    if (kbar_norm) { // |kbar|, from the fp32 mean as stored; lanes < R hold all d features
        double nsq = 0.0;
#pragma unroll
        for (int e = 0; e < EPC; ++e)
            nsq += (double)m[e] * (double)m[e];
#pragma unroll
        for (int mm = 1; mm < R; mm <<= 1)
            nsq += shfl_xor_d(nsq, mm);
        if (lane == 0)
            kbar_norm[cell] = (float)sqrt(nsq);
    }
    if (kbar64 && lane < R) { // the fp64 mean (exact for bf16 keys: the sums are)
#pragma unroll
        for (int e = 0; e < EPC; ++e)
            kbar64[cell * D + group * EPC + e] = colsum[e] * (1.0 / 32.0);
    }
    if (lane < R) {
        float *dst = kbar + cell * D + group * EPC;
#pragma unroll
        for (int e = 0; e < EPC; ++e)
            dst[e] = m[e];
        if (kbar_split) { // bf16 hi, mid, lo parts of the fp32 mean (24 mantissa bits in all)
            uint32_t pk[3][EPC / 2];
#pragma unroll
            for (int e = 0; e < EPC; e += 2) {
                const uint32_t hi = cvt_pk_bf16(m[e], m[e + 1]);
                const float r0 = m[e] - bf16_bits_to_f32(hi & 0xffffu), r1 = m[e + 1] - bf16_bits_to_f32(hi >> 16);
                const uint32_t mid = cvt_pk_bf16(r0, r1);
                const float s0 = r0 - bf16_bits_to_f32(mid & 0xffffu), s1 = r1 - bf16_bits_to_f32(mid >> 16);
                pk[0][e / 2] = hi;
                pk[1][e / 2] = mid;
                pk[2][e / 2] = cvt_pk_bf16(s0, s1);
            }
#pragma unroll
            for (int part = 0; part < 3; ++part) {
                uint32_t *o = reinterpret_cast<uint32_t *>(kbar_split + (cell * 3 + part) * D + group * EPC);
#pragma unroll
                for (int e = 0; e < EPC / 2; ++e)
                    o[e] = pk[part][e];
            }
        }
    }
    if (lane == 0) {
        a[cell] = (float)sqrt(best);
        if (a64)
            a64[cell] = sqrt(best);
    }
}

template <typename T, int D>
hipError_t launch_t(const Geometry &g, const void *k, float *kbar, float *a, uint16_t *kbar_split, float *kbar_norm,
                    double *kbar64, double *a64, hipStream_t st)
{
    const int64_t total = (int64_t)g.bh * g.M;
    if (total == 0)
        return hipSuccess;
    const int64_t blocks = (total + 3) / 4;
    hipLaunchKernelGGL((cell_summaries_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, st,
                       static_cast<const T *>(k), kbar, a, kbar_split, kbar_norm, kbar64, a64, g.N, g.M, total);
    return hipGetLastError();
}

} // namespace

hipError_t launch_cell_summaries(const Geometry &g, const void *k, float *kbar, float *a, uint16_t *kbar_split,
                                 float *kbar_norm, hipStream_t st, double *kbar64, double *a64)
{
    if (g.bf16)
        return g.d == 64 ? launch_t<uint16_t, 64>(g, k, kbar, a, kbar_split, kbar_norm, kbar64, a64, st)
                         : launch_t<uint16_t, 128>(g, k, kbar, a, kbar_split, kbar_norm, kbar64, a64, st);
    return g.d == 64 ? launch_t<float, 64>(g, k, kbar, a, kbar_split, kbar_norm, kbar64, a64, st)
                     : launch_t<float, 128>(g, k, kbar, a, kbar_split, kbar_norm, kbar64, a64, st);
}

} // namespace fsl
