// Streaming decode of the local branch (FreeSolo, Sec. 3.2, Eqs. 3-4; the
// window moves one token per step) with the branch combination of Eq. 2: the
// state (a rotation table shared by every head and a ring of the last w raw
// keys and values per (sequence, head)), its construction, and the step
// kernel.  The step's arithmetic lives in decode_local.h, which the fused
// attention decode kernel shares.
#include "decode_local.h"

namespace fsl {
namespace {

using ldec::kThreads;

// ---- rotation table: (cos, sin) of o * theta_m, theta_m = base^(-2m/d) ----
__global__ __launch_bounds__(256) void local_table_kernel(float2 *__restrict__ table, int64_t R, int NP, int d,
                                                          float rope_base)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= R * NP)
        return;
    const int m = (int)(e % NP);
    const double theta = pow((double)rope_base, -2.0 * (double)m / (double)d);
    double sn, cs;
    sincos((double)(e / NP) * theta, &sn, &cs);
    table[e] = make_float2((float)cs, (float)sn);
}

// ---- records from the n tokens before position pos (the window keeps the last min(n, w)) ----
template <typename T, int D>
__global__ __launch_bounds__(256) void local_state_build_kernel(char *__restrict__ state, LocalStateLayout L,
                                                                LocalStateHeader hdr, const T *__restrict__ k,
                                                                const T *__restrict__ v, int64_t n, int64_t pos)
{
    const int64_t bh = blockIdx.x;
    const int t = threadIdx.x;
    if (bh == 0 && t == 0)
        *reinterpret_cast<LocalStateHeader *>(state) = hdr;
    char *rec = state + L.off_rec + bh * L.rec_bytes;
    if (t == 0)
        *reinterpret_cast<int64_t *>(rec) = pos;
    constexpr int CPR = D * (int)sizeof(T) / 16; // 16-byte chunks per row
    const int64_t keep = n < L.w ? n : L.w;
    for (int64_t e = t; e < keep * CPR; e += 256) {
        const int64_t r = n - keep + e / CPR; // row of the given tokens; its position is pos - n + r
        const int ch = (int)(e % CPR);
        const int64_t slot = (pos - n + r) % L.slots;
        reinterpret_cast<u32x4 *>(rec + L.off_k + slot * D * (int64_t)sizeof(T))[ch] =
            reinterpret_cast<const u32x4 *>(k + (bh * n + r) * D)[ch];
        reinterpret_cast<u32x4 *>(rec + L.off_v + slot * D * (int64_t)sizeof(T))[ch] =
            reinterpret_cast<const u32x4 *>(v + (bh * n + r) * D)[ch];
    }
}

// ---- one step: one workgroup of 512 threads per (sequence, head) ----
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void local_decode_kernel(char *__restrict__ state, LocalStateLayout L,
                                                                LocalStateHeader expect, LocalConsts lc,
                                                                const T *__restrict__ q,
                                                                const T *__restrict__ k_new,
                                                                const T *__restrict__ v_new,
                                                                const T *__restrict__ o_lr, T *__restrict__ out,
                                                                int H)
{
    using S = ldec::Shape<T, D>;
    __shared__ ldec::Smem<D> sm;
    const int64_t bh = blockIdx.x;
    const int t = threadIdx.x;
    const int te = t / S::TPF; // the feature this thread finishes
    const ldec::Entry<T, D> e = ldec::step_entry<T, D>(state, L, q, k_new, v_new, bh, t % ldec::kLanesPerRow, te);
    // what the combination adds for feature te: requested now, not after the
    // softmax, and without a branch (a load under a branch is waited for at its end)
    const T *olr_src = o_lr ? o_lr : q; // q stands in when there is no o_lr (then unused)
    const T olr_t = olr_src[bh * D + te];
    ldec::step_group<T, D>(e, L, t / ldec::kLanesPerRow, t % ldec::kLanesPerRow, sm);
    __syncthreads();
    ldec::step_finish<T, D>(e, L, expect, sm, t, o_lr != nullptr, lc.alpha[bh % H], ldec::to_f32<T>(olr_t), out, bh);
}

template <typename T, int D>
hipError_t build_t(int32_t bh, const LocalStateLayout &L, const LocalStateHeader &hdr, void *state, const void *k,
                   const void *v, int64_t n, int64_t pos, hipStream_t st)
{
    hipLaunchKernelGGL((local_state_build_kernel<T, D>), dim3((unsigned)bh), dim3(256), 0, st,
                       static_cast<char *>(state), L, hdr, static_cast<const T *>(k), static_cast<const T *>(v), n,
                       pos);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t step_t(int32_t bh, int32_t H, const LocalStateLayout &L, const LocalStateHeader &expect,
                  const LocalConsts &lc, void *state, const void *q, const void *k_new, const void *v_new,
                  const void *o_lr, void *out, hipStream_t st)
{
    hipLaunchKernelGGL((local_decode_kernel<T, D>), dim3((unsigned)bh), dim3(kThreads), 0, st,
                       static_cast<char *>(state), L, expect, lc, static_cast<const T *>(q),
                       static_cast<const T *>(k_new), static_cast<const T *>(v_new), static_cast<const T *>(o_lr),
                       static_cast<T *>(out), H);
    return hipGetLastError();
}

} // namespace

hipError_t launch_local_state_build(int32_t bh, int32_t d, int32_t bf16, const LocalStateLayout &L,
                                    const LocalStateHeader &hdr, void *state, const void *k, const void *v,
                                    int64_t n, int64_t pos, hipStream_t st)
{
    const int NP = d / 2;
    const int64_t entries = (L.w + 1) * NP;
    hipLaunchKernelGGL(local_table_kernel, dim3((unsigned)((entries + 255) / 256)), dim3(256), 0, st,
                       reinterpret_cast<float2 *>(static_cast<char *>(state) + L.off_table), L.w + 1, NP, d,
                       hdr.rope_base);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if (bf16)
        return d == 64 ? build_t<uint16_t, 64>(bh, L, hdr, state, k, v, n, pos, st)
                       : build_t<uint16_t, 128>(bh, L, hdr, state, k, v, n, pos, st);
    return d == 64 ? build_t<float, 64>(bh, L, hdr, state, k, v, n, pos, st)
                   : build_t<float, 128>(bh, L, hdr, state, k, v, n, pos, st);
}

hipError_t launch_local_decode(int32_t bh, int32_t H, int32_t d, int32_t bf16, const LocalStateLayout &L,
                               const LocalStateHeader &expect, const LocalConsts &lc, void *state, const void *q,
                               const void *k_new, const void *v_new, const void *o_lr, void *out, hipStream_t st)
{
    if (bf16)
        return d == 64 ? step_t<uint16_t, 64>(bh, H, L, expect, lc, state, q, k_new, v_new, o_lr, out, st)
                       : step_t<uint16_t, 128>(bh, H, L, expect, lc, state, q, k_new, v_new, o_lr, out, st);
    return d == 64 ? step_t<float, 64>(bh, H, L, expect, lc, state, q, k_new, v_new, o_lr, out, st)
                   : step_t<float, 128>(bh, H, L, expect, lc, state, q, k_new, v_new, o_lr, out, st);
}

} // namespace fsl
