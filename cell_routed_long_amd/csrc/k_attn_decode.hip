// One launch for the whole attention decode step of FreeSolo (Sec. 3.1, Eq. 2:
// out = o_sr + alpha_h o_lr): the long-range step (Sec. 3.3 "Inference"; App.
// C "Bounded cache", Eq. 15) and the local-branch step (Sec. 3.2, Eqs. 3-4) of
// every (sequence, head) in one workgroup.
//
// Each step alone is a chain of dependent phases that leaves the memory system
// idle most of the time (the long-range step) or a stream of ring reads
// followed by a short combination (the local step).  Here the workgroup's
// first four waves run the long-range step while the other four have the
// local ring in flight: the ring streams in under the long-range chain.  The
// workgroup has 512 threads, the local step's 32 groups of 16 lanes; waves 4-7
// run groups 0-15 and then groups 16-31.  The long-range waves meet at
// barriers of their own (an LDS counter), so the local waves are never held by
// the long-range chain; the whole workgroup meets once at the start (the
// counter is set) and once at the end, where the local step's combination
// reads every group's partials and the long-range output.  That output stays
// in LDS, rounded as the standalone step stores it, so the result is bitwise
// that of fs_longrange_decode followed by fs_local_decode with its output as
// o_lr.
#include "decode_local.h"
#include "decode_lr.h"

namespace fsl {
namespace {

constexpr int kAttnThreads = ldec::kThreads;
static_assert(kAttnThreads == 2 * kThreads, "half the workgroup runs the long-range step");
static_assert(ldec::kGroups % 2 == 0, "the local groups split evenly between the halves");

template <typename T, int D>
__global__ __launch_bounds__(kAttnThreads) void attn_decode_kernel(
    char *__restrict__ state, StateLayout L, StateHeader expect, HeadConsts hc, char *__restrict__ lstate,
    LocalStateLayout LL, LocalStateHeader lexpect, LocalConsts lc, const T *__restrict__ q,
    const T *__restrict__ k_new, const T *__restrict__ v_new, const float *__restrict__ gain, T *__restrict__ out,
    int32_t *__restrict__ sel, int H, int K, int P, int W, float eps)
{
    using S = ldec::Shape<T, D>;
    __shared__ ldec::Smem<D> sm;
    __shared__ float s_olr[D];
    const int64_t bh = blockIdx.x;
    const int t = threadIdx.x;
    const int part = t % ldec::kLanesPerRow;
    const int te = t / S::TPF; // the feature this thread finishes
    __shared__ uint32_t s_bar; // the long-range waves' barrier counter
    if (t == 0)
        s_bar = 0;
    __syncthreads();
    ldec::Entry<T, D> e;
    if (t < kThreads) { // waves 0-3 (wave-uniform): the long-range step
        decode_step_body<T, D, kDecodeFused>(state, L, expect, hc, q, k_new, v_new, gain, nullptr, sel, H, K, P, W,
                                             eps, 1, s_olr, &s_bar);
        e = ldec::step_entry<T, D>(lstate, LL, q, k_new, v_new, bh, part, te);
    } else { // waves 4-7: the local ring, groups 0-15 then 16-31
        e = ldec::step_entry<T, D>(lstate, LL, q, k_new, v_new, bh, part, te);
        const int g = (t - kThreads) / ldec::kLanesPerRow;
        ldec::step_group<T, D>(e, LL, g, part, sm);
        ldec::step_group<T, D>(e, LL, ldec::kGroups / 2 + g, part, sm);
    }
    __syncthreads(); // every group's partials and the long-range output are in LDS
    ldec::step_finish<T, D>(e, LL, lexpect, sm, t, true, lc.alpha[bh % H], s_olr[te], out, bh);
}

template <typename T, int D>
hipError_t attn_t(int32_t bh, int32_t H, int32_t K, int32_t P, int32_t W, float eps, const StateLayout &L,
                  const StateHeader &expect, const HeadConsts &hc, void *state, const LocalStateLayout &LL,
                  const LocalStateHeader &lexpect, const LocalConsts &lc, void *lstate, const void *q,
                  const void *k_new, const void *v_new, const float *gain, void *out, int32_t *sel, hipStream_t st)
{
    hipLaunchKernelGGL((attn_decode_kernel<T, D>), dim3((unsigned)bh), dim3(kAttnThreads), 0, st,
                       static_cast<char *>(state), L, expect, hc, static_cast<char *>(lstate), LL, lexpect, lc,
                       static_cast<const T *>(q), static_cast<const T *>(k_new), static_cast<const T *>(v_new), gain,
                       static_cast<T *>(out), sel, H, K, P, W, eps);
    return hipGetLastError();
}

} // namespace

hipError_t launch_attn_decode(int32_t bh, int32_t H, int32_t d, int32_t bf16, int32_t K, int32_t P, int32_t W,
                              float eps, const StateLayout &L, const StateHeader &expect, const HeadConsts &hc,
                              void *state, const LocalStateLayout &LL, const LocalStateHeader &lexpect,
                              const LocalConsts &lc, void *lstate, const void *q, const void *k_new,
                              const void *v_new, const float *gain, void *out, int32_t *sel, hipStream_t st)
{
    if (bf16)
        return d == 64 ? attn_t<uint16_t, 64>(bh, H, K, P, W, eps, L, expect, hc, state, LL, lexpect, lc, lstate, q,
                                              k_new, v_new, gain, out, sel, st)
                       : attn_t<uint16_t, 128>(bh, H, K, P, W, eps, L, expect, hc, state, LL, lexpect, lc, lstate, q,
                                               k_new, v_new, gain, out, sel, st);
    return d == 64 ? attn_t<float, 64>(bh, H, K, P, W, eps, L, expect, hc, state, LL, lexpect, lc, lstate, q, k_new,
                                       v_new, gain, out, sel, st)
                   : attn_t<float, 128>(bh, H, K, P, W, eps, L, expect, hc, state, LL, lexpect, lc, lstate, q, k_new,
                                        v_new, gain, out, sel, st);
}

} // namespace fsl
