// fs_longrange_prefill_noalloc: the whole-prompt prefill of the long-range
// branch with its workspace taken from a fixed device array of this library
// instead of the caller, for callers that cannot allocate device memory (code
// under HIP graph capture, serving loops, harnesses that forbid allocation).
//
// `scratch` below is a file-scope device array of kScratchBytes.  Every GPU the
// library runs on holds its own copy until the process ends.  In host code its
// name is only a stand-in for the symbol, not a device address: the address of
// this device's copy comes from hipGetSymbolAddress, looked up once per device
// on the first call made with that device current, and only that address is
// ever handed to a kernel.
//
// Every call on one GPU uses the same array, so calls that overlap on one GPU
// (on different streams, or from different host threads without ordering)
// race on it; calls on one stream are ordered.  Nothing in the workspace needs
// to start at zero: every kernel of the prefill writes what it later reads, so
// the previous call's contents never matter.  No call here allocates or frees
// memory.
#include <mutex>

#include "fsl_internal.h"

#define FSL_EXPORT extern "C" __attribute__((visibility("default")))

namespace fsl {
namespace {

constexpr size_t kScratchBytes = size_t(32) << 20; // 32 MiB
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_lock;
void *g_scratch_ptr[kMaxDevices]; // this device's copy of `scratch`, once looked up

// The address of the current device's `scratch`, looked up on the first call per device.
hipError_t scratch_ptr(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> guard(g_lock);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

} // namespace
} // namespace fsl

using namespace fsl;

FSL_EXPORT size_t fs_noalloc_scratch_bytes(void) { return kScratchBytes; }

FSL_EXPORT fs_status fs_longrange_prefill_noalloc(const fs_shape *shape, const fs_params *prm, const void *q,
                                                  const void *k, const void *v, const float *sigma_h,
                                                  const float *lambda_h, const float *gain, void *out,
                                                  int32_t *sel, void *state, size_t state_bytes, void *stream)
{
    size_t need = 0;
    const fs_status st = prefill_check(shape, prm, q, k, v, sigma_h, lambda_h, out, sel, state, state_bytes, &need);
    if (st != FS_OK)
        return st;
    if (need > kScratchBytes)
        return FS_ERR_WORKSPACE; // the shape needs more workspace than the fixed array holds
    void *ws = nullptr;
    if (scratch_ptr(&ws) != hipSuccess)
        return FS_ERR_HIP;
    return fs_longrange_prefill(shape, prm, q, k, v, sigma_h, lambda_h, gain, out, sel, state, state_bytes, ws,
                                kScratchBytes, stream);
}
