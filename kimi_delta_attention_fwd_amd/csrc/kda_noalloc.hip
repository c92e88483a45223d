/*
 * kda_noalloc.hip -- the built-in scratch of kda_fwd_noalloc.
 *
 * kda_fwd takes its workspace from the caller. Some callers cannot allocate
 * device memory at call time (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc); kda_fwd_noalloc serves them from
 * the file-scope device array below instead. Each GPU the library runs on holds
 * its own copy of the array (KDA_NOALLOC_SCRATCH_BYTES) until the process ends.
 *
 * In host code the array's name is only a host-side stand-in for the symbol:
 * its device address is looked up once per device, with that device current,
 * through hipGetSymbolAddress, and host code passes that address (never the
 * name) to the kernels, exactly where kda_fwd passes the caller's workspace.
 */
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda.h"

static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices]; /* device address of `scratch` per device, or NULL before the lookup */
} // namespace

/* Device address of the scratch array on the GPU that `stream` belongs to (the
 * current device for the NULL stream). The first call on a device makes that
 * device current, looks the address up and restores the previous device.
 * Returns hipSuccess, or the HIP error of the lookup. */
extern "C" hipError_t kda_noalloc_scratch(void *stream, void **ptr)
{
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (p == nullptr || ((uintptr_t)p & 255u) != 0) return hipErrorInvalidValue;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}
