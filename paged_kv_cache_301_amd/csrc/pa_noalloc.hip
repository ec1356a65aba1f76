// pa_noalloc.hip -- the static device scratch of pa_decode_noalloc.
//
// Callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc) get the split plan's
// partial results (m, l, o per partition) in `scratch`, a file-scope device
// array of kNoAllocScratchBytes that each GPU holds from the library's load
// until the process ends.  Every call on one GPU shares that GPU's copy and
// leaves its contents behind; the partition kernels write every partial the
// combine reads, so nothing needs clearing between calls, and calls that
// overlap on one GPU (several streams, several host threads) race for it.
//
// In host code `scratch` names a host-side stand-in, not a device address:
// host code uses only the per-device address hipGetSymbolAddress returns,
// looked up once per device with that device current.
#include <mutex>

#include "pa_internal.h"

namespace pa {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
}  // namespace

hipError_t noalloc_scratch(hipStream_t st, void **ptr) {
    static std::mutex mu;
    static void *addr[kMaxScratchDevices] = {};
    int dev = 0;
    hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
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
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace pa
