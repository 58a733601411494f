// The static device scratch of pf_gemm_noalloc: the allocation-free form of
// pf_gemm_ws for callers that cannot allocate (code under stream capture, serving
// loops, harnesses that forbid hipMalloc).
//
// `scratch` is a file-scope device array; each GPU the library runs on holds its own
// copy, at its own address, until the process ends. In host code its name is only a
// stand-in for the device symbol, so the address kernels receive comes from
// hipGetSymbolAddress, taken once per device with that device current and cached
// below. Nothing is allocated or freed here.
//
// Every call on a GPU shares that GPU's copy, and the copy keeps the last call's
// contents. The kernels never read scratch they did not write in the same call (the
// fp16 X copy, then any split-K partial sums), so nothing needs clearing; calls that
// overlap on one GPU (different streams, no ordering) race on it.
#include <mutex>

#include "pf_internal.h"

namespace pf {

namespace {

static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(hipStream_t s, void **ptr) {
    int dev = -1;
    hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        int cur = -1;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return e;
        if (e2 != hipSuccess) return e2;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace pf
