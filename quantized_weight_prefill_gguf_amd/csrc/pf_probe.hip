// The benchmark's plain-read floor (include/pf_probe.h): a launch that only streams
// bytes from HBM, with the launch shape of a persistent streaming kernel (every CU,
// four 16-byte loads in flight per lane per iteration).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pf_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kBlocks = 256 * 8;  // 8 workgroups per CU on 256 CUs

typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void probe_read_kernel(const u4_t *__restrict__ src, int64_t n16,
                                                              uint32_t *__restrict__ sink) {
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u4_t a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^
               d[2] ^ d[3];
    }
    for (; i < n16; i += stride) {
        const u4_t a = src[i];
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
    // one word per workgroup (xor over its lanes), so the loads are live
    for (int d = 32; d >= 1; d >>= 1) acc ^= __shfl_xor(acc, d, 64);
    __shared__ uint32_t part[kThreads / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

extern "C" {

int pf_probe_read(const void *src, int64_t bytes, uint32_t *sink, void *stream) {
    if (bytes < 16 || bytes % 16 != 0) return 5;
    if (!src || !sink) return 1;
    if ((reinterpret_cast<uintptr_t>(src) & 15u) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return 6;
    hipLaunchKernelGGL(probe_read_kernel, dim3(kBlocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u4_t *>(src), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : 8;
}

int64_t pf_probe_read_sink_words(void) { return kBlocks; }

}  // extern "C"
