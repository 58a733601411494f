// Greedy token of the lm_head logits: the index of the largest logit, the largest
// such index among equal maxima (-0 and +0 equal). The page "oxibonsai-kernels 0.1.4
// - src/gpu_backend/cuda_q_std_prefill.rs" copies the logits of its lm_head GEMV to
// the host and picks the token with Rust's Iterator::max_by over partial_cmp, which
// returns the last of equal maxima; here the pick runs on the device over the same
// f32 logits.
//
// One workgroup of 1024 threads: each thread folds its strided share of the row
// into one 64-bit key, (order-preserving bits of the value) << 32 | index, so that
// the unsigned maximum of the keys is the largest value and, among equal values,
// the largest index; then a reduction across lanes, waves and the workgroup.
#include "pf_device.h"
#include "pf_internal.h"

namespace pf {

namespace {

__device__ __forceinline__ uint64_t argmax_key(float v, uint32_t i) {
    // -0 -> +0; then an order-preserving map of IEEE bits to unsigned integers.
    uint32_t u = __builtin_bit_cast(uint32_t, v == 0.f ? 0.f : v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | i;
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__global__ __launch_bounds__(1024) void argmax_kernel(const float *__restrict__ logits, int n,
                                                      int32_t *__restrict__ token) {
    uint64_t best = 0;  // below every real key
    const int quads = n >> 2;
    for (int q = threadIdx.x; q < quads; q += 1024) {
        const f4_t v = reinterpret_cast<const f4_t *>(logits)[q];
#pragma unroll
        for (int e = 0; e < 4; ++e) best = max_u64(best, argmax_key(v[e], (uint32_t)(4 * q + e)));
    }
    for (int i = 4 * quads + threadIdx.x; i < n; i += 1024)
        best = max_u64(best, argmax_key(logits[i], (uint32_t)i));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)best, off, 64);
        const uint32_t hi = __shfl_xor((uint32_t)(best >> 32), off, 64);
        best = max_u64(best, ((uint64_t)hi << 32) | lo);
    }
    __shared__ uint64_t part[16];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t b = part[0];
        for (int w = 1; w < 16; ++w) b = max_u64(b, part[w]);
        token[0] = (int32_t)(uint32_t)b;
    }
}

}  // namespace

hipError_t launch_argmax(const float *logits, int n, int32_t *token, hipStream_t s) {
    hipLaunchKernelGGL(argmax_kernel, dim3(1), dim3(1024), 0, s, logits, n, token);
    return hipGetLastError();
}

}  // namespace pf
