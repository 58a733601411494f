// Greedy token of the lm_head logits: the index of the largest logit, the largest
// such index among equal maxima (-0 and +0 equal). The page "oxibonsai-kernels 0.1.4
// - src/gpu_backend/cuda_q_std_prefill.rs" copies the logits of its lm_head GEMV to
// the host and picks the token with Rust's Iterator::max_by over partial_cmp, which
// returns the last of equal maxima; here the pick runs on the device over the same
// f32 logits.
//
// One workgroup of 1024 threads. Each thread scans its strided share of the row in
// increasing index order keeping (value, index) with `v >= best`, so among equal
// values its later index wins, and -0 == +0 as IEEE compares them; then the pairs
// are combined across lanes, waves and the workgroup (larger value, or the larger
// index on equal values). NaN never wins a comparison; a row of NaN gives 0.
#include "pf_device.h"
#include "pf_internal.h"

namespace pf {

namespace {

struct Best {
    float v;
    int i;
};

__device__ __forceinline__ Best pick(Best a, Best b) {
    return (b.v > a.v || (b.v == a.v && b.i > a.i)) ? b : a;
}

__global__ __launch_bounds__(1024) void argmax_kernel(const float *__restrict__ logits, int n,
                                                      int32_t *__restrict__ token) {
    Best best{-__builtin_inff(), -1};
    const int quads = n >> 2;
    // Eight independent 16-byte loads in flight per thread per round.
    constexpr int U = 8;
    for (int q0 = threadIdx.x; q0 < quads; q0 += 1024 * U) {
        f4_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int q = q0 + 1024 * u;
            v[u] = q < quads ? reinterpret_cast<const f4_t *>(logits)[q] : f4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int q = q0 + 1024 * u;
            if (q < quads) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (v[u][e] >= best.v) best = Best{v[u][e], 4 * q + e};
                }
            }
        }
    }
    for (int i = 4 * quads + threadIdx.x; i < n; i += 1024)
        if (logits[i] >= best.v) best = Best{logits[i], i};
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        best = pick(best, Best{__shfl_xor(best.v, off, 64), __shfl_xor(best.i, off, 64)});
    __shared__ Best part[16];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        Best b = part[0];
        for (int w = 1; w < 16; ++w) b = pick(b, part[w]);
        token[0] = b.i < 0 ? 0 : b.i;
    }
}

}  // namespace

hipError_t launch_argmax(const float *logits, int n, int32_t *token, hipStream_t s) {
    hipLaunchKernelGGL(argmax_kernel, dim3(1), dim3(1024), 0, s, logits, n, token);
    return hipGetLastError();
}

}  // namespace pf
