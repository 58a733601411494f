// Batched RMSNorm prologue of a projection: x_t -> x_t / sqrt(mean_j x_t[j]^2 + eps)
// * w[j], the step that precedes the QKV and gate/up GEMMs on the page "aprender-serve
// 0.70.2 - src/gguf/cuda/forward_qwen35_cuda_prefill.rs" (`batched_rmsnorm_into`,
// one norm weight of hidden floats shared by every row, one eps).
//
//  - rms_inv_kernel: one workgroup per row; inv[t] = 1 / sqrt(mean + eps), the sum
//    of squares in f32 (per-thread partial sums, then a tree over lanes and waves).
//  - rms_apply_kernel: Xn[t][j] = X[t][j] * inv[t] * w[j] in f32, for the kernels
//    that read f32 X. The f16 leg's matrix-core GEMM instead applies inv and w in
//    its conversion of X to binary16 (pf_gemm_f16.hip), so there the normalised
//    rows never exist in f32.
#include "pf_device.h"
#include "pf_internal.h"

namespace pf {

namespace {

// k % 256 == 0 (checked by the API), so a row is whole float4s, 16-byte aligned.
__global__ __launch_bounds__(256) void rms_inv_kernel(const float *__restrict__ X, int k, float eps,
                                                      float *__restrict__ inv) {
    const int t = blockIdx.x;
    const f4_t *x = reinterpret_cast<const f4_t *>(X + (size_t)t * k);
    float s = 0.f;
    for (int q = threadIdx.x; q < k / 4; q += 256) {
        const f4_t v = x[q];
        s += (v[0] * v[0] + v[1] * v[1]) + (v[2] * v[2] + v[3] * v[3]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    __shared__ float part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        const float total = (part[0] + part[1]) + (part[2] + part[3]);
        inv[t] = 1.0f / sqrtf(total / (float)k + eps);
    }
}

__global__ __launch_bounds__(256) void rms_apply_kernel(const float *__restrict__ X,
                                                        const float *__restrict__ inv,
                                                        const float *__restrict__ w,
                                                        float *__restrict__ Xn, int k, int quads) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= quads) return;
    const int t = (int)((long)i * 4 / k), j = i * 4 - t * k;
    const f4_t v = reinterpret_cast<const f4_t *>(X)[i];
    const f4_t g = *reinterpret_cast<const f4_t *>(w + j);
    const float r = inv[t];
    reinterpret_cast<f4_t *>(Xn)[i] = f4_t{v[0] * r * g[0], v[1] * r * g[1], v[2] * r * g[2],
                                           v[3] * r * g[3]};
}

}  // namespace

hipError_t launch_rms_inv(const float *X, int T, int k, float eps, float *inv, hipStream_t s) {
    hipLaunchKernelGGL(rms_inv_kernel, dim3(T), dim3(256), 0, s, X, k, eps, inv);
    return hipGetLastError();
}

hipError_t launch_rms_apply(const float *X, const float *inv, const float *w, float *Xn, int T, int k,
                            hipStream_t s) {
    const int quads = T * (k / 4);
    hipLaunchKernelGGL(rms_apply_kernel, dim3((quads + 255) / 256), dim3(256), 0, s, X, inv, w, Xn, k,
                       quads);
    return hipGetLastError();
}

}  // namespace pf
