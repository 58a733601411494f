// Small-T twin of the GEMM (1 <= T <= 8): the weight stream is the cost, so each
// weight block is read from HBM once, decoded in registers and applied to all T
// activation rows; partial sums are combined by a cross-lane reduction. This is
// the kernel-level form of the single-token `gemv_q4_0_pf` / `gemv_q8_0_pf` on the
// page "oxibonsai-kernels 0.1.4 - src/gpu_backend/cuda_q_std_prefill.rs", widened
// to up to 8 rows (the same page's batch tests step tokens 8 at a time).
//
// f32 arithmetic throughout: exact f32 weights, fp32 FMA accumulation.
// One wave computes one output column (both gate and up rows for SWIGLU); its
// lanes split the row's blocks; a butterfly over the 64 lanes sums them.
#include "pf_device.h"
#include "pf_internal.h"

namespace pf {

template <int QT, int TT>
__device__ __forceinline__ void gemv_row_accumulate(const uint8_t *__restrict__ row,
                                                    const float *__restrict__ X, int k, int T,
                                                    int lane, float acc[TT]) {
    constexpr int BB = BlockTraits<QT>::BYTES;
    constexpr int HW = BlockTraits<QT>::HALFWORDS;
    const int nb = k >> 5;
    for (int b = lane; b < nb; b += 64) {
        const uint16_t *src = reinterpret_cast<const uint16_t *>(row + (size_t)b * BB);
        uint16_t hw[HW];
#pragma unroll
        for (int i = 0; i < HW; ++i) hw[i] = src[i];
        const float d = fp16_bits_to_f32(hw[0]);
        float w[32];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t byte = (hw[1 + (j >> 1)] >> (8 * (j & 1))) & 0xFFu;
            if constexpr (QT == Q4_0) {
                w[j] = d * (float)((int)(byte & 15u) - 8);
                w[j + 16] = d * (float)((int)(byte >> 4) - 8);
            } else {
                w[j] = d * (float)(int)(int8_t)(uint8_t)byte;
            }
        }
        if constexpr (QT == Q8_0) {
#pragma unroll
            for (int j = 16; j < 32; ++j) {
                const uint32_t byte = (hw[1 + (j >> 1)] >> (8 * (j & 1))) & 0xFFu;
                w[j] = d * (float)(int)(int8_t)(uint8_t)byte;
            }
        }
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            if (t >= T) break;
            const f4_t *x = reinterpret_cast<const f4_t *>(X + (size_t)t * k + 32 * b);
            float s = acc[t];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const f4_t v = x[q];
                s = fmaf(w[4 * q + 0], v[0], s);
                s = fmaf(w[4 * q + 1], v[1], s);
                s = fmaf(w[4 * q + 2], v[2], s);
                s = fmaf(w[4 * q + 3], v[3], s);
            }
            acc[t] = s;
        }
    }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

template <int QT, int EPI>
__global__ __launch_bounds__(256) void gemv_kernel(const uint8_t *__restrict__ W,
                                                   const float *__restrict__ X,
                                                   float *__restrict__ Y, int n, int k, int T) {
    constexpr int TT = GEMV_MAX_T;
    const int lane = threadIdx.x & 63;
    const int o = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (o >= n) return;
    const size_t row_bytes = (size_t)(k >> 5) * BlockTraits<QT>::BYTES;
    float acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = 0.f;
    gemv_row_accumulate<QT, TT>(W + (size_t)o * row_bytes, X, k, T, lane, acc);
    float accu[TT];
    if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int t = 0; t < TT; ++t) accu[t] = 0.f;
        gemv_row_accumulate<QT, TT>(W + (size_t)(n + o) * row_bytes, X, k, T, lane, accu);
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        if (t >= T) break;
        const float g = wave_sum(acc[t]);
        float v = g;
        if constexpr (EPI == EPI_SWIGLU) v = silu_f32(g) * wave_sum(accu[t]);
        if (lane == 0) {
            float *y = Y + (size_t)t * n + o;
            if constexpr (EPI == EPI_RESIDUAL)
                *y = *y + v;
            else
                *y = v;
        }
    }
}

template <int QT, int EPI>
static hipError_t launch_gemv_typed(const GemmArgs &a, hipStream_t s) {
    const dim3 grid((a.n + 3) / 4);
    hipLaunchKernelGGL((gemv_kernel<QT, EPI>), grid, dim3(256), 0, s, a.W, a.X, a.Y, a.n, a.k, a.T);
    return hipGetLastError();
}

template <int QT>
static hipError_t launch_gemv_q(const GemmArgs &a, hipStream_t s) {
    switch (a.epilogue) {
    case EPI_PLAIN: return launch_gemv_typed<QT, EPI_PLAIN>(a, s);
    case EPI_RESIDUAL: return launch_gemv_typed<QT, EPI_RESIDUAL>(a, s);
    default: return launch_gemv_typed<QT, EPI_SWIGLU>(a, s);
    }
}

hipError_t launch_gemv(const GemmArgs &a, hipStream_t s) {
    return a.qtype == Q4_0 ? launch_gemv_q<Q4_0>(a, s) : launch_gemv_q<Q8_0>(a, s);
}

}  // namespace pf
