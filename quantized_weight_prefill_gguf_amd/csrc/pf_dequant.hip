// Bit-exact block decode to f32 (the f32 leg's weights) and to binary16 (the f16
// leg's weights). It stands where the page "aprender-serve 0.70.2 -
// src/cuda/executor/gdn_prefill_ops.rs" (`qwen35_dequant_f32`, `Q8_0DequantKernel`)
// decodes a weight into an f32 scratch; here it exists to check the in-register
// decode of the GEMM kernels bit for bit, not on the GEMM path.
//
// One thread decodes one 32-weight block: 9 (Q4_0) or 17 (Q8_0) 16-bit loads,
// since blocks are only 2-byte aligned, and 32 outputs as 8 (f32) or 4 (f16)
// 16-byte stores.
#include "pf_device.h"
#include "pf_internal.h"

namespace pf {

template <int QT, bool F16>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ W,
                                                      int nblocks, void *__restrict__ out) {
    const int b = blockIdx.x * 256 + threadIdx.x;
    if (b >= nblocks) return;
    constexpr int HW = BlockTraits<QT>::HALFWORDS;
    const uint16_t *src = reinterpret_cast<const uint16_t *>(W + (size_t)b * BlockTraits<QT>::BYTES);
    uint16_t hw[HW];
#pragma unroll
    for (int i = 0; i < HW; ++i) hw[i] = src[i];
    const float d = fp16_bits_to_f32(hw[0]);
    float v[32];
    if constexpr (QT == Q4_0) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t byte = (hw[1 + (j >> 1)] >> (8 * (j & 1))) & 0xFFu;
            v[j] = d * (float)((int)(byte & 15u) - 8);
            v[j + 16] = d * (float)((int)(byte >> 4) - 8);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const uint32_t byte = (hw[1 + (j >> 1)] >> (8 * (j & 1))) & 0xFFu;
            v[j] = d * (float)(int)(int8_t)(uint8_t)byte;
        }
    }
    if constexpr (!F16) {
        f4_t *o = reinterpret_cast<f4_t *>(static_cast<float *>(out) + (size_t)b * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = f4_t{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
    } else {
        uint4 *o = reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out) + (size_t)b * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t p[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // RNE rounding of the exact f32 value
                const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)v[8 * i + 2 * j]);
                const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)v[8 * i + 2 * j + 1]);
                p[j] = lo | (hi << 16);
            }
            o[i] = make_uint4(p[0], p[1], p[2], p[3]);
        }
    }
}

template <bool F16>
static hipError_t launch_dequant(int qtype, const uint8_t *W, int rows, int k, void *out,
                                 hipStream_t s) {
    const int nblocks = rows * (k / 32);
    const dim3 grid((nblocks + 255) / 256);
    if (qtype == Q4_0)
        hipLaunchKernelGGL((dequant_kernel<Q4_0, F16>), grid, dim3(256), 0, s, W, nblocks, out);
    else
        hipLaunchKernelGGL((dequant_kernel<Q8_0, F16>), grid, dim3(256), 0, s, W, nblocks, out);
    return hipGetLastError();
}

hipError_t launch_dequant_f32(int qtype, const uint8_t *W, int rows, int k, float *out,
                              hipStream_t s) {
    return launch_dequant<false>(qtype, W, rows, k, out, s);
}

hipError_t launch_dequant_f16(int qtype, const uint8_t *W, int rows, int k, uint16_t *out,
                              hipStream_t s) {
    return launch_dequant<true>(qtype, W, rows, k, out, s);
}

}  // namespace pf
