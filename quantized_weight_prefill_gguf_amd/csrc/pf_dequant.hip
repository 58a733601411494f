// Bit-exact block decode to f32 (the f32 leg's weights) and to binary16 (the f16
// leg's weights). It stands where the page "aprender-serve 0.70.2 -
// src/cuda/executor/gdn_prefill_ops.rs" (`qwen35_dequant_f32`, `Q8_0DequantKernel`)
// decodes a weight into an f32 scratch; here it is not on the GEMM path. It runs
// the very decode helpers the GEMM kernels use in registers (pf_device.h), so a
// bit-exact check of its output is a check of the GEMMs' weight decode.
//
// One thread decodes one 32-weight block: 9 (Q4_0) or 17 (Q8_0) 16-bit loads,
// since blocks are only 2-byte aligned, and 32 outputs as 16-byte stores.
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
    uint32_t hw[HW];
#pragma unroll
    for (int i = 0; i < HW; ++i) hw[i] = src[i];
    // qs word i = qs bytes 4i .. 4i+3 (block bytes 2+4i .. 5+4i).
    constexpr int NWORDS = QT == Q4_0 ? 4 : 8;
    uint32_t qw[NWORDS];
#pragma unroll
    for (int i = 0; i < NWORDS; ++i) qw[i] = hw[1 + 2 * i] | (hw[2 + 2 * i] << 16);

    if constexpr (!F16) {
        const float d = fp16_bits_to_f32(hw[0]);
        float v[32];
#pragma unroll
        for (int i = 0; i < NWORDS; ++i) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if constexpr (QT == Q4_0) {
                    v[4 * i + s] = q4_nibble_f32(qw[i], 8 * s, d);           // low nibble
                    v[16 + 4 * i + s] = q4_nibble_f32(qw[i], 8 * s + 4, d);  // high nibble
                } else {
                    v[4 * i + s] = q8_byte_f32(qw[i], s, d);
                }
            }
        }
        f4_t *o = reinterpret_cast<f4_t *>(static_cast<float *>(out) + (size_t)b * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = f4_t{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
    } else {
        const h2_t d2 = as_h2(hw[0] | (hw[0] << 16));
        uint16_t h[32];
#pragma unroll
        for (int i = 0; i < NWORDS; ++i) {
            if constexpr (QT == Q4_0) {
                // halves in k order 4i, 4i+2, 4i+1, 4i+3, 16+4i, 16+4i+2, 16+4i+1, 16+4i+3
                uint32_t p[4];
                q4_word_to_h8(qw[i], d2, p);
                h[4 * i + 0] = p[0] & 0xFFFFu;
                h[4 * i + 2] = p[0] >> 16;
                h[4 * i + 1] = p[1] & 0xFFFFu;
                h[4 * i + 3] = p[1] >> 16;
                h[16 + 4 * i + 0] = p[2] & 0xFFFFu;
                h[16 + 4 * i + 2] = p[2] >> 16;
                h[16 + 4 * i + 1] = p[3] & 0xFFFFu;
                h[16 + 4 * i + 3] = p[3] >> 16;
            } else {
                uint32_t p[2];
                q8_word_to_h4(qw[i], d2, p);
                h[4 * i + 0] = p[0] & 0xFFFFu;
                h[4 * i + 1] = p[0] >> 16;
                h[4 * i + 2] = p[1] & 0xFFFFu;
                h[4 * i + 3] = p[1] >> 16;
            }
        }
        uint4 *o = reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out) + (size_t)b * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = make_uint4(h[8 * i] | ((uint32_t)h[8 * i + 1] << 16),
                              h[8 * i + 2] | ((uint32_t)h[8 * i + 3] << 16),
                              h[8 * i + 4] | ((uint32_t)h[8 * i + 5] << 16),
                              h[8 * i + 6] | ((uint32_t)h[8 * i + 7] << 16));
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
