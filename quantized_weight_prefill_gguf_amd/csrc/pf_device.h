// Device-side helpers shared by the gfx950 kernels: block traits, fp16 bit
// handling, in-register block decode and the epilogue store.
//
// Block formats (GGUF): Q4_0 = 18 bytes (fp16 scale d little-endian, then 16
// nibble bytes; weight j < 16 is the low nibble of byte j, weight j >= 16 the
// high nibble of byte j-16; value d*(q-8)). Q8_0 = 34 bytes (fp16 d, then 32
// int8 q; value d*q). Weight rows are stored block after block (AoS), as the page
// "oxibonsai-kernels 0.1.4 - src/gpu_backend/cuda_q_std_prefill.rs" (module doc,
// "Weight layout") keeps them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pf {

enum { Q4_0 = 0, Q8_0 = 1 };
enum { EPI_PLAIN = 0, EPI_RESIDUAL = 1, EPI_SWIGLU = 2 };
constexpr int GEMV_MAX_T = 8;  // largest T the GEMV handles

template <int QT> struct BlockTraits;
template <> struct BlockTraits<Q4_0> {
    static constexpr int BYTES = 18;
    static constexpr int HALFWORDS = 9;  // the block is 2-byte aligned: 9 u16
};
template <> struct BlockTraits<Q8_0> {
    static constexpr int BYTES = 34;
    static constexpr int HALFWORDS = 17;
};

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float fp16_bits_to_f32(uint32_t bits16) {
    // binary16 -> f32 is exact.
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

__device__ __forceinline__ h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }
__device__ __forceinline__ uint32_t h2_bits(h2_t v) { return __builtin_bit_cast(uint32_t, v); }

// ---------------------------------------------------------------------------
// f16-leg weight decode: 8 weights from one 32-bit word of block bytes.
//
// 0x6400 | v (v < 1024) is the binary16 value 1024 + v exactly. Subtracting
// 1024 + offset gives the small integer exactly, and one f16 multiply by the
// scale rounds d * integer once, to nearest even: the same value as rounding the
// exact f32 product.
// ---------------------------------------------------------------------------

// Q4_0: w holds qs bytes 4g .. 4g+3 of a block. Returns 4 packed half2 whose 8
// halves are the weights at k = 4g, 4g+2, 4g+1, 4g+3, 16+4g, 16+4g+2, 16+4g+1,
// 16+4g+3 (low nibbles, then high nibbles). The activation side stores X in this
// same order, so the k order inside a block never matters to the dot product.
__device__ __forceinline__ void q4_word_to_h8(uint32_t w, h2_t d2, uint32_t out[4]) {
    const h2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
    uint32_t r0 = (w & 0x000F000Fu) | 0x64006400u;
    uint32_t r1 = ((w >> 8) & 0x000F000Fu) | 0x64006400u;
    uint32_t r2 = ((w >> 4) & 0x000F000Fu) | 0x64006400u;
    uint32_t r3 = ((w >> 12) & 0x000F000Fu) | 0x64006400u;
    out[0] = h2_bits((as_h2(r0) - off) * d2);
    out[1] = h2_bits((as_h2(r1) - off) * d2);
    out[2] = h2_bits((as_h2(r2) - off) * d2);
    out[3] = h2_bits((as_h2(r3) - off) * d2);
}

// Q8_0: w holds 4 int8 q (bytes 4i .. 4i+3). Returns 2 packed half2 = d*q for the
// 4 bytes in order. x ^ 0x80 turns int8 q into the unsigned byte q + 128.
__device__ __forceinline__ void q8_word_to_h4(uint32_t w, h2_t d2, uint32_t out[2]) {
    const h2_t off = {(_Float16)1152.0f, (_Float16)1152.0f};
    uint32_t x = w ^ 0x80808080u;
    uint32_t r0 = (x & 0xFFu) | ((x & 0xFF00u) << 8) | 0x64006400u;
    uint32_t r1 = ((x >> 16) & 0xFFu) | ((x >> 8) & 0xFF0000u) | 0x64006400u;
    out[0] = h2_bits((as_h2(r0) - off) * d2);
    out[1] = h2_bits((as_h2(r1) - off) * d2);
}

// ---------------------------------------------------------------------------
// f32-leg weight decode: exact d * (q - 8) and d * q.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float q4_nibble_f32(uint32_t w, int shift, float d) {
    return d * (float)((int)((w >> shift) & 15u) - 8);
}
__device__ __forceinline__ float q8_byte_f32(uint32_t w, int byte, float d) {
    return d * (float)(int)(int8_t)(uint8_t)(w >> (8 * byte));
}

// ---------------------------------------------------------------------------
// Epilogue helpers. silu(g) = g / (1 + e^-g), evaluated in f32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + expf(-g)); }

}  // namespace pf
