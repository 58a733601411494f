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

// v_perm_b32 byte selection: result byte i = byte sel[i] of {src0 (bytes 4-7),
// src1 (bytes 0-3)}. With src0 = 0x64646464 this builds binary16 patterns
// 0x64vv = 1024 + v from chosen bytes v of src1.
constexpr uint32_t MAGIC_BYTES = 0x64646464u;
constexpr uint32_t SEL_B02 = 0x04020400u;  // (src1.b0, 0x64, src1.b2, 0x64)
constexpr uint32_t SEL_B13 = 0x04030401u;  // (src1.b1, 0x64, src1.b3, 0x64)
constexpr uint32_t SEL_B01 = 0x04010400u;  // (src1.b0, 0x64, src1.b1, 0x64)
constexpr uint32_t SEL_B23 = 0x04030402u;  // (src1.b2, 0x64, src1.b3, 0x64)

__device__ __forceinline__ uint32_t magic_pair(uint32_t bytes, uint32_t sel) {
    return __builtin_amdgcn_perm(MAGIC_BYTES, bytes, sel);
}

// Q4_0: w holds 4 qs bytes b0..b3 (weights j, j+1, j+2, j+3 in their low nibbles
// and j+16 .. j+19 in their high nibbles). Outputs, each a packed half2 of
// RNE(d * (q - 8)): lo02 = low nibbles of b0, b2; lo13 = low nibbles of b1, b3;
// hi02, hi13 likewise for the high nibbles.
__device__ __forceinline__ void q4_word_decode(uint32_t w, h2_t d2, uint32_t &lo02,
                                               uint32_t &lo13, uint32_t &hi02,
                                               uint32_t &hi13) {
    const h2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
    const uint32_t lo = w & 0x0F0F0F0Fu;
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
    lo02 = h2_bits((as_h2(magic_pair(lo, SEL_B02)) - off) * d2);
    lo13 = h2_bits((as_h2(magic_pair(lo, SEL_B13)) - off) * d2);
    hi02 = h2_bits((as_h2(magic_pair(hi, SEL_B02)) - off) * d2);
    hi13 = h2_bits((as_h2(magic_pair(hi, SEL_B13)) - off) * d2);
}

// Q4_0, 16x16x32 fragment form: the 8 halves of out[0..3] are the weights at
// k = 4g, 4g+2, 4g+1, 4g+3, 16+4g, 16+4g+2, 16+4g+1, 16+4g+3 when w holds qs
// bytes 4g .. 4g+3.
__device__ __forceinline__ void q4_word_to_h8(uint32_t w, h2_t d2, uint32_t out[4]) {
    q4_word_decode(w, d2, out[0], out[1], out[2], out[3]);
}

// Q8_0: w holds 4 int8 q (bytes 4i .. 4i+3). Returns 2 packed half2 = RNE(d*q)
// for the 4 bytes in order. x ^ 0x80 turns int8 q into the unsigned byte q + 128.
__device__ __forceinline__ void q8_word_to_h4(uint32_t w, h2_t d2, uint32_t out[2]) {
    const h2_t off = {(_Float16)1152.0f, (_Float16)1152.0f};
    const uint32_t x = w ^ 0x80808080u;
    out[0] = h2_bits((as_h2(magic_pair(x, SEL_B01)) - off) * d2);
    out[1] = h2_bits((as_h2(magic_pair(x, SEL_B23)) - off) * d2);
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

// IQ4_XS's grid as int8 bytes, code order, little-endian in four words: byte c of the
// 16 is the value of code c.
constexpr uint32_t IQ4_GRID_B0 = 0x81u | (0x98u << 8) | (0xADu << 16) | (0xBFu << 24);  // -127 -104 -83 -65
constexpr uint32_t IQ4_GRID_B1 = 0xCFu | (0xDDu << 8) | (0xEAu << 16) | (0xF6u << 24);  // -49 -35 -22 -10
constexpr uint32_t IQ4_GRID_B2 = 0x01u | (0x0Du << 8) | (0x19u << 16) | (0x26u << 24);  // 1 13 25 38
constexpr uint32_t IQ4_GRID_B3 = 0x35u | (0x45u << 8) | (0x59u << 16) | (0x71u << 24);  // 53 69 89 113

// Four codes (one per byte, each 0..15) -> their grid bytes. v_perm_b32
// picks bytes 0..3 of its second source and 4..7 of its first: the low three bits
// of a code select within codes 0..7 or 8..15, bit 3 chooses between the two picks.
__device__ __forceinline__ uint32_t iq4_grid_bytes(uint32_t codes) {
    const uint32_t sel = codes & 0x07070707u;
    const uint32_t lo = __builtin_amdgcn_perm(IQ4_GRID_B1, IQ4_GRID_B0, sel);
    const uint32_t hi = __builtin_amdgcn_perm(IQ4_GRID_B3, IQ4_GRID_B2, sel);
    const uint32_t m = ((codes >> 3) & 0x01010101u) * 0xFFu;
    return (lo & ~m) | (hi & m);
}

// Orders one wave's LDS accesses before the call against those after it, for
// communication between the lanes of that wave through LDS.
//  - The fences keep the compiler from moving accesses across (without them, a
//    store whose address no load of the same thread can alias may be sunk past
//    another lane's read of it).
//  - The wait (lgkmcnt = 0) makes the wave's LDS operations complete before any
//    later one issues. The compiler emits nothing for wavefront-scope fences, on
//    the assumption that a wave's LDS operations are performed in order; on gfx950
//    that did not hold for the SwiGLU epilogue's exchange (16-byte stores of
//    accumulator registers, then 16-byte loads of other lanes' values issued right
//    behind them): without the wait, whole groups of loads intermittently returned
//    values other than the ones just stored.
constexpr int WAITCNT_LGKM0 = 0xC07F;  // s_waitcnt lgkmcnt(0), vmcnt and expcnt not waited
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_waitcnt(WAITCNT_LGKM0);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// Epilogue helpers. silu(g) = g / (1 + e^-g), evaluated in f32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + expf(-g)); }

// The same with the hardware exp2 and reciprocal (a few ulp; for the f16 leg,
// whose tolerance is far above that). g -> -inf gives -0, as the definition does.
__device__ __forceinline__ float silu_fast(float g) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

}  // namespace pf
