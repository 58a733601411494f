// The further weight types of the f32 and f16 legs: F16, Q4_K, Q5_K, Q6_K and IQ4_XS,
// the types the page "aprender-serve 0.70.2 - src/cuda/executor/gdn_prefill_ops.rs"
// dequantizes besides Q8_0 (`qwen35_dequant_f32`: F16 over 32-element groups, the K
// types and IQ4_XS over 256-element super-blocks; `qwen35_fp16_weight`: the f16 leg's
// weight is that f32 value rounded to binary16). The pages print no layout; these are
// GGUF's:
//
//  F16   64 bytes per 32 weights: little-endian binary16 values.
//  Q4_K  144 bytes per 256: fp16 d, fp16 dmin, 12 bytes of 6-bit scales s_j and mins
//        m_j (8 sub-blocks of 32), 128 bytes of nibbles. Element e: group p = e / 64,
//        l = e % 32, low nibble of qs[32p + l] for e % 64 < 32, else its high nibble;
//        value (d s_j) q - dmin m_j, j = e / 32.
//  Q5_K  176 bytes: as Q4_K, with 32 bytes qh between the scales and the nibbles; bit
//        j of qh[l] adds 16 to element 32 j + l.
//  Q6_K  210 bytes: ql[128], qh[64], 16 int8 scales, fp16 d. Element e: half h = e /
//        128, quarter c = (e % 128) / 32, l = e % 32; low 4 bits from ql[64h + l + 32
//        (c % 2)] (low nibble for c < 2, high for c >= 2), top 2 from bits 2c, 2c+1 of
//        qh[32h + l]; value (d sc[8h + l/16 + 2c]) (q - 32).
//  IQ4_XS 136 bytes per 256: fp16 d, uint16 scales_h, 4 bytes scales_l, 128 bytes of
//        codes. Sub-block b = e / 32 has the 6-bit scale ls whose low 4 bits are
//        nibble b % 2 of scales_l[b / 2] and whose top 2 are bits 2b, 2b+1 of
//        scales_h; element e, l = e % 32, takes the low (l < 16) or high nibble of
//        qs[16 b + l % 16] as its code; value (d (ls - 32)) grid[code], with GGUF's
//        16-value grid (the IQ4_NL one).
//
// The decode is exact in f32 as these definitions give it: d s_j, dmin m_j and
// (d s_j) q are exact, so the Q4_K / Q5_K value has the one rounding of the
// subtraction (an FMA gives the same bits); Q6_K's d sc is exact and the product with
// q - 32 rounds once; IQ4_XS's d (ls - 32) and its product with a grid value (11 + 6 +
// 7 significant bits) are exact. The f16 leg rounds that f32 value to binary16 (RNE).
//
// Kernels (no workspace; nothing splits, one writer per output):
//  - xq_dequant_kernel: one 16-weight run per thread, f32 or binary16 out.
//  - xq_gemv_kernel (T <= 8): a wave per output (or gate/up pair), lanes stride over
//    16-weight runs, f32 FMAs, a butterfly over the lanes.
//  - xq_gemm_kernel: 64 token rows x 128 weight rows per workgroup of 4 waves; per
//    32-k step the workgroup decodes its 128 x 32 weights into LDS (binary16 or f32
//    as the leg), stages X likewise, and each wave runs 32 x 64 outputs on the
//    matrix cores (v_mfma_f32_32x32x16_f16, or v_mfma_f32_32x32x2f32 on the f32 leg).
//    The accumulators go through LDS to the epilogue, so each store is a whole row.
#include <type_traits>

#include "pf_device.h"
#include "pf_internal.h"

namespace pf {

namespace {

template <int QT> struct XqTraits;
template <> struct XqTraits<XQ_F16> {
    static constexpr int ELEMS = 32, BYTES = 64;
};
template <> struct XqTraits<XQ_Q4_K> {
    static constexpr int ELEMS = 256, BYTES = 144;
};
template <> struct XqTraits<XQ_Q5_K> {
    static constexpr int ELEMS = 256, BYTES = 176;
};
template <> struct XqTraits<XQ_Q6_K> {
    static constexpr int ELEMS = 256, BYTES = 210;
};
template <> struct XqTraits<XQ_IQ4_XS> {
    static constexpr int ELEMS = 256, BYTES = 136;
};

__device__ __forceinline__ uint32_t byte_of(const u4_t &v, int i) {
    return (v[i >> 2] >> (8 * (i & 3))) & 0xFFu;
}

// The 6-bit scale and min of sub-block j (0..7) from the 12 scale bytes held in the
// words w1..w3 of a Q4_K / Q5_K header (header bytes 4..15).
__device__ __forceinline__ void k_scale_min(const u4_t &hdr, int j, uint32_t &s, uint32_t &m) {
    auto sb = [&](int i) { return byte_of(hdr, 4 + i); };  // scale byte i (0..11)
    if (j < 4) {
        s = sb(j) & 63u;
        m = sb(j + 4) & 63u;
    } else {
        s = (sb(j + 4) & 15u) | ((sb(j - 4) >> 6) << 4);
        m = (sb(j + 4) >> 4) | ((sb(j) >> 6) << 4);
    }
}

// The bytes that weights e0 .. e0 + 15 (e0 % 16 == 0) of a block decode from, loaded
// by load_raw16 and turned into exact f32 by decode_raw16, so that a caller can keep
// the loads in flight across other work.
template <int QT> struct Raw16;
template <> struct Raw16<XQ_F16> {
    u4_t a, b;             // the 16 binary16 values
};
template <> struct Raw16<XQ_Q4_K> {
    u4_t hdr, qs;          // d, dmin and the 12 scale bytes; the 16 code bytes
};
template <> struct Raw16<XQ_Q5_K> {
    u4_t hdr, qs, qh;      // and the 16 qh bytes of the same l
};
template <> struct Raw16<XQ_Q6_K> {
    // 210-byte blocks are only 2-byte aligned: the 16 ql and 16 qh bytes are read as
    // five dwords each from the dword boundary at or below them, and `sh` (0 or 2) is
    // the bytes to skip.
    u4_t ql, qh;
    uint32_t ql4, qh4, sh;
    uint32_t sc, d;        // the halfword holding the scale byte; d
};
typedef uint32_t u4a4_t __attribute__((ext_vector_type(4), aligned(4)));  // 4-byte aligned
template <> struct Raw16<XQ_IQ4_XS> {
    u2_t hdr;              // d, scales_h, scales_l (136-byte blocks are 8-byte aligned)
    u2_t qa, qb;           // the 16 code bytes of the sub-block
};

template <int QT>
__device__ __forceinline__ void load_raw16(const uint8_t *__restrict__ blk, int e0, Raw16<QT> &r) {
    if constexpr (QT == XQ_F16) {
        r.a = *reinterpret_cast<const u4_t *>(blk + 2 * e0);
        r.b = *reinterpret_cast<const u4_t *>(blk + 2 * e0 + 16);
    } else if constexpr (QT == XQ_Q4_K || QT == XQ_Q5_K) {
        // 144 and 176 are multiples of 16, and so is every offset read here: the
        // block's rows start 16-byte aligned (k % 256 == 0, W 16-byte aligned).
        const int p = e0 >> 6, l0 = e0 & 31;
        constexpr int QS = QT == XQ_Q5_K ? 48 : 16;
        r.hdr = *reinterpret_cast<const u4_t *>(blk);
        r.qs = *reinterpret_cast<const u4_t *>(blk + QS + 32 * p + l0);
        if constexpr (QT == XQ_Q5_K) r.qh = *reinterpret_cast<const u4_t *>(blk + 16 + l0);
    } else if constexpr (QT == XQ_IQ4_XS) {
        const int b = e0 >> 5;
        r.hdr = *reinterpret_cast<const u2_t *>(blk);
        r.qa = *reinterpret_cast<const u2_t *>(blk + 8 + 16 * b);
        r.qb = *reinterpret_cast<const u2_t *>(blk + 16 + 16 * b);
    } else {
        const int h = e0 >> 7, c = (e0 & 127) >> 5, l0 = e0 & 31;
        // ql and qh offsets are even, so blk + offset is 0 or 2 mod 4 as blk is; the
        // extra dword ends at block byte 132 (ql) or 196 (qh), inside the block.
        const uint32_t sh = (uint32_t)(reinterpret_cast<uintptr_t>(blk) & 3);
        const uint32_t *ql = reinterpret_cast<const uint32_t *>(blk + 64 * h + l0 + 32 * (c & 1) - sh);
        const uint32_t *qh = reinterpret_cast<const uint32_t *>(blk + 128 + 32 * h + l0 - sh);
        const u4a4_t a = *reinterpret_cast<const u4a4_t *>(ql), b = *reinterpret_cast<const u4a4_t *>(qh);
        r.ql = u4_t{a[0], a[1], a[2], a[3]};
        r.qh = u4_t{b[0], b[1], b[2], b[3]};
        r.ql4 = ql[4];
        r.qh4 = qh[4];
        r.sh = sh;
        const int si = 192 + 8 * h + (l0 >> 4) + 2 * c;
        r.sc = *reinterpret_cast<const uint16_t *>(blk + (si & ~1));
        r.d = *reinterpret_cast<const uint16_t *>(blk + 208);
    }
}

// Weights e0 .. e0 + 15 from their bytes, exact f32. Each value is then made opaque
// to the optimizer: the f16 leg's weight is this f32 value rounded to binary16, and
// without that the compiler fuses the last multiply-add with the conversion
// (v_fma_mix*_f16: one rounding straight to binary16), which differs from rounding
// the f32 value where the two roundings meet a tie.
template <int QT>
__device__ __forceinline__ void decode_raw16(const Raw16<QT> &r, int e0, float (&w)[16]) {
    if constexpr (QT == XQ_F16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[2 * i] = fp16_bits_to_f32(r.a[i] & 0xFFFFu);
            w[2 * i + 1] = fp16_bits_to_f32(r.a[i] >> 16);
            w[8 + 2 * i] = fp16_bits_to_f32(r.b[i] & 0xFFFFu);
            w[8 + 2 * i + 1] = fp16_bits_to_f32(r.b[i] >> 16);
        }
    } else if constexpr (QT == XQ_Q4_K || QT == XQ_Q5_K) {
        const int j = e0 >> 5;
        uint32_t s, m;
        k_scale_min(r.hdr, j, s, m);
        const float a = fp16_bits_to_f32(r.hdr[0] & 0xFFFFu) * (float)s;
        const float b = fp16_bits_to_f32(r.hdr[0] >> 16) * (float)m;
        // the codes of four weights a word (their nibble half, and for Q5_K bit j of qh
        // as bit 4), each then one byte conversion; (d s) q is exact, so the FMA rounds
        // once, as the subtraction does
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
            uint32_t q4 = (r.qs[wd] >> (4 * (j & 1))) & 0x0F0F0F0Fu;
            if constexpr (QT == XQ_Q5_K) q4 |= ((r.qh[wd] >> j) & 0x01010101u) << 4;
            asm("" : "+v"(q4));
#pragma unroll
            for (int c = 0; c < 4; ++c) w[4 * wd + c] = fmaf(a, (float)((q4 >> (8 * c)) & 0xFFu), -b);
        }
    } else if constexpr (QT == XQ_IQ4_XS) {
        const int b = e0 >> 5;
        const bool upper = (e0 & 16) != 0;
        const uint32_t sl = (r.hdr[1] >> (8 * (b >> 1))) & 0xFFu;
        const uint32_t ls = ((sl >> (4 * (b & 1))) & 15u) | (((r.hdr[0] >> (16 + 2 * b)) & 3u) << 4);
        const float dl = fp16_bits_to_f32(r.hdr[0] & 0xFFFFu) * (float)((int)ls - 32);
        const uint32_t q[4] = {r.qa[0], r.qa[1], r.qb[0], r.qb[1]};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t codes = upper ? (q[j] >> 4) & 0x0F0F0F0Fu : q[j] & 0x0F0F0F0Fu;
            const uint32_t g = iq4_grid_bytes(codes);
            // the grid value (a signed byte, converted exactly), then one product:
            // a zero scale keeps the sign the definition gives (dl * value)
#pragma unroll
            for (int c = 0; c < 4; ++c) w[4 * j + c] = dl * (float)(int8_t)(uint8_t)(g >> (8 * c));
        }
    } else {
        const int h = e0 >> 7, c = (e0 & 127) >> 5, l0 = e0 & 31;
        const int si = 192 + 8 * h + (l0 >> 4) + 2 * c;
        const int sc = (int)(int8_t)(uint8_t)(r.sc >> (8 * (si & 1)));
        const float ds = fp16_bits_to_f32(r.d) * (float)sc;
        const uint32_t qlw[5] = {r.ql[0], r.ql[1], r.ql[2], r.ql[3], r.ql4};
        const uint32_t qhw[5] = {r.qh[0], r.qh[1], r.qh[2], r.qh[3], r.qh4};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lw = __builtin_amdgcn_alignbyte(qlw[i + 1], qlw[i], r.sh);
            const uint32_t hw = __builtin_amdgcn_alignbyte(qhw[i + 1], qhw[i], r.sh);
            // four 6-bit codes a word, each then one byte conversion; ds (q - 32) as the
            // definition writes it (q - 32 is exact; an FMA with -32 ds would turn the
            // -0 of a negative ds at q = 32 into +0)
            uint32_t q4 = ((lw >> (4 * (c >> 1))) & 0x0F0F0F0Fu) | (((hw >> (2 * c)) & 0x03030303u) << 4);
            asm("" : "+v"(q4));
#pragma unroll
            for (int b = 0; b < 4; ++b) w[4 * i + b] = ds * ((float)((q4 >> (8 * b)) & 0xFFu) - 32.0f);
        }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) asm("" : "+v"(w[i]));
}

template <int QT>
__device__ __forceinline__ void decode16(const uint8_t *__restrict__ blk, int e0, float (&w)[16]) {
    Raw16<QT> r;
    load_raw16<QT>(blk, e0, r);
    decode_raw16<QT>(r, e0, w);
}

// Weights e .. e + 15 of a row (e % 16 == 0): the block holding them and the offset.
template <int QT>
__device__ __forceinline__ void decode_row16(const uint8_t *__restrict__ row, int e, float (&w)[16]) {
    using TR = XqTraits<QT>;
    decode16<QT>(row + (size_t)(e / TR::ELEMS) * TR::BYTES, e % TR::ELEMS, w);
}

// out[r][k]: f32 (F16OUT false) or binary16 bits; one 16-weight run per thread.
template <int QT, bool F16OUT>
__global__ __launch_bounds__(256) void xq_dequant_kernel(const uint8_t *__restrict__ W, int rows, int k,
                                                         void *__restrict__ out) {
    using TR = XqTraits<QT>;
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    const long runs = (long)rows * (k / 16);
    if (i >= runs) return;
    const int r = (int)(i / (k / 16)), e = (int)(i % (k / 16)) * 16;
    float w[16];
    decode_row16<QT>(W + (size_t)r * (k / TR::ELEMS) * TR::BYTES, e, w);
    if constexpr (F16OUT) {
        uint32_t p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = h2_bits(h2_t{(_Float16)w[2 * j], (_Float16)w[2 * j + 1]});
        u4_t *dst = reinterpret_cast<u4_t *>(static_cast<uint16_t *>(out) + (size_t)r * k + e);
        dst[0] = u4_t{p[0], p[1], p[2], p[3]};
        dst[1] = u4_t{p[4], p[5], p[6], p[7]};
    } else {
        f4_t *dst = reinterpret_cast<f4_t *>(static_cast<float *>(out) + (size_t)r * k + e);
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[j] = f4_t{w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]};
    }
}

// GEMV, T <= 8 tokens (TT of them per launch): wave g of the grid owns R weight rows,
// outputs R g .. R g + R - 1 (PLAIN / RESIDUAL), or outputs (R / 2) g .. with their
// gate and up rows (SwiGLU), so that each x value a lane loads serves R rows. Lanes
// take 16-weight runs 64 apart; the R rows' raw bytes are all loaded before any is
// decoded. R = 4 where that still leaves at least 8 waves per CU, else 1 (2 for
// SwiGLU): memory latency wants the waves more than x wants the reuse.
// XL: x staged once per workgroup of WV waves in LDS (dynamic, xtok float4 per token),
// lane-transposed: float4 i of run `lane + 64 it` at (4 it + i) 64 + lane, so that a
// wave's read of one i is 1 KB of consecutive bytes. Each run's 64 bytes of x per token
// would otherwise come from L2 for every row: four times the weight bytes of Q6_K.
template <int QT, int EPI, int TT, int R, bool XL = false, int WV = 4>
__global__ __launch_bounds__(64 * WV) void xq_gemv_kernel(const uint8_t *__restrict__ W,
                                                          const float *__restrict__ X, float *__restrict__ Y,
                                                          int n, int ldy, int k, int xtok) {
    using TR = XqTraits<QT>;
    constexpr int OUTW = EPI == EPI_SWIGLU ? R / 2 : R;
    const int lane = threadIdx.x & 63;
    const int g = blockIdx.x * WV + (threadIdx.x >> 6);
    extern __shared__ __attribute__((aligned(16))) uint8_t xsm[];
    f4_t *xs = reinterpret_cast<f4_t *>(xsm);
    if constexpr (XL) {
        // every thread of the workgroup stages, before any wave leaves
        const int q4 = k / 4;
        for (int j = threadIdx.x; j < TT * q4; j += 64 * WV) {
            const int t = j / q4, jj = j - t * q4;
            int slot;
            if constexpr (QT == XQ_Q6_K) {
                // the paired loop's order: unit u (32 weights: 16 at ea, 16 at ea + 64)
                // reads float4 i of run `hi` (0: ea, 1: ea + 64) from slot
                // ((u / 64 * 2 + hi) * 4 + i) * 64 + u % 64
                const int w = (4 * jj) & 255;
                const int u = (jj >> 6) * 8 + (w >> 7) * 4 + ((w >> 5) & 1) * 2 + ((w >> 4) & 1);
                slot = (((u >> 6) * 2 + ((w >> 6) & 1)) * 4 + ((w >> 2) & 3)) * 64 + (u & 63);
            } else {
                const int run = jj >> 2, it = run >> 6;
                slot = (4 * it + (jj & 3)) * 64 + (run & 63);
            }
            xs[t * xtok + slot] = *reinterpret_cast<const f4_t *>(X + (size_t)t * k + 4 * jj);
        }
        __syncthreads();
    } else {
        (void)xs;
        (void)xtok;
    }
    if (g * OUTW >= n) return;  // whole waves leave
    const size_t row_bytes = (size_t)(k / TR::ELEMS) * TR::BYTES;
    const uint8_t *rows[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        int wr;
        if constexpr (EPI == EPI_SWIGLU)
            wr = (r < OUTW ? 0 : n) + min(g * OUTW + r % OUTW, n - 1);
        else
            wr = min(g * OUTW + r, n - 1);
        rows[r] = W + (size_t)wr * row_bytes;
    }
    float acc[R][TT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[r][t] = 0.f;
    if constexpr (QT == XQ_Q6_K) {
        // Q6_K: sub-blocks c and c + 2 of a half take the low and high nibbles of the same
        // ql bytes and other bits of the same qh bytes, so a lane takes weights l0 ..
        // l0 + 15 of both (32 weights, x read as two runs of 16): one set of ql, qh and d
        // loads, and the two scale bytes, serves both.
        for (int u = lane, it = 0; u < k / 32; u += 64, ++it) {
            const int j = u & 7;
            const int ea = (u >> 3) * 256 + (j >> 2) * 128 + ((j >> 1) & 1) * 32 + (j & 1) * 16;
            const size_t boff = (size_t)(ea / TR::ELEMS) * TR::BYTES;
            const int e0a = ea % TR::ELEMS, e0b = e0a + 64;
            Raw16<QT> ra[R];
            uint32_t scb[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                load_raw16<QT>(rows[r] + boff, e0a, ra[r]);
                const int sib = 192 + 8 * (e0b >> 7) + ((e0b & 31) >> 4) + 2 * ((e0b & 127) >> 5);
                scb[r] = *reinterpret_cast<const uint16_t *>(rows[r] + boff + (sib & ~1));
            }
            f4_t xa[TT][4], xb[TT][4];
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                if constexpr (XL) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        xa[t][i] = xs[t * xtok + ((2 * it) * 4 + i) * 64 + lane];
                        xb[t][i] = xs[t * xtok + ((2 * it + 1) * 4 + i) * 64 + lane];
                    }
                } else {
                    const f4_t *xp = reinterpret_cast<const f4_t *>(X + (size_t)t * k + ea);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        xa[t][i] = xp[i];
                        xb[t][i] = xp[16 + i];
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    Raw16<QT> rr = ra[r];
                    if (half) rr.sc = scb[r];
                    float w[16];
                    decode_raw16<QT>(rr, half ? e0b : e0a, w);
#pragma unroll
                    for (int t = 0; t < TT; ++t) {
                        float a = acc[r][t];
#pragma unroll
                        for (int i = 0; i < 16; ++i) a = fmaf(w[i], (half ? xb : xa)[t][i >> 2][i & 3], a);
                        acc[r][t] = a;
                    }
                }
            }
        }
    } else
    for (int e = 16 * lane, it = 0; e < k; e += 16 * 64, ++it) {
        Raw16<QT> raw[R];
        const size_t boff = (size_t)(e / TR::ELEMS) * TR::BYTES;
#pragma unroll
        for (int r = 0; r < R; ++r) load_raw16<QT>(rows[r] + boff, e % TR::ELEMS, raw[r]);
        f4_t xv[TT][4];
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            if constexpr (XL) {
#pragma unroll
                for (int i = 0; i < 4; ++i) xv[t][i] = xs[t * xtok + (4 * it + i) * 64 + lane];
            } else {
                const f4_t *xp = reinterpret_cast<const f4_t *>(X + (size_t)t * k + e);
#pragma unroll
                for (int i = 0; i < 4; ++i) xv[t][i] = xp[i];
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float w[16];
            decode_raw16<QT>(raw[r], e % TR::ELEMS, w);
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                float a = acc[r][t];
#pragma unroll
                for (int i = 0; i < 16; ++i) a = fmaf(w[i], xv[t][i >> 2][i & 3], a);
                acc[r][t] = a;
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int dist = 32; dist >= 1; dist >>= 1) acc[r][t] += __shfl_xor(acc[r][t], dist, 64);
    if (lane == 0) {
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int q = 0; q < OUTW; ++q) {
                const int o = g * OUTW + q;
                if (o >= n) continue;
                float *y = Y + (size_t)t * ldy + o;
                if constexpr (EPI == EPI_SWIGLU)
                    *y = silu_f32(acc[q][t]) * acc[OUTW + q][t];
                else if constexpr (EPI == EPI_RESIDUAL)
                    *y = *y + acc[q][t];
                else
                    *y = acc[q][t];
            }
    }
}

typedef float f16v_t __attribute__((ext_vector_type(16)));

// GEMM. Workgroup tile: MT token rows (128 on the f16 leg, 64 on the f32 leg) x XNW
// = 128 weight rows (SwiGLU: the 64 gate rows of 64 outputs, then their 64 up rows).
// Waves 2 x 2, each MT/2 rows x 64 weight rows (MT/64 x 2 accumulator tiles of
// 32 x 32). LEG16: binary16 operands and v_mfma_f32_32x32x16_f16; else f32 operands
// and v_mfma_f32_32x32x2f32. Per 32-k step: the next step's raw weight bytes and X
// are loaded first, this step's MFMAs run while they arrive, then the next step is
// decoded into the other LDS buffer, one barrier.
constexpr int XNW = 128, XKS = 32;
constexpr int XPF = 4;  // steps of weight bytes and X in flight per thread
template <int QT, int EPI, bool LEG16, int MT, bool SPLIT = false>
__global__ __launch_bounds__(256) void xq_gemm_kernel(const uint8_t *__restrict__ W,
                                                      const float *__restrict__ X, float *__restrict__ Y,
                                                      int n, int ldy, int k, int T, int tiles_m, int tiles_n,
                                                      int splits, long pstride) {
    using TR = XqTraits<QT>;
    typedef typename std::conditional<LEG16, _Float16, float>::type op_t;
    static_assert(MT == 64 || MT == 128, "tile rows");
    constexpr int IT = MT / 64;                         // 32-row tiles per wave
    constexpr int PADK = LEG16 ? XKS + 8 : XKS + 4;    // LDS row pitch, elements
    constexpr int A_ELEMS = MT * PADK, B_ELEMS = XNW * PADK;
    constexpr int LOOP_BYTES = 2 * (A_ELEMS + B_ELEMS) * (int)sizeof(op_t);
    constexpr int C_PITCH = XNW + 4;
    constexpr int EPI_BYTES = MT * C_PITCH * 4;
    __shared__ __attribute__((aligned(16))) uint8_t smem[LOOP_BYTES > EPI_BYTES ? LOOP_BYTES : EPI_BYTES];
    op_t *As = reinterpret_cast<op_t *>(smem);
    op_t *Bs = As + 2 * A_ELEMS;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tile = blockIdx.x % (tiles_m * tiles_n), split = blockIdx.x / (tiles_m * tiles_n);
    const int tm = tile % tiles_m, tn = tile / tiles_m;
    const int m0 = tm * MT;
    // SPLIT (PLAIN only): this workgroup's share of the 32-k steps, whose sums go to
    // block `split` of the partial sums ([T][n], pstride floats apart).
    const int nks_all = k / XKS;
    const int ks_begin = (int)((long)nks_all * split / splits);
    const int ks_end = (int)((long)nks_all * (split + 1) / splits);
    static_assert(!SPLIT || EPI == EPI_PLAIN, "a split stores PLAIN partial sums");
    if constexpr (SPLIT) {
        Y += (size_t)split * pstride;
        ldy = n;
    }
    constexpr int OUT = EPI == EPI_SWIGLU ? XNW / 2 : XNW;  // outputs per tile
    const int o0 = tn * OUT;

    // Staging: thread t decodes weights 16 (t & 1) .. + 15 of the step for tile row
    // t >> 1, and converts X floats APT (t % (32 / APT)) .. + APT - 1 of token row
    // t / (32 / APT).
    const int brow = tid >> 1, bhalf = tid & 1;
    int wr;  // global weight row of tile row brow (clamped inside the weight)
    if constexpr (EPI == EPI_SWIGLU) {
        const int o = min(o0 + (brow & (XNW / 2 - 1)), n - 1);
        wr = brow < XNW / 2 ? o : n + o;
    } else {
        wr = min(o0 + brow, n - 1);
    }
    const uint8_t *wrow = W + (size_t)wr * (k / TR::ELEMS) * TR::BYTES;
    constexpr int APT = MT * XKS / 256;                 // X floats per thread per step (8 / 16)
    constexpr int AF4 = APT / 4;
    const int arow = tid / (XKS / APT), acol = (tid % (XKS / APT)) * APT;
    const float *xrow = X + (size_t)min(m0 + arow, T - 1) * k + acol;

    // Ring of XPF steps' raw weight bytes and X in registers: slot j % XPF holds step j
    // from XPF steps before its decode. Step indices past the last are clamped, so
    // every load is issued unconditionally (in-order wait counts then never wait for
    // a younger load).
    const int nks = ks_end - ks_begin;
    Raw16<QT> raw[XPF];
    f4_t xv[XPF][AF4];
    auto load_step = [&](int ks, int slot) __attribute__((always_inline)) {
        const int e = (ks_begin + min(ks, nks - 1)) * XKS + 16 * bhalf;
        load_raw16<QT>(wrow + (size_t)(e / TR::ELEMS) * TR::BYTES, e % TR::ELEMS, raw[slot]);
        const f4_t *xp = reinterpret_cast<const f4_t *>(xrow + (ks_begin + min(ks, nks - 1)) * XKS);
#pragma unroll
        for (int i = 0; i < AF4; ++i) xv[slot][i] = xp[i];
    };
    // Decode, then 16-byte LDS stores (row pitches and offsets are multiples of 16 bytes).
    auto store_step = [&](int ks, int slot, int buf) __attribute__((always_inline)) {
        float wv[16];
        op_t *b = Bs + buf * B_ELEMS + brow * PADK + 16 * bhalf;
        op_t *a = As + buf * A_ELEMS + arow * PADK + acol;
        if constexpr (LEG16) {
            uint32_t p[8];
            if constexpr (QT == XQ_F16) {
                // the binary16 weights themselves (their f32 values round back to them)
                reinterpret_cast<u4_t *>(b)[0] = raw[slot].a;
                reinterpret_cast<u4_t *>(b)[1] = raw[slot].b;
            } else {
                decode_raw16<QT>(raw[slot], ((ks_begin + min(ks, nks - 1)) * XKS + 16 * bhalf) % TR::ELEMS, wv);
#pragma unroll
                for (int j = 0; j < 8; ++j) p[j] = h2_bits(h2_t{(_Float16)wv[2 * j], (_Float16)wv[2 * j + 1]});
                reinterpret_cast<u4_t *>(b)[0] = u4_t{p[0], p[1], p[2], p[3]};
                reinterpret_cast<u4_t *>(b)[1] = u4_t{p[4], p[5], p[6], p[7]};
            }
#pragma unroll
            for (int i = 0; i < AF4 / 2; ++i) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f4_t &v = xv[slot][2 * i + (j >> 1)];
                    p[j] = h2_bits(h2_t{(_Float16)v[2 * (j & 1)], (_Float16)v[2 * (j & 1) + 1]});
                }
                reinterpret_cast<u4_t *>(a)[i] = u4_t{p[0], p[1], p[2], p[3]};
            }
        } else {
            decode_raw16<QT>(raw[slot], ((ks_begin + min(ks, nks - 1)) * XKS + 16 * bhalf) % TR::ELEMS, wv);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                reinterpret_cast<f4_t *>(b)[j] = f4_t{wv[4 * j], wv[4 * j + 1], wv[4 * j + 2], wv[4 * j + 3]};
#pragma unroll
            for (int i = 0; i < AF4; ++i) reinterpret_cast<f4_t *>(a)[i] = xv[slot][i];
        }
    };

    f16v_t acc[IT][2];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        acc[i][0] = f16v_t{};
        acc[i][1] = f16v_t{};
    }
    const int c = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int j = 0; j < XPF; ++j) load_step(j, j);
    store_step(0, 0, 0);
    load_step(XPF, 0);
    __syncthreads();
    // Steps are walked in groups of XPF (the ring's slots are indexed statically); a
    // step past the last only moves data, and every wave reaches every barrier.
    for (int ks0 = 0; ks0 < nks; ks0 += XPF)
#pragma unroll
    for (int jj = 0; jj < XPF; ++jj) {
        const int ks = ks0 + jj;
        const int buf = ks & 1;
        if (ks < nks) {
            const op_t *a = As + buf * A_ELEMS + (wm * (MT / 2) + c) * PADK;
            const op_t *b = Bs + buf * B_ELEMS + (wn * 64 + c) * PADK;
            if constexpr (LEG16) {
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    h8_t bf[2];
#pragma unroll
                    for (int j = 0; j < 2; ++j) bf[j] = *reinterpret_cast<const h8_t *>(b + j * 32 * PADK + 16 * s + 8 * hh);
#pragma unroll
                    for (int i = 0; i < IT; ++i) {
                        const h8_t af = *reinterpret_cast<const h8_t *>(a + i * 32 * PADK + 16 * s + 8 * hh);
#pragma unroll
                        for (int j = 0; j < 2; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bf[j], acc[i][j], 0, 0, 0);
                    }
                }
            } else {
#pragma unroll
                for (int s = 0; s < XKS / 2; ++s) {
#pragma unroll
                    for (int i = 0; i < IT; ++i) {
                        const float af = a[i * 32 * PADK + 2 * s + hh];
#pragma unroll
                        for (int j = 0; j < 2; ++j) {
                            const float bf = b[j * 32 * PADK + 2 * s + hh];
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af, bf, acc[i][j], 0, 0, 0);
                        }
                    }
                }
            }
        }
        // Step ks + 1 into the other LDS buffer (its last reader finished before the
        // barrier that ended step ks - 1); its slot then takes step ks + 1 + XPF.
        store_step(ks + 1, (jj + 1) % XPF, buf ^ 1);
        load_step(ks + 1 + XPF, (jj + 1) % XPF);
        __syncthreads();
    }

    // Accumulators -> LDS C [token row][tile column] (lane (c, hh) of tile (i, j) holds
    // rows 32 i + 8 (r / 4) + 4 hh + r % 4 of column 32 j + c), then whole rows to Y.
    float *C = reinterpret_cast<float *>(smem);
#pragma unroll
    for (int i = 0; i < IT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                C[(wm * (MT / 2) + i * 32 + 8 * (r >> 2) + 4 * hh + (r & 3)) * C_PITCH + wn * 64 + j * 32 + c] =
                    acc[i][j][r];
    __syncthreads();
    for (int i = tid; i < MT * OUT; i += 256) {
        const int t = i / OUT, oc = i % OUT;
        const int tt = m0 + t, o = o0 + oc;
        if (tt >= T || o >= n) continue;
        float *y = Y + (size_t)tt * ldy + o;
        const float v = C[t * C_PITCH + oc];
        if constexpr (EPI == EPI_SWIGLU) {
            const float u = C[t * C_PITCH + XNW / 2 + oc];
            *y = LEG16 ? silu_fast(v) * u : silu_f32(v) * u;
        } else if constexpr (EPI == EPI_RESIDUAL) {
            *y = *y + v;
        } else {
            *y = v;
        }
    }
}

// x staged in LDS (xq_gemv_kernel's XL) for the one-row waves (n < 8192) where a
// launch's tokens take at most 64 KB of it, eight waves sharing it: 4096 x 12288 at T = 1
// Q4_K 17.1 -> 13.0 us, Q5_K 20.0 -> 14.2, Q6_K 22.8 -> 17.3. The four-row waves of the
// wider weights already share x among their rows, and workgroups of eight such waves
// (384 for 12288 rows) leave the CUs unevenly loaded: Q4_K 12288 x 4096 at T = 1 10.5
// -> 17.7 us with it.
constexpr int XQ_GEMV_XL_BYTES = 64 * 1024;
constexpr int XQ_GEMV_XL_WV = 8;  // waves per workgroup sharing the staged x
// Up to 128 KB of x (two tokens at k = 12288) sixteen waves share it, one workgroup per
// CU; the launch's tokens are chunked so that x fits. Sixteen waves also take up to two
// tokens wherever that still makes 256 workgroups (x staged half as often): 4096 x 12288
// at T = 1 Q4_K 13.0 -> 11.9 us, Q6_K 15.5 -> 14.6, IQ4_XS 14.8 -> 13.7.
constexpr int XQ_GEMV_XL_MAX = 128 * 1024;

// x per token in LDS (float4 units): the transposed layout fills whole rounds of the
// wave's loop, 1024 k (Q6_K's paired loop: 2048 k)
inline int xq_gemv_xtok(int qt, int k) {
    return qt == XQ_Q6_K ? (k + 2047) / 2048 * 512 : (k + 1023) / 1024 * 256;
}

template <int QT, int EPI, int R, int TT>
void launch_gemv_tt(const GemmArgs &a, const float *x, float *y, hipStream_t s) {
    constexpr int OUTW = EPI == EPI_SWIGLU ? R / 2 : R;  // outputs per wave
    const int xtok = xq_gemv_xtok(QT, a.k);
    const int xl_bytes = TT * xtok * 16;
    const int wg16 = (a.n + 16 * OUTW - 1) / (16 * OUTW);
    if (R <= 2 && TT <= 2 && xl_bytes <= XQ_GEMV_XL_MAX && (xl_bytes > XQ_GEMV_XL_BYTES || wg16 >= 256)) {
        constexpr int WV = 16;
        const dim3 grid(wg16);
        hipLaunchKernelGGL((xq_gemv_kernel<QT, EPI, TT <= 2 ? TT : 2, R, true, WV>), grid, dim3(64 * WV), xl_bytes, s,
                           a.W, x, y, a.n, a.ldy, a.k, xtok);
    } else if (R <= 2 && xl_bytes <= XQ_GEMV_XL_BYTES) {
        constexpr int WV = XQ_GEMV_XL_WV;
        const dim3 grid((a.n + WV * OUTW - 1) / (WV * OUTW));
        hipLaunchKernelGGL((xq_gemv_kernel<QT, EPI, TT, R, true, WV>), grid, dim3(64 * WV), xl_bytes, s, a.W, x, y,
                           a.n, a.ldy, a.k, xtok);
    } else {
        const dim3 grid((a.n + 4 * OUTW - 1) / (4 * OUTW));
        hipLaunchKernelGGL((xq_gemv_kernel<QT, EPI, TT, R>), grid, dim3(256), 0, s, a.W, x, y, a.n, a.ldy, a.k, 0);
    }
}

template <int QT, int EPI, int R>
hipError_t launch_gemv_r(const GemmArgs &a, hipStream_t s) {
    // tokens per launch: four, or fewer where that keeps one-row waves' x in LDS
    const int xb = xq_gemv_xtok(QT, a.k) * 16;
    const int per = (R <= 2 && xb <= XQ_GEMV_XL_MAX) ? min(4, XQ_GEMV_XL_MAX / xb) : 4;
    for (int t0 = 0; t0 < a.T; t0 += per) {
        const int tt = min(per, a.T - t0);
        const float *x = a.X + (size_t)t0 * a.k;
        float *y = a.Y + (size_t)t0 * a.ldy;
        switch (tt) {
        case 1: launch_gemv_tt<QT, EPI, R, 1>(a, x, y, s); break;
        case 2: launch_gemv_tt<QT, EPI, R, 2>(a, x, y, s); break;
        case 3: launch_gemv_tt<QT, EPI, R, 3>(a, x, y, s); break;
        default: launch_gemv_tt<QT, EPI, R, 4>(a, x, y, s); break;
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Four rows per wave where n / 4 waves still give 8 per CU (256 CUs): n >= 8192.
template <int QT, int EPI>
hipError_t launch_gemv_e(const GemmArgs &a, hipStream_t s) {
    if (a.n >= 8192) return launch_gemv_r<QT, EPI, 4>(a, s);
    return launch_gemv_r<QT, EPI, EPI == EPI_SWIGLU ? 2 : 1>(a, s);
}

template <int QT>
hipError_t launch_gemv_q(const GemmArgs &a, hipStream_t s) {
    switch (a.epilogue) {
    case EPI_PLAIN: return launch_gemv_e<QT, EPI_PLAIN>(a, s);
    case EPI_RESIDUAL: return launch_gemv_e<QT, EPI_RESIDUAL>(a, s);
    default: return launch_gemv_e<QT, EPI_SWIGLU>(a, s);
    }
}

// Tile rows: 128 on the f16 leg (twice the matrix-core work per decoded weight) when
// that still makes at least 256 workgroups, else 64 (the f32 leg always).
int xq_tile_rows(int T, int n, int epilogue, bool leg16) {
    const int out = epilogue == EPI_SWIGLU ? XNW / 2 : XNW;
    return leg16 && (long)((T + 127) / 128) * ((n + out - 1) / out) >= 256 ? 128 : 64;
}

#ifndef PF_XQ_TARGET_WG
#define PF_XQ_TARGET_WG 768
#endif
// K split of the f16 leg's tiles through a workspace where the tiles alone leave the
// resident slots idle (three workgroups per CU): that many splits, each of at least 16
// steps of 32 k (512 k), at most 16. PLAIN / RESIDUAL: the splits' partial sums are
// added (with R) in split order by split_sum_kernel. SwiGLU up to XQ_SCRATCH_T rows: the
// gate and up rows run as one split PLAIN GEMM over the 2n rows into G, and
// swiglu_apply_kernel sums each half in split order and applies silu(g) * u (above that
// the fused epilogue runs unsplit, as G's round trip grows with T). The f32 leg does not
// split. Deterministic either way.
#ifndef PF_XQ_SCRATCH_T
#define PF_XQ_SCRATCH_T 64
#endif
constexpr int XQ_SCRATCH_T = PF_XQ_SCRATCH_T;
int xq_splits(int T, int n, int k, int epilogue, bool leg16) {
    if (!leg16 || (epilogue == EPI_SWIGLU && T > XQ_SCRATCH_T)) return 1;
    const int rows = epilogue == EPI_SWIGLU ? 2 * n : n;  // the PLAIN GEMM's weight rows
    const int mt = xq_tile_rows(T, rows, EPI_PLAIN, leg16);
    const long tiles = (long)((T + mt - 1) / mt) * ((rows + XNW - 1) / XNW);
    if (tiles >= PF_XQ_TARGET_WG) return 1;
    int splits = (int)(PF_XQ_TARGET_WG / tiles);
    const int by_k = (k / XKS) / 16;
    if (splits > by_k) splits = by_k;
    if (splits > 16) splits = 16;
    return splits < 1 ? 1 : splits;
}

template <int QT, int EPI, bool LEG16, int MT, bool SPLIT>
hipError_t launch_tiles(const GemmArgs &a, float *ps, int splits, hipStream_t s) {
    constexpr int OUT = EPI == EPI_SWIGLU ? XNW / 2 : XNW;
    const int tm = (a.T + MT - 1) / MT, tn = (a.n + OUT - 1) / OUT;
    if constexpr (SPLIT)
        hipLaunchKernelGGL((xq_gemm_kernel<QT, EPI, LEG16, MT, true>), dim3(tm * tn * splits), dim3(256), 0, s, a.W,
                           a.X, ps, a.n, a.n, a.k, a.T, tm, tn, splits, part_stride(a.T, a.n));
    else
        hipLaunchKernelGGL((xq_gemm_kernel<QT, EPI, LEG16, MT>), dim3(tm * tn), dim3(256), 0, s, a.W, a.X, a.Y,
                           a.n, a.ldy, a.k, a.T, tm, tn, 1, 0L);
    return hipGetLastError();
}

// The split PLAIN GEMM of `a` (its n weight rows) into the partial-sum blocks at ps.
template <int QT>
hipError_t launch_split_plain(const GemmArgs &a, float *ps, int splits, hipStream_t s) {
    if (xq_tile_rows(a.T, a.n, EPI_PLAIN, true) == 128)
        return launch_tiles<QT, EPI_PLAIN, true, 128, true>(a, ps, splits, s);
    return launch_tiles<QT, EPI_PLAIN, true, 64, true>(a, ps, splits, s);
}

template <int QT, int EPI, bool LEG16>
hipError_t launch_gemm_e(const GemmArgs &a, float *ps, hipStream_t s) {
    const int splits = ps ? xq_splits(a.T, a.n, a.k, EPI, LEG16) : 1;
    if constexpr (LEG16) {
        if (splits > 1) {
            hipError_t e;
            if constexpr (EPI == EPI_SWIGLU) {
                GemmArgs g = a;  // the gate and up rows as one PLAIN GEMM over 2n rows
                g.epilogue = EPI_PLAIN;
                g.n = 2 * a.n;
                g.ldy = 2 * a.n;
                e = launch_split_plain<QT>(g, ps, splits, s);
                if (e != hipSuccess) return e;
                return launch_swiglu_apply(ps, a, splits, s);
            } else {
                // PLAIN partial sums; the sum kernel adds R for RESIDUAL
                e = launch_split_plain<QT>(a, ps, splits, s);
            }
            if (e != hipSuccess) return e;
            return launch_split_sum(a, ps, splits, s);
        }
        if (xq_tile_rows(a.T, a.n, EPI, true) == 128) return launch_tiles<QT, EPI, true, 128, false>(a, ps, 1, s);
    }
    return launch_tiles<QT, EPI, LEG16, 64, false>(a, ps, 1, s);
}

template <int QT, bool LEG16>
hipError_t launch_gemm_q(const GemmArgs &a, float *ps, hipStream_t s) {
    switch (a.epilogue) {
    case EPI_PLAIN: return launch_gemm_e<QT, EPI_PLAIN, LEG16>(a, ps, s);
    case EPI_RESIDUAL: return launch_gemm_e<QT, EPI_RESIDUAL, LEG16>(a, ps, s);
    default: return launch_gemm_e<QT, EPI_SWIGLU, LEG16>(a, ps, s);
    }
}

template <int QT, bool F16OUT>
hipError_t launch_dequant_q(const uint8_t *W, int rows, int k, void *out, hipStream_t s) {
    const long runs = (long)rows * (k / 16);
    hipLaunchKernelGGL((xq_dequant_kernel<QT, F16OUT>), dim3((unsigned)((runs + 255) / 256)), dim3(256), 0, s, W,
                       rows, k, out);
    return hipGetLastError();
}

template <bool F16OUT>
hipError_t launch_dequant_t(int qtype, const uint8_t *W, int rows, int k, void *out, hipStream_t s) {
    switch (qtype) {
    case XQ_F16: return launch_dequant_q<XQ_F16, F16OUT>(W, rows, k, out, s);
    case XQ_Q4_K: return launch_dequant_q<XQ_Q4_K, F16OUT>(W, rows, k, out, s);
    case XQ_Q5_K: return launch_dequant_q<XQ_Q5_K, F16OUT>(W, rows, k, out, s);
    case XQ_Q6_K: return launch_dequant_q<XQ_Q6_K, F16OUT>(W, rows, k, out, s);
    default: return launch_dequant_q<XQ_IQ4_XS, F16OUT>(W, rows, k, out, s);
    }
}

}  // namespace

hipError_t launch_xq_gemv(const GemmArgs &a, hipStream_t s) {
    switch (a.qtype) {
    case XQ_F16: return launch_gemv_q<XQ_F16>(a, s);
    case XQ_Q4_K: return launch_gemv_q<XQ_Q4_K>(a, s);
    case XQ_Q5_K: return launch_gemv_q<XQ_Q5_K>(a, s);
    case XQ_Q6_K: return launch_gemv_q<XQ_Q6_K>(a, s);
    default: return launch_gemv_q<XQ_IQ4_XS>(a, s);
    }
}

hipError_t launch_xq_gemm(const GemmArgs &a, bool leg16, void *ws, hipStream_t s) {
    float *ps = static_cast<float *>(ws);
    switch (a.qtype) {
    case XQ_F16: return leg16 ? launch_gemm_q<XQ_F16, true>(a, ps, s) : launch_gemm_q<XQ_F16, false>(a, ps, s);
    case XQ_Q4_K: return leg16 ? launch_gemm_q<XQ_Q4_K, true>(a, ps, s) : launch_gemm_q<XQ_Q4_K, false>(a, ps, s);
    case XQ_Q5_K: return leg16 ? launch_gemm_q<XQ_Q5_K, true>(a, ps, s) : launch_gemm_q<XQ_Q5_K, false>(a, ps, s);
    case XQ_Q6_K: return leg16 ? launch_gemm_q<XQ_Q6_K, true>(a, ps, s) : launch_gemm_q<XQ_Q6_K, false>(a, ps, s);
    default: return leg16 ? launch_gemm_q<XQ_IQ4_XS, true>(a, ps, s) : launch_gemm_q<XQ_IQ4_XS, false>(a, ps, s);
    }
}

int64_t xq_ws_bytes(int T, int n, int k, int epilogue, bool leg16) {
    const int splits = xq_splits(T, n, k, epilogue, leg16);
    return splits > 1 ? (int64_t)splits * part_stride(T, epilogue == EPI_SWIGLU ? 2 * n : n) * 4 : 0;
}

hipError_t launch_xq_dequant(int qtype, const uint8_t *W, int rows, int k, void *out, bool f16_out, hipStream_t s) {
    return f16_out ? launch_dequant_t<true>(qtype, W, rows, k, out, s)
                   : launch_dequant_t<false>(qtype, W, rows, k, out, s);
}

}  // namespace pf
