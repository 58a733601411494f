/*
 * CPU ORACLE for the quantized-weight prefill GEMM — TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load this library. The product path never calls it, and it shares no source,
 * header, table or helper with the GPU library.
 *
 * What it computes is the plain definition of the method, in fp64:
 *
 *     W_hat = decode(W_blocks)                 (GGUF Q4_0 / Q8_0, 32-element blocks)
 *     Y_ref = epilogue(X . W_hat^T)            (PLAIN, RESIDUAL or GATE_UP_SWIGLU)
 *
 * Sources (pages):
 *  - aprender-serve 0.70.2, src/cuda/executor/gdn_prefill_ops.rs, module doc
 *    group 1 "Projections as GEMMs" and `qwen35_project_rows`: every projection
 *    is Y[rows x n] = X[rows x k] . W^T, all row-major, fp32 in and out (f32 leg)
 *    or fp16 inputs with fp32 accumulation (f16 leg).
 *  - aprender-serve 0.70.2, src/gguf/cuda/forward_qwen35_cuda_prefill.rs,
 *    `prefill_ffn_rows`: gate GEMM, up GEMM, `fused_swiglu_into(gate, up, act)`,
 *    down GEMM, `residual_add_into(x, proj, x)`.
 *  - oxibonsai-kernels 0.1.4, src/gpu_backend/cuda_q_std_prefill.rs, module doc
 *    ("Weight layout": AoS blocks as stored in GGUF), `launch_gemm_q4_0`
 *    (accumulates with +=), `launch_fused_gate_up_swiglu_q4_0` (gate rows then
 *    up rows in one buffer), and test `test_q_std_prefill_batch12_no_capof8`
 *    (18-byte Q4_0 block, fp16 scale 0x3C00 little-endian, nibble 8 = weight 0).
 *  - GGUF block formats: Q4_0 = fp16 d + 16 bytes of nibbles, element j < 16 is
 *    the low nibble of byte j, element j >= 16 the high nibble of byte j-16,
 *    value d*(q-8). Q8_0 = fp16 d + 32 int8 q, value d*q.
 *  - aprender-serve 0.70.2, src/cuda/executor/gdn_prefill_ops.rs,
 *    `qwen35_dequant_f32`: the further weight types the f32 leg dequantizes (F16,
 *    Q4_K, Q5_K, Q6_K over 256-element super-blocks, F16 over 32-element groups),
 *    and `qwen35_fp16_weight`: the f16 leg's weight is that f32 value rounded to
 *    binary16. The pages print none of these layouts; they are GGUF's, restated
 *    at decode_k_block and decode_iq4_xs_block below. The same function also
 *    dequantizes IQ4_XS over 256-element super-blocks (`Iq4XsDequantKernel`).
 *  - IEEE 754 binary16 for the scale and for the f16 leg's input rounding.
 *
 * Every floating-point step is written out: no fast-math, no FMA contraction
 * (built with -O2 -ffp-contract=off), sums in ascending index order. OpenMP splits
 * only over independent outputs, so no result depends on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_Q4_0 0
#define ORACLE_Q8_0 1
#define ORACLE_F16 2
#define ORACLE_Q4_K 3
#define ORACLE_Q5_K 4
#define ORACLE_Q6_K 5
#define ORACLE_IQ4_XS 6

#define ORACLE_PLAIN 0
#define ORACLE_RESIDUAL 1
#define ORACLE_GATE_UP_SWIGLU 2

/* Threads the OpenMP loops below use (1 without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------------------
 * IEEE 754 binary16, decoded from its definition (sign, 5-bit biased exponent,
 * 10-bit fraction). Subnormals: (-1)^s * f * 2^-24. Normals: (-1)^s *
 * (1024 + f) * 2^(e - 25). Exponent 31: infinity (f == 0) or NaN.
 * ------------------------------------------------------------------------- */
double oracle_fp16_to_f64(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double mag;
    if (e == 0) {
        mag = ldexp((double)f, -24);
    } else if (e == 31) {
        mag = (f == 0) ? INFINITY : NAN;
    } else {
        mag = ldexp((double)(1024 + f), e - 25);
    }
    return s ? -mag : mag;
}

void oracle_fp16_decode_array(const uint16_t *h, int64_t count, double *out)
{
    for (int64_t i = 0; i < count; ++i)
        out[i] = oracle_fp16_to_f64(h[i]);
}

/* ---------------------------------------------------------------------------
 * f32 -> binary16 with round-to-nearest, ties-to-even, gradual underflow and
 * overflow to infinity, written from the definition on the exact binary value
 * of the f32 input (an integer significand times a power of two).
 * ------------------------------------------------------------------------- */
uint16_t oracle_f32_to_fp16_rne(float x)
{
    uint32_t bits;
    memcpy(&bits, &x, 4);
    uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    uint32_t ex = (bits >> 23) & 0xFFu;
    uint32_t fr = bits & 0x7FFFFFu;
    if (ex == 0xFFu) /* inf or NaN */
        return (uint16_t)(sign | 0x7C00u | (fr ? 0x200u : 0u));
    if (ex == 0 && fr == 0)
        return sign;
    /* |x| = M * 2^E exactly, with M < 2^24. */
    uint64_t M;
    int E;
    if (ex == 0) {
        M = fr;
        E = -149;
    } else {
        M = fr | 0x800000u;
        E = (int)ex - 150;
    }
    /* Normalise so that 2^23 <= M < 2^24; then |x| = (M / 2^23) * 2^(E + 23). */
    while (M < 0x800000u) {
        M <<= 1;
        E -= 1;
    }
    int unbiased = E + 23; /* |x| in [2^unbiased, 2^(unbiased+1)) */
    /* Target quantum: normals have 11 significant bits -> ulp 2^(unbiased-10);
     * below 2^-14 the quantum is fixed at 2^-24 (subnormal range). */
    int q = (unbiased >= -14) ? unbiased - 10 : -24;
    /* |x| / 2^q = M * 2^(E - q); shift right by (q - E) bits with RNE. */
    int sh = q - E;
    uint64_t n; /* rounded count of quanta */
    if (sh <= 0) {
        n = M << (-sh);
    } else if (sh >= 64) {
        n = 0;
    } else {
        uint64_t whole = M >> sh;
        uint64_t rem = M - (whole << sh);
        uint64_t half = (uint64_t)1 << (sh - 1);
        if (rem > half || (rem == half && (whole & 1u)))
            whole += 1;
        n = whole;
    }
    /* Re-express n * 2^q as a binary16 pattern. */
    if (q == -24) {
        /* subnormal range: n quanta of 2^-24; n == 1024 is the smallest normal */
        return (uint16_t)(sign | (uint16_t)n); /* n <= 1024 here; 1024 -> 0x0400 */
    }
    /* normal range: n in [1024, 2048]; n == 2048 bumps the exponent */
    int e16 = unbiased + 15;
    if (n == 2048) {
        n = 1024;
        e16 += 1;
    }
    if (e16 >= 31)
        return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (uint16_t)(e16 << 10) | (uint16_t)(n - 1024));
}

void oracle_f32_to_fp16_array(const float *x, int64_t count, uint16_t *out)
{
    for (int64_t i = 0; i < count; ++i)
        out[i] = oracle_f32_to_fp16_rne(x[i]);
}

/* ---------------------------------------------------------------------------
 * GGUF block decode.
 * ------------------------------------------------------------------------- */
int oracle_block_bytes(int qtype)
{
    switch (qtype) {
    case ORACLE_Q4_0: return 18;
    case ORACLE_Q8_0: return 34;
    case ORACLE_F16: return 64;     /* 32 binary16 values */
    case ORACLE_Q4_K: return 144;
    case ORACLE_Q5_K: return 176;
    case ORACLE_Q6_K: return 210;
    case ORACLE_IQ4_XS: return 136;
    default: return -1;
    }
}

/* Weights per block: 32, or 256 for the super-block types. */
int oracle_block_elems(int qtype)
{
    return (qtype == ORACLE_Q4_K || qtype == ORACLE_Q5_K || qtype == ORACLE_Q6_K ||
            qtype == ORACLE_IQ4_XS) ? 256 : 32;
}

/* The scale: a binary16 stored little-endian in bytes 0-1 of the block. Its
 * value is exactly representable in f32, so the conversion is exact. */
static float block_scale(const uint8_t *blk)
{
    uint16_t h = (uint16_t)(blk[0] | (blk[1] << 8));
    return (float)oracle_fp16_to_f64(h);
}

static float fp16_at(const uint8_t *p)
{
    return (float)oracle_fp16_to_f64((uint16_t)(p[0] | (p[1] << 8)));
}

/* The 6-bit scale and min of sub-block j (0..7) of a Q4_K / Q5_K super-block, from
 * its 12 packed bytes: sub-blocks 0-3 keep theirs in the low 6 bits of bytes j
 * (scale) and j + 4 (min); sub-blocks 4-7 take their low 4 bits from the two
 * nibbles of byte j + 4 (scale low, min high) and their top 2 bits from the top
 * bits of bytes j - 4 (scale) and j (min). */
static void k_scale_min(const uint8_t sc[12], int j, int *s, int *m)
{
    if (j < 4) {
        *s = sc[j] & 63;
        *m = sc[j + 4] & 63;
    } else {
        *s = (sc[j + 4] & 15) | ((sc[j - 4] >> 6) << 4);
        *m = (sc[j + 4] >> 4) | ((sc[j] >> 6) << 4);
    }
}

/* Decode one 256-element super-block (GGUF's K types) into f32.
 *
 * Q4_K (144 bytes): fp16 d, fp16 dmin, 12 bytes of 6-bit scales and mins, 128
 *   bytes of nibbles. Element e lies in 64-element group p = e / 64; within it,
 *   element l < 32 is the low nibble of qs[32p + l] and 32 + l its high nibble;
 *   its sub-block is j = e / 32. Value (d s_j) q - dmin m_j: d s_j, dmin m_j and
 *   (d s_j) q are exact in f32 (11 + 6 + 4 significant bits), so the one rounding
 *   is the subtraction's.
 * Q5_K (176 bytes): as Q4_K with 32 bytes qh after the scales (then the 128 qs):
 *   element e = 32 b + l (b = 0..7, l = 0..31) adds 16 times bit b of qh[l].
 * Q6_K (210 bytes): ql[128], qh[64], 16 int8 scales, fp16 d last. In half
 *   h = e / 128 (ql from 64 h, qh from 32 h, scales from 8 h), quarter c = (e % 128)
 *   / 32 and l = e % 32: the low 4 bits are the low (c = 0, 1) or high (c = 2, 3)
 *   nibble of ql[l + 32 (c % 2)], the top 2 bits are bits 2c, 2c+1 of qh[l], and the
 *   scale is scales[l / 16 + 2c]. Value (d sc) (q - 32): d sc is exact, the product
 *   with q - 32 rounds once. */
static void decode_k_block(int qtype, const uint8_t *blk, float *out)
{
    if (qtype == ORACLE_Q6_K) {
        const uint8_t *ql = blk, *qh = blk + 128;
        const int8_t *sc = (const int8_t *)(blk + 192);
        float d = fp16_at(blk + 208);
        for (int e = 0; e < 256; ++e) {
            int h = e / 128, c = (e % 128) / 32, l = e % 32;
            int lo = ql[64 * h + l + 32 * (c % 2)];
            lo = (c < 2) ? (lo & 15) : (lo >> 4);
            int hi = (qh[32 * h + l] >> (2 * c)) & 3;
            int q = lo | (hi << 4);
            float ds = d * (float)sc[8 * h + l / 16 + 2 * c];
            out[e] = ds * (float)(q - 32);
        }
        return;
    }
    float d = fp16_at(blk), dmin = fp16_at(blk + 2);
    const uint8_t *sc = blk + 4;
    const uint8_t *qh = (qtype == ORACLE_Q5_K) ? blk + 16 : NULL;
    const uint8_t *qs = (qtype == ORACLE_Q5_K) ? blk + 48 : blk + 16;
    for (int e = 0; e < 256; ++e) {
        int p = e / 64, l = e % 32, upper = (e % 64) >= 32;
        int q = upper ? (qs[32 * p + l] >> 4) : (qs[32 * p + l] & 15);
        if (qh)
            q += ((qh[l] >> (e / 32)) & 1) * 16;
        int s, m;
        k_scale_min(sc, e / 32, &s, &m);
        float a = d * (float)s, b = dmin * (float)m;
        float aq = a * (float)q;
        out[e] = aq - b;
    }
}

/* The 16 values an IQ4_XS code selects (GGUF's non-linear 4-bit grid, shared with
 * IQ4_NL), indexed by the code. */
static const int IQ4_GRID[16] = {-127, -104, -83, -65, -49, -35, -22, -10,
                                 1, 13, 25, 38, 53, 69, 89, 113};

/* Decode one IQ4_XS super-block (136 bytes, 256 elements) into f32: fp16 d, a
 * little-endian uint16 scales_h, 4 bytes scales_l, then 128 bytes of codes. Element
 * e lies in sub-block b = e / 32; its 6-bit scale has its low 4 bits in the nibble b
 * % 2 (low for even b) of scales_l[b / 2] and its top 2 bits in bits 2b, 2b+1 of
 * scales_h. With l = e % 32, the code is the low (l < 16) or high (l >= 16) nibble
 * of qs[16 b + l % 16]. Value (d (ls - 32)) grid[code]: d (ls - 32) is exact in f32
 * (11 + 6 significant bits) and so is its product with a grid value (7 more bits). */
static void decode_iq4_xs_block(const uint8_t *blk, float *out)
{
    float d = fp16_at(blk);
    int scales_h = blk[2] | (blk[3] << 8);
    const uint8_t *scales_l = blk + 4, *qs = blk + 8;
    for (int e = 0; e < 256; ++e) {
        int b = e / 32, l = e % 32;
        int lo4 = (scales_l[b / 2] >> (4 * (b % 2))) & 15;
        int hi2 = (scales_h >> (2 * b)) & 3;
        int ls = lo4 | (hi2 << 4);
        float dl = d * (float)(ls - 32);
        int byte = qs[16 * b + l % 16];
        int code = (l < 16) ? (byte & 15) : (byte >> 4);
        out[e] = dl * (float)IQ4_GRID[code];
    }
}

/* Decode one block into f32 (32 or 256 elements, see oracle_block_elems). Q4_0 /
 * Q8_0: each value is one f32 multiply of the scale by a small integer; the
 * product of an 11-bit and a <= 8-bit significand is exact in f32, so these are
 * the canonical bits (including -0.0 when the scale is negative and the integer
 * is zero). F16: 32 little-endian binary16 values, widened exactly. */
static void decode_block(int qtype, const uint8_t *blk, float *out)
{
    if (qtype == ORACLE_F16) {
        for (int j = 0; j < 32; ++j)
            out[j] = fp16_at(blk + 2 * j);
        return;
    }
    if (qtype == ORACLE_IQ4_XS) {
        decode_iq4_xs_block(blk, out);
        return;
    }
    if (qtype >= ORACLE_Q4_K) {
        decode_k_block(qtype, blk, out);
        return;
    }
    float d = block_scale(blk);
    const uint8_t *qs = blk + 2;
    if (qtype == ORACLE_Q4_0) {
        for (int j = 0; j < 32; ++j) {
            int q = (j < 16) ? (qs[j] & 0x0F) : (qs[j - 16] >> 4);
            out[j] = d * (float)(q - 8);
        }
    } else {
        for (int j = 0; j < 32; ++j) {
            int q = (int)(int8_t)qs[j];
            out[j] = d * (float)q;
        }
    }
}

/* Decode `rows` rows of k / E blocks each (E = oracle_block_elems; row r, block b
 * at byte (r*(k/E) + b) * block_bytes) into out[rows][k]. */
void oracle_dequant_f32(int qtype, const uint8_t *W, int64_t rows, int64_t k, float *out)
{
    int bb = oracle_block_bytes(qtype), be = oracle_block_elems(qtype);
    int64_t nb = k / be;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b)
            decode_block(qtype, W + (r * nb + b) * bb, out + r * k + b * be);
}

/* f16-leg weights: the f32 decode, then one RNE rounding to binary16. */
void oracle_dequant_f16(int qtype, const uint8_t *W, int64_t rows, int64_t k, uint16_t *out)
{
    int bb = oracle_block_bytes(qtype), be = oracle_block_elems(qtype);
    int64_t nb = k / be;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float tmp[256];
        for (int64_t b = 0; b < nb; ++b) {
            decode_block(qtype, W + (r * nb + b) * bb, tmp);
            for (int j = 0; j < be; ++j)
                out[r * k + b * be + j] = oracle_f32_to_fp16_rne(tmp[j]);
        }
    }
}

static void decode_row(int qtype, const uint8_t *W, int64_t r, int64_t k, float *row)
{
    int bb = oracle_block_bytes(qtype), be = oracle_block_elems(qtype);
    int64_t nb = k / be;
    for (int64_t b = 0; b < nb; ++b)
        decode_block(qtype, W + (r * nb + b) * bb, row + b * be);
}

/* Dot product in fp64, ascending index: each product of two f32 values is exact
 * in fp64 (24 + 24 significant bits), so only the additions round. */
static double dot_f64(const float *w, const float *x, int64_t k)
{
    double acc = 0.0;
    for (int64_t i = 0; i < k; ++i)
        acc += (double)w[i] * (double)x[i];
    return acc;
}

/* out[t][r] = sum_i W_hat[r][i] * X[t][i] for all t < T, r < rows (fp64).
 * This is X . W_hat^T with X [T][k] and W_hat [rows][k], both row-major. */
void oracle_matmul(int qtype, const uint8_t *W, int64_t rows, int64_t k, const float *X,
                   int64_t T, double *out)
{
#pragma omp parallel
    {
        float *row = (float *)malloc((size_t)k * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            decode_row(qtype, W, r, k, row);
            for (int64_t t = 0; t < T; ++t)
                out[t * rows + r] = dot_f64(row, X + t * k, k);
        }
        free(row);
    }
}

/* The same sums for m chosen (t, r) pairs only: out[i] = sum_k W_hat[ri[i]][k] *
 * X[ti[i]][k]. Used to check full-size results element by element. */
void oracle_matmul_sampled(int qtype, const uint8_t *W, int64_t rows, int64_t k,
                           const float *X, int64_t T, const int64_t *ti, const int64_t *ri,
                           int64_t m, double *out)
{
    (void)rows;
    (void)T;
#pragma omp parallel
    {
        float *row = (float *)malloc((size_t)k * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t i = 0; i < m; ++i) {
            decode_row(qtype, W, ri[i], k, row);
            out[i] = dot_f64(row, X + ti[i] * k, k);
        }
        free(row);
    }
}

/* Euclidean norm of each decoded weight row, in fp64. */
void oracle_row_norms(int qtype, const uint8_t *W, int64_t rows, int64_t k, double *out)
{
#pragma omp parallel
    {
        float *row = (float *)malloc((size_t)k * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            decode_row(qtype, W, r, k, row);
            out[r] = sqrt(dot_f64(row, row, k));
        }
        free(row);
    }
}

/* SiLU from its textbook definition: g * sigma(g) = g / (1 + e^-g). */
double oracle_silu(double g)
{
    return g / (1.0 + exp(-g));
}

/* Epilogues on the fp64 products acc[T][rows]:
 *   PLAIN:          Y[t][r] = acc[t][r]                       (rows == n)
 *   RESIDUAL:       Y[t][r] = R[t][r] + acc[t][r]             (rows == n; R is the
 *                   Y buffer's prior content, updated in place)
 *   GATE_UP_SWIGLU: Y[t][r] = silu(acc[t][r]) * acc[t][n + r] (rows == 2n: gate
 *                   rows first, then up rows)
 * Y is [T][n] fp64. */
void oracle_epilogue(int epilogue, const double *acc, int64_t T, int64_t n, const float *R,
                     double *Y)
{
    int64_t rows = (epilogue == ORACLE_GATE_UP_SWIGLU) ? 2 * n : n;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t r = 0; r < n; ++r) {
            double v;
            if (epilogue == ORACLE_PLAIN) {
                v = acc[t * rows + r];
            } else if (epilogue == ORACLE_RESIDUAL) {
                v = (double)R[t * n + r] + acc[t * rows + r];
            } else {
                double g = acc[t * rows + r];
                double u = acc[t * rows + n + r];
                v = oracle_silu(g) * u;
            }
            Y[t * n + r] = v;
        }
    }
}

/* The whole method: Y_ref = epilogue(X . W_hat^T), fp64. W has 2n rows for
 * GATE_UP_SWIGLU, n rows otherwise. R may be NULL unless RESIDUAL. */
void oracle_gemm(int qtype, const uint8_t *W, int64_t n, int64_t k, const float *X, int64_t T,
                 const float *R, int epilogue, double *Y)
{
    int64_t rows = (epilogue == ORACLE_GATE_UP_SWIGLU) ? 2 * n : n;
    double *acc = (double *)malloc((size_t)(T * rows) * sizeof(double));
    oracle_matmul(qtype, W, rows, k, X, T, acc);
    oracle_epilogue(epilogue, acc, T, n, R, Y);
    free(acc);
}
