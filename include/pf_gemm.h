/*
 * pf_gemm.h - C ABI of the quantized-weight prefill GEMM library for MI355X (gfx950).
 *
 * One projection of a batched prompt prefill is one GEMM of T activation rows
 * against a GGUF block-quantized weight:
 *
 *     Y[T][n] = epilogue( X[T][k] . W_hat^T )      W_hat = decode(W_blocks)
 *
 * Pages this follows:
 *  - aprender-serve 0.70.2, src/cuda/executor/gdn_prefill_ops.rs: module doc,
 *    group 1 "Projections as GEMMs" (an f32 leg, fp32 in and out with no TF32, and
 *    an f16 leg, fp16 inputs with fp32 accumulation and fp32 output) and
 *    `qwen35_project_rows` (Y[rows x n] = X[rows x k] . W^T, all row-major).
 *  - aprender-serve 0.70.2, src/gguf/cuda/forward_qwen35_cuda_prefill.rs: module
 *    doc (every projection is one GEMM over the chunk's T rows instead of a
 *    per-token GEMV loop) and `prefill_ffn_rows` (gate, up, SwiGLU, down, residual).
 *  - oxibonsai-kernels 0.1.4, src/gpu_backend/cuda_q_std_prefill.rs: module doc
 *    (GGUF AoS blocks, no SoA reformatting), the Q4_0/Q8_0 kernel set
 *    (`CudaQStdPrefillModules`: GEMM, residual GEMM, fused gate/up SwiGLU GEMM and
 *    a single-token GEMV per block type), `launch_fused_gate_up_swiglu_q4_0` and
 *    the weight upload in `try_cuda_prefill_q_std` (gate rows, then up rows, in one
 *    buffer), and `try_cuda_prefill_q_std` (an empty batch is a no-op).
 *
 * Block formats (GGUF, rows stored block after block):
 *  - Q4_0, 18 bytes per 32 weights: fp16 scale d (little-endian, bytes 0-1), 16
 *    bytes qs. Weight j < 16 is the low nibble of qs[j], weight j >= 16 the high
 *    nibble of qs[j-16]; value d * (q - 8).
 *  - Q8_0, 34 bytes per 32 weights: fp16 scale d, then 32 int8 q; value d * q.
 *  The further types the page "aprender-serve 0.70.2 -
 *  src/cuda/executor/gdn_prefill_ops.rs" dequantizes (`qwen35_dequant_f32`; the f16
 *  leg's weight is that f32 value rounded to binary16, `qwen35_fp16_weight`). The
 *  pages print no layout; these are GGUF's:
 *  - F16, 64 bytes per 32 weights: little-endian binary16.
 *  - Q4_K, 144 bytes per 256: fp16 d, fp16 dmin, 12 bytes of 6-bit sub-block scales
 *    s_j and mins m_j (j = e / 32; j < 4: low 6 bits of bytes j and j+4; j >= 4: the
 *    nibbles of byte j+4 and the top 2 bits of bytes j-4 and j), 128 bytes of
 *    nibbles (element e: qs[32 (e/64) + e%32], low nibble if e%64 < 32 else high);
 *    value (d s_j) q - dmin m_j.
 *  - Q5_K, 176 bytes per 256: as Q4_K with 32 bytes qh before the nibbles; bit j of
 *    qh[l] adds 16 to element 32 j + l.
 *  - Q6_K, 210 bytes per 256: ql[128], qh[64], 16 int8 scales, fp16 d; element e (h
 *    = e/128, c = e%128/32, l = e%32) takes the low (c < 2) or high nibble of ql[64h
 *    + l + 32 (c%2)] and bits 2c, 2c+1 of qh[32h + l]; value (d sc[8h + l/16 + 2c]) *
 *    (q - 32).
 *  - IQ4_XS, 136 bytes per 256: fp16 d, uint16 scales_h, 4 bytes scales_l, 128 bytes
 *    of codes; sub-block b = e/32 has the 6-bit scale ls (low 4 bits: nibble b%2 of
 *    scales_l[b/2]; top 2: bits 2b, 2b+1 of scales_h); element e takes the low (e%32 <
 *    16) or high nibble of qs[16b + e%16] as its code; value (d (ls - 32)) *
 *    grid[code], grid = {-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53,
 *    69, 89, 113} (GGUF's IQ4_NL values).
 *  Block b of weight row r starts at byte (r * (k/E) + b) * block_bytes, E = 32 or
 *  256 weights per block.
 *
 * Memory and ownership: every pointer is a device pointer (HBM) owned by the
 * caller. The library allocates nothing, frees nothing and keeps no pointer after
 * a call returns. X and Y are f32, contiguous and row-major ([T][k] and [T][n]).
 * Calls only enqueue work on `stream` (a hipStream_t; NULL = the default stream)
 * and never synchronize; a kernel fault shows at the caller's next synchronize.
 *
 * Errors: every argument is checked before anything is launched; a call that
 * returns an error has enqueued nothing and written nothing. Status codes are the
 * PF_* values below; pf_strerror() names them.
 */
#ifndef PF_GEMM_H
#define PF_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Block types. F16 .. IQ4_XS run their own kernels on both legs and need no
 * workspace, except on the f16 leg's GEMM: there pf_gemm_ws runs Q4_K, Q5_K, IQ4_XS and
 * Q6_K (k % 512 == 0) at every T, and F16 above 128 rows, on Q4_0's matrix-core GEMMs
 * (the 4-wave tiles below 256 rows, for Q6_K up to 128, the cooperative-decode kernel
 * from there),
 * with that GEMM's workspace, and elsewhere their own GEMM splits K through the
 * workspace where its tiles leave CUs idle. Without a workspace (pf_gemm, and
 * pf_gemm_noalloc where the workspace exceeds the static scratch) Q4_K, Q5_K, IQ4_XS
 * and Q6_K (k % 512 == 0) run the 4-wave GEMM unsplit, F16 and the other Q6_K rows
 * their own GEMM unsplit. pf_prepare_x and pf_gemm_prepared take Q4_0, Q8_0 and, where
 * pf_gemm_ws runs them on those GEMMs, the further types (else PF_E_QTYPE). */
enum { PF_Q4_0 = 0, PF_Q8_0 = 1, PF_F16 = 2, PF_Q4_K = 3, PF_Q5_K = 4, PF_Q6_K = 5, PF_IQ4_XS = 6 };

/* Epilogues.
 *  PF_PLAIN          Y = X . W_hat^T                      (W has n rows; Y overwritten)
 *  PF_RESIDUAL       Y = Y + X . W_hat^T, in place        (W has n rows; Y holds R on entry)
 *  PF_GATE_UP_SWIGLU Y = silu(X . Wg^T) * (X . Wu^T)      (W has 2n rows: the n gate
 *                    rows, then the n up rows; silu(g) = g / (1 + e^-g))
 */
enum { PF_PLAIN = 0, PF_RESIDUAL = 1, PF_GATE_UP_SWIGLU = 2 };

/* Legs.
 *  PF_LEG_F32  f32 weights (exact decode) and f32 activations, fp32 accumulation.
 *  PF_LEG_F16  weights RNE_fp16(d * (q - 8)) or RNE_fp16(d * q), activations
 *              RNE_fp16(x), fp32 accumulation, f32 output. X stays f32 in memory;
 *              pf_gemm rounds it inside the GEMM, pf_gemm_ws once into its
 *              workspace.
 *  Where the GEMV runs (T <= PF_GEMV_MAX_T, see PF_PATH_AUTO) both legs compute in
 *  f32, whose error bound is the f32 leg's and therefore also meets the f16 leg's.
 *  From 3 rows the Q4_0 / Q8_0 GEMV runs on the fp32 matrix cores (exact f32
 *  operands, f32 accumulation), below on the vector ALU.
 */
enum { PF_LEG_F32 = 0, PF_LEG_F16 = 1 };

/* Kernel family. PF_PATH_AUTO picks the GEMV for 1 <= T <= PF_GEMV_MAX_T and the
 * tiled matrix-core GEMM otherwise, except that for Q4_0, Q8_0, Q4_K, Q5_K, IQ4_XS and
 * Q6_K (k % 512 == 0) the f16 leg takes the GEMM from T = 3 for PLAIN and RESIDUAL and
 * from T = 5 for SwiGLU (faster there through a workspace, whose K split spreads the
 * weight stream over every CU). The other two force a family (tests compare them);
 * PF_PATH_GEMV requires T <= PF_GEMV_MAX_T. */
enum { PF_PATH_AUTO = 0, PF_PATH_GEMM = 1, PF_PATH_GEMV = 2 };
#define PF_GEMV_MAX_T 8

/* Status codes. */
enum {
    PF_OK = 0,
    PF_E_NULL = 1,     /* a required pointer is NULL */
    PF_E_QTYPE = 2,    /* unknown block type (or one the call does not take) */
    PF_E_EPILOGUE = 3, /* unknown epilogue */
    PF_E_LEG = 4,      /* unknown leg */
    PF_E_SHAPE = 5,    /* n < 1, T < 0, k < 256 or k % 256 != 0 (pf_gemm), k not a
                          whole number of blocks (pf_dequant_*, pf_weight_bytes), or
                          an element count of X, Y or W_hat, or W's bytes, reaching
                          2^31 */
    PF_E_ALIGN = 6,    /* W, X, Y or out not 16-byte aligned */
    PF_E_ALIAS = 7,    /* Y (or out) overlaps W or X */
    PF_E_LAUNCH = 8,   /* the HIP runtime refused the launch */
    PF_E_PATH = 9,     /* unknown path, or PF_PATH_GEMV with T > PF_GEMV_MAX_T */
    PF_E_WORKSPACE = 10, /* workspace NULL, smaller than pf_workspace_bytes(), not
                            16-byte aligned, or overlapping W, X or Y */
    PF_E_SCRATCH = 11    /* pf_gemm_noalloc: pf_workspace_bytes() of the call exceeds
                            PF_NOALLOC_SCRATCH_BYTES */
};

/* The projection GEMM.
 *  qtype     PF_Q4_0 or PF_Q8_0.
 *  W_blocks  device, n_w * (k/32) blocks, n_w = 2n for PF_GATE_UP_SWIGLU, else n.
 *  n         output width (columns of Y); k reduction length, a multiple of 256.
 *  X         device, f32 [T][k] row-major. T = 0 is a no-op that returns PF_OK.
 *  Y         device, f32 [T][n] row-major; read as R by PF_RESIDUAL.
 *  epilogue  PF_PLAIN, PF_RESIDUAL or PF_GATE_UP_SWIGLU.
 *  leg       PF_LEG_F32 or PF_LEG_F16.
 *  stream    hipStream_t to enqueue on (NULL = default stream).
 * Deterministic: with no workspace nothing is split across workgroups, so each
 * output element is computed by one workgroup in a fixed order and repeated calls
 * return the same bits. pf_gemm_ws is the faster form where the output alone leaves
 * matrix cores idle (narrow n, short chunks): it splits k through its workspace.
 * Returns PF_OK or a PF_E_* code. */
int pf_gemm(int qtype, const void *W_blocks, int64_t n, int64_t k, const float *X, int64_t T,
            float *Y, int epilogue, int leg, void *stream);

/* pf_gemm with an explicit kernel family (PF_PATH_*); same arguments otherwise. */
int pf_gemm_path(int qtype, const void *W_blocks, int64_t n, int64_t k, const float *X,
                 int64_t T, float *Y, int epilogue, int leg, void *stream, int path);

/* Workspace bytes pf_gemm_ws needs for these sizes, or -PF_E_* for arguments pf_gemm
 * would refuse. Host-only; touches no GPU state.
 *  - 0 when pf_gemm_ws runs a kernel that needs none (the f32 leg, the GEMV, T == 0);
 *  - the further types' own GEMM (where Q4_0's matrix-core GEMMs do not take them):
 *    S * ceil(T * n / 4) * 16 for a K split of PLAIN / RESIDUAL (S > 1), and
 *    S * ceil(T * 2n / 4) * 16 for SwiGLU on up to 64 rows split as a PLAIN GEMM over the
 *    2n gate and up rows; else 0;
 *  - the f16 leg's matrix-core GEMM: X_b = ceil(T / 32) * 32 * k * 2 (X rounded to
 *    binary16, T padded to whole 32-row tiles);
 *  - and where that GEMM splits k across S workgroups (PLAIN or RESIDUAL with too few
 *    output tiles to fill the chip; S is the largest count Q4_0 and Q8_0 take, and for
 *    Q4_K, Q5_K and IQ4_XS their own count):
 *    ceil(X_b / 256) * 256 + S * ceil(T * n / 4) * 16, room for S blocks of [T][n] f32
 *    partial sums;
 *  - the SwiGLU epilogue on up to 64 rows, which runs as a split PLAIN GEMM over the 2n
 *    gate and up rows: ceil(X_b / 256) * 256 + S * ceil(T * 2n / 4) * 16 (S >= 1). */
int64_t pf_workspace_bytes(int qtype, int64_t n, int64_t k, int64_t T, int epilogue, int leg);

/* pf_gemm with a caller workspace. On the f16 leg's matrix-core GEMM, X is first
 * rounded to binary16 once, into the workspace, and the GEMM then streams that copy
 * instead of rounding X again in every tile. The operands (RNE_fp16(x) and the
 * decoded weights) and the accumulation are the same as pf_gemm's, so the result is
 * pf_gemm's, bit for bit wherever this GEMM does not split k across workgroups
 * (pf_gemm never does). Where it splits k, each split stores its partial sums in the
 * workspace and a second kernel adds R (RESIDUAL), then the splits in order: the
 * result is deterministic at every T.
 *  workspace        device, owned by the caller, 16-byte aligned, at least
 *                   pf_workspace_bytes() bytes, not overlapping W, X or Y. Its
 *                   contents on entry are ignored and undefined on return. May be
 *                   NULL when pf_workspace_bytes() is 0.
 *  workspace_bytes  its size in bytes.
 * Calls that share a workspace must be ordered (same stream, or synchronized).
 * Returns PF_OK or a PF_E_* code (PF_E_WORKSPACE for a workspace that is missing,
 * too small, misaligned or overlapping). */
int pf_gemm_ws(int qtype, const void *W_blocks, int64_t n, int64_t k, const float *X, int64_t T,
               float *Y, int epilogue, int leg, void *workspace, int64_t workspace_bytes,
               void *stream);

/* pf_gemm / pf_gemm_ws with a strided Y: row t of the output starts ldy floats after
 * row t-1, so the result can land in a wider destination (a column range of a
 * [T][ldy] buffer, such as one head group's columns of a KV cache) without a copy;
 * the columns between rows are neither read nor written. This is the `ldc >= n` of
 * `qwen35_project_rows` on the page "aprender-serve 0.70.2 -
 * src/cuda/executor/gdn_prefill_ops.rs". A fused projection (the q, k and v weights
 * stacked row-wise in one buffer, as the page "oxibonsai-kernels 0.1.4 -
 * src/gpu_backend/cuda_q_std_prefill.rs" runs its fused QKV GEMM) is one call with n
 * = the stacked row count; ldy then places its output inside a wider row.
 *  ldy        floats between consecutive rows of Y, ldy >= n (ldy == n is pf_gemm).
 *             Y's rows lie in the (T - 1) * ldy + n floats from Y; PF_RESIDUAL reads
 *             R with the same stride. ldy < n, or T * ldy >= 2^31, is PF_E_SHAPE.
 *  workspace  NULL with workspace_bytes 0: as pf_gemm (X rounded inside the GEMM).
 *             Otherwise as pf_gemm_ws: at least pf_workspace_bytes() bytes (the
 *             size does not depend on ldy), 16-byte aligned, overlapping nothing.
 * Other arguments, ownership and errors as pf_gemm / pf_gemm_ws. */
int pf_gemm_ex(int qtype, const void *W_blocks, int64_t n, int64_t k, const float *X, int64_t T,
               float *Y, int64_t ldy, int epilogue, int leg, void *workspace,
               int64_t workspace_bytes, void *stream);

/* The projection with its batched RMSNorm prologue: Y = epilogue(Xn . W_hat^T) where
 * Xn[t][j] = X[t][j] / sqrt(mean_j' X[t][j']^2 + eps) * norm_w[j], the norm that
 * precedes the QKV and gate/up projections on the page "aprender-serve 0.70.2 -
 * src/gguf/cuda/forward_qwen35_cuda_prefill.rs" (`batched_rmsnorm_into`: one weight
 * of k floats for every row, one eps). The mean square and its reciprocal square
 * root are f32; Xn is f32 (then RNE_fp16 on the f16 leg). On the f16 leg's
 * matrix-core GEMM the norm is applied while X is rounded into the workspace, so
 * the normalised rows never go to memory in f32; the GEMV and the f32 leg read Xn
 * from the workspace. X is not modified.
 *  norm_w     device, f32 [k], 16-byte aligned, not overlapping Y.
 *  eps        finite, >= 0 (else PF_E_SHAPE).
 *  Y, ldy     as pf_gemm_ex.
 *  workspace  required (T > 0): device, 16-byte aligned, at least
 *             pf_rmsnorm_workspace_bytes() bytes, overlapping none of W, X, Y,
 *             norm_w; contents ignored on entry, undefined on return.
 * Other arguments, ownership and errors as pf_gemm_ex. */
int pf_gemm_rmsnorm(int qtype, const void *W_blocks, int64_t n, int64_t k, const float *X, int64_t T,
                    const float *norm_w, float eps, float *Y, int64_t ldy, int epilogue, int leg,
                    void *workspace, int64_t workspace_bytes, void *stream);

/* Workspace bytes pf_gemm_rmsnorm needs, or -PF_E_* for sizes pf_gemm would refuse.
 * 0 for T == 0; else ceil(T * 4 / 256) * 256 (the rows' 1 / rms) plus, where
 * pf_gemm_ws would run the f16 leg's matrix-core GEMMs with a workspace (the family
 * PF_PATH_AUTO picks; for the further types where those GEMMs take them),
 * pf_workspace_bytes() for the same sizes, otherwise T * k * 4 (Xn in f32). Host-only. */
int64_t pf_rmsnorm_workspace_bytes(int qtype, int64_t n, int64_t k, int64_t T, int epilogue, int leg);

/* pf_gemm_ws without a caller workspace and without any allocation, for callers that
 * cannot allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid hipMalloc). The workspace is a static device array of
 * PF_NOALLOC_SCRATCH_BYTES in the library, one per GPU, held until the process
 * ends; its address is looked up once per device, at the first call there (that
 * call may load the library's code object on that device). Results equal
 * pf_gemm_ws's bit for bit (the same kernels on the same operands).
 *  - Calls needing more than PF_NOALLOC_SCRATCH_BYTES (pf_workspace_bytes() of the
 *    same arguments) return PF_E_SCRATCH and launch nothing. 64 MiB holds every
 *    shape of the FFN at hidden 4096 / intermediate 12288 up to T = 2048.
 *  - Every call on a GPU shares that GPU's scratch: calls that may overlap on one
 *    GPU (different streams without ordering) race and must be serialised by the
 *    caller. The scratch keeps the last call's contents; no call reads what it
 *    did not write itself, so nothing needs clearing.
 *  - The scratch lives on the device of `stream` (the current device for NULL).
 * Other arguments, ownership and errors as pf_gemm. */
#define PF_NOALLOC_SCRATCH_BYTES (64ll << 20)
int pf_gemm_noalloc(int qtype, const void *W_blocks, int64_t n, int64_t k, const float *X, int64_t T,
                    float *Y, int epilogue, int leg, void *stream);

/* The lm_head step of a prefill: logits = x . W_hat^T for one activation row (the
 * GEMV, f32), then the greedy token, on the device. The page "oxibonsai-kernels 0.1.4 -
 * src/gpu_backend/cuda_q_std_prefill.rs" runs this GEMV on the normed last row and
 * picks the token on the host with Rust's max_by over partial_cmp, the last of equal
 * maxima; here token[0] is the largest index among the maxima of the f32 logits
 * just written (-0 and +0 equal; NaN logits make the pick unspecified).
 *  W_blocks  device, n rows (the vocabulary) of k/32 blocks; k a multiple of 256.
 *  x         device, f32 [k] (e.g. the output of the final RMSNorm), 16-byte aligned.
 *  logits    device, f32 [n], written; 16-byte aligned; overlapping neither W nor x.
 *  token     device, one int32, written; 4-byte aligned; overlapping nothing above.
 * Two launches on the stream (the GEMV, then a one-workgroup pick); nothing is
 * allocated. Returns PF_OK or a PF_E_* code as pf_gemm. */
int pf_lm_head_argmax(int qtype, const void *W_blocks, int64_t n, int64_t k, const float *x,
                      float *logits, int32_t *token, void *stream);

/* The f16 leg's matrix-core GEMM of pf_gemm_ws in two calls, so that one rounding of X
 * serves several projections of the same rows (separate q, k and v weights, say):
 *  pf_prepare_x   rounds X [T][k] (f32, 16-byte aligned) to binary16 into the workspace,
 *                 in the layout the GEMM for (qtype, T) reads; the copy depends on qtype
 *                 (the k order within groups of four follows the block type's decode).
 *                 Needs ceil(T / 32) * 32 * k * 2 bytes of workspace.
 *  pf_gemm_prepared  the GEMM on that copy: Y = epilogue(X . W_hat^T) with Y, ldy as
 *                 pf_gemm_ex; the workspace must hold pf_workspace_bytes(qtype, n, k, T,
 *                 epilogue, PF_LEG_F16) bytes and its first part a pf_prepare_x copy for
 *                 the same qtype, k and T, enqueued before it on the same stream (or
 *                 synchronised). The GEMM reads the copy and writes only past it (split-K
 *                 partial sums), so the copy stays valid for further calls.
 * The result is pf_gemm_ws's, bit for bit. pf_gemm_prepared
 * returns PF_E_PATH where PF_PATH_AUTO picks the GEMV for the f16 leg (which reads f32 X:
 * T <= 2, or T <= 4 with the SwiGLU epilogue); T == 0 is a no-op. Other
 * errors as pf_gemm_ws. */
int pf_prepare_x(int qtype, int64_t k, const float *X, int64_t T, void *workspace, int64_t workspace_bytes,
                 void *stream);
int pf_gemm_prepared(int qtype, const void *W_blocks, int64_t n, int64_t k, int64_t T, float *Y, int64_t ldy,
                     int epilogue, void *workspace, int64_t workspace_bytes, void *stream);

/* Which family pf_gemm would run for these sizes: PF_PATH_GEMM, PF_PATH_GEMV, 0
 * for T == 0 (nothing runs), or -PF_E_* for arguments pf_gemm would refuse
 * (pointers are not checked). Host-only; touches no GPU state. */
int pf_select_path(int qtype, int64_t n, int64_t k, int64_t T, int epilogue, int leg);

/* Bit-exact block decode into out[rows][k] (device, f32): d * (q - 8), d * q, or the
 * value each further type defines (see the block formats above). Same block layout
 * as pf_gemm; k a whole number of blocks. This is the f32 leg's weight. */
int pf_dequant_f32(int qtype, const void *W_blocks, int64_t rows, int64_t k, float *out,
                   void *stream);

/* Block decode into binary16 bit patterns out[rows][k] (device): RNE_fp16 of the f32
 * decode. This is the f16 leg's weight. */
int pf_dequant_f16(int qtype, const void *W_blocks, int64_t rows, int64_t k, uint16_t *out,
                   void *stream);

/* Bytes of a weight of `rows` rows and reduction length k: rows * (k/E) *
 * block_bytes (see the block formats above). Returns -PF_E_QTYPE or -PF_E_SHAPE (k
 * not a multiple of E, rows < 0) on bad arguments. Host-only. */
int64_t pf_weight_bytes(int qtype, int64_t rows, int64_t k);

/* Static, NUL-terminated name of a status code ("unknown status" otherwise). */
const char *pf_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* PF_GEMM_H */
