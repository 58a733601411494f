// The C ABI: argument checks, then dispatch to one kernel launch on the caller's
// stream. Every check runs on the host before any HIP call, so a refused call
// enqueues nothing and touches no GPU state (the refusal style of the page
// "aprender-serve 0.70.2 - src/gguf/cuda/forward_qwen35_cuda_prefill.rs",
// `prefill`: refuse with a reason, leave nothing half applied; null pointers are
// refused as `qp_launch` on "aprender-serve 0.70.2 -
// src/cuda/executor/gdn_prefill_ops.rs" does, and an unknown block type as in
// `qwen35_dequant_f32` there).
#include <stdint.h>

#include <cmath>

#include "../../include/pf_gemm.h"
#include "pf_internal.h"

namespace {

constexpr int64_t kMax31 = (int64_t(1) << 31) - 1;

// Bytes and weights of one block of each type (the K types' super-blocks hold 256).
int block_bytes(int qtype) {
    switch (qtype) {
    case PF_Q4_0: return 18;
    case PF_Q8_0: return 34;
    case PF_F16: return 64;
    case PF_Q4_K: return 144;
    case PF_Q5_K: return 176;
    case PF_Q6_K: return 210;
    case PF_IQ4_XS: return 136;
    default: return -1;
    }
}
int block_elems(int qtype) { return (qtype >= PF_Q4_K && qtype <= PF_IQ4_XS) ? 256 : 32; }
// The further types (F16, Q4_K, Q5_K, Q6_K, IQ4_XS) run their own kernels (pf_xq.hip), except
// where the f16 leg's matrix-core GEMMs decode them (pf::f16_takes_xq with a workspace,
// pf::f16_direct_takes_xq without); on the f16 leg their own GEMM splits K through the
// workspace where its tiles leave CUs idle.
bool is_xq(int qtype) { return qtype >= PF_F16 && qtype <= PF_IQ4_XS; }
int64_t w_bytes_of(int qtype, int64_t rows, int64_t k) { return rows * (k / block_elems(qtype)) * block_bytes(qtype); }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void *a, int64_t a_bytes, const void *b, int64_t b_bytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a_bytes > 0 && b_bytes > 0 && a0 < b0 + (uintptr_t)b_bytes && b0 < a0 + (uintptr_t)a_bytes;
}

// Checks that need no pointers. On success stores the weight row count.
int check_sizes(int qtype, int64_t n, int64_t k, int64_t T, int epilogue, int leg, int64_t *n_w) {
    if (block_bytes(qtype) < 0) return PF_E_QTYPE;
    if (epilogue != PF_PLAIN && epilogue != PF_RESIDUAL && epilogue != PF_GATE_UP_SWIGLU)
        return PF_E_EPILOGUE;
    if (leg != PF_LEG_F32 && leg != PF_LEG_F16) return PF_E_LEG;
    if (n < 1 || T < 0 || k < 256 || k % 256 != 0) return PF_E_SHAPE;
    const int64_t rows = epilogue == PF_GATE_UP_SWIGLU ? 2 * n : n;
    // Element counts stay below 2^31 so that 32-bit index arithmetic is exact.
    if (k > kMax31 / rows || (T > 0 && (k > kMax31 / T || n > kMax31 / T))) return PF_E_SHAPE;
    if ((rows * (k / block_elems(qtype))) > kMax31 / block_bytes(qtype)) return PF_E_SHAPE;
    *n_w = rows;
    return PF_OK;
}

// Kernel family of PF_PATH_AUTO for T >= 1 rows. The GEMV up to PF_GEMV_MAX_T rows,
// except on the f16 leg from 3 rows for PLAIN and RESIDUAL and from 5 for SwiGLU:
// there the matrix-core GEMM's 32-row tile, split along K over every CU, streams the
// weights faster than the GEMV (whose time grows with each pair of rows). SwiGLU
// splits K only through a workspace, so its crossing comes later (gate/up 2 x 12288 x
// 4096: GEMV 36 us at 4 rows and 54 at 6, GEMM 43 unsplit or 28 through a workspace).
// The further types that the f16 leg's 4-wave GEMM takes (Q4_K, Q5_K, IQ4_XS, Q6_K with
// k % 512 == 0) cross over at the same row counts (their GEMVs are slower than Q4_0's:
// down 4096 x 12288 Q4_K at T = 4 through a workspace 56.8 -> 20.0 us, gate/up T = 8
// 70.1 -> 29.6; PLAIN 12288 x 4096 at T = 3 gives up 2 us, Q6_K's 12 at T = 3 and 8 at
// T = 4); F16 and the other Q6_K rows take the GEMV up to PF_GEMV_MAX_T rows on both legs.
int auto_path(int qtype, int64_t k, int64_t T, int epilogue, int leg) {
    if (T > PF_GEMV_MAX_T) return PF_PATH_GEMM;
    if ((!is_xq(qtype) || pf::f16_direct_takes_xq(qtype, (int)k)) && leg == PF_LEG_F16 &&
        T >= (epilogue == PF_GATE_UP_SWIGLU ? 5 : 3))
        return PF_PATH_GEMM;
    return PF_PATH_GEMV;
}

// The Q4_0 / Q8_0 GEMV: from 3 tokens on the fp32 matrix cores, else on the vector
// ALU (both compute in f32 on either leg). The vector-ALU form spends an FMA and an LDS
// read of x per weight and token, which from about 3 tokens costs more than the matrix
// cores' fixed decode (measured on Q4_0 12288 x 4096: T = 4 20.3 -> 15.7 us, T = 8
// 38.3 -> 20.6 us; at T = 2 12.5 against 15.0). On the f16 leg the GEMV runs up to 4
// rows, for SwiGLU only (auto_path).
hipError_t launch_gemv_q(const pf::GemmArgs &a, int leg, hipStream_t s) {
    (void)leg;
    return a.T >= 3 ? pf::launch_gemv_mfma(a, s) : pf::launch_gemv(a, s);
}

// Bytes of workspace the f16 leg's GEMM takes (X as binary16, T rounded up to a
// multiple of 32 for the fragment-ordered copy, plus the partial sums of a K split),
// else 0.
int64_t ws_need(int qtype, int64_t n, int64_t k, int64_t T, int epilogue, int leg, int use) {
    if (use != PF_PATH_GEMM || leg != PF_LEG_F16) return 0;
    if (!is_xq(qtype) || pf::f16_takes_xq(qtype, (int)T, (int)k))
        return pf::f16_ws_bytes(qtype, (int)T, (int)n, (int)k, epilogue);
    return pf::xq_ws_bytes((int)T, (int)n, (int)k, epilogue, true);  // their own GEMM's K split
}

// Where a call's workspace comes from: none (the kernels that need none, or the
// f16 GEMM rounding X inside itself), the caller, or the static device scratch.
enum WsMode { WS_NONE = 0, WS_CALLER = 1, WS_STATIC = 2 };

int gemm_impl(int qtype, const void *W, int64_t n, int64_t k, const float *X, int64_t T, float *Y,
              int64_t ldy, int epilogue, int leg, void *stream, int path, int ws_mode, void *ws,
              int64_t ws_bytes) {
    int64_t n_w = 0;
    int st = check_sizes(qtype, n, k, T, epilogue, leg, &n_w);
    if (st != PF_OK) return st;
    if (ldy < n || (T > 0 && ldy > kMax31 / T)) return PF_E_SHAPE;
    if (path != PF_PATH_AUTO && path != PF_PATH_GEMM && path != PF_PATH_GEMV) return PF_E_PATH;
    if (path == PF_PATH_GEMV && T > PF_GEMV_MAX_T) return PF_E_PATH;
    if (T == 0) return PF_OK;  // an empty batch is a no-op
    if (!W || !X || !Y) return PF_E_NULL;
    if (!aligned16(W) || !aligned16(X) || !aligned16(Y)) return PF_E_ALIGN;
    const int64_t w_bytes = w_bytes_of(qtype, n_w, k);
    const int64_t x_bytes = T * k * 4, y_bytes = ((T - 1) * ldy + n) * 4;  // Y's rows and gaps
    if (overlap(Y, y_bytes, X, x_bytes) || overlap(Y, y_bytes, W, w_bytes)) return PF_E_ALIAS;
    const int use = path == PF_PATH_AUTO ? auto_path(qtype, k, T, epilogue, leg) : path;
    int64_t need = ws_mode != WS_NONE ? ws_need(qtype, n, k, T, epilogue, leg, use) : 0;
    // A further type whose workspace would not fit the static scratch runs as it does
    // without a workspace (the 4-wave GEMM unsplit, or its own GEMM), which needs none.
    if (ws_mode == WS_STATIC && is_xq(qtype) && need > pf::kNoallocScratchBytes) need = 0;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (need > 0 && ws_mode == WS_STATIC) {
        // every check is done: the first HIP call of the request
        if (need > pf::kNoallocScratchBytes) return PF_E_SCRATCH;
        if (pf::noalloc_scratch(s, &ws) != hipSuccess) return PF_E_LAUNCH;
        ws_bytes = pf::kNoallocScratchBytes;
    } else if (need > 0) {
        if (!ws || ws_bytes < need || !aligned16(ws)) return PF_E_WORKSPACE;
        if (overlap(ws, need, W, w_bytes) || overlap(ws, need, X, x_bytes) ||
            overlap(ws, need, Y, y_bytes))
            return PF_E_WORKSPACE;
    }

    pf::GemmArgs a;
    a.qtype = qtype;
    a.epilogue = epilogue;
    a.W = static_cast<const uint8_t *>(W);
    a.X = X;
    a.Y = Y;
    a.n = (int)n;
    a.ldy = (int)ldy;
    a.k = (int)k;
    a.T = (int)T;
    hipError_t err;
    // The further types on the f16 leg's matrix-core GEMMs, where those take them (with
    // the workspace, or without it on the 4-wave kernel); else their own kernels.
    const bool xq_f16 = use == PF_PATH_GEMM && leg == PF_LEG_F16 &&
                        (need > 0 ? pf::f16_takes_xq(qtype, (int)T, (int)k) : pf::f16_direct_takes_xq(qtype, (int)k));
    if (is_xq(qtype) && !xq_f16)
        err = use == PF_PATH_GEMV ? pf::launch_xq_gemv(a, s)
                                  : pf::launch_xq_gemm(a, leg == PF_LEG_F16, need > 0 ? ws : nullptr, s);
    else if (use == PF_PATH_GEMV)
        err = launch_gemv_q(a, leg, s);
    else if (leg == PF_LEG_F32)
        err = pf::launch_gemm_f32(a, s);
    else if (need > 0)
        err = pf::launch_gemm_f16_ws(a, ws, s);
    else
        err = pf::launch_gemm_f16(a, s);
    return err == hipSuccess ? PF_OK : PF_E_LAUNCH;
}

int64_t round256(int64_t b) { return (b + 255) / 256 * 256; }

// Whether the RMSNorm entry point applies the norm inside the f16 leg GEMM's conversion
// of X to binary16 (Q4_0, Q8_0 and the further types those GEMMs take), rather than
// materialising Xn for a kernel that reads f32 X.
bool rms_fused(int qtype, int64_t k, int64_t T, int leg, int use) {
    return use == PF_PATH_GEMM && leg == PF_LEG_F16 && (!is_xq(qtype) || pf::f16_takes_xq(qtype, (int)T, (int)k));
}

// Workspace of the RMSNorm entry point: inv[T] (rounded up to 256 bytes), then the
// f16 GEMM's own workspace (X rounded to binary16 with the norm applied, and any
// split-K partial sums), or, for the kernels that read f32 X, Xn [T][k] f32.
int64_t rms_ws_need(int qtype, int64_t n, int64_t k, int64_t T, int epilogue, int leg, int use) {
    if (T == 0) return 0;
    const int64_t tail = rms_fused(qtype, k, T, leg, use) ? pf::f16_ws_bytes(qtype, (int)T, (int)n, (int)k, epilogue)
                                                          : T * k * 4;
    return round256(T * 4) + tail;
}

int rms_impl(int qtype, const void *W, int64_t n, int64_t k, const float *X, int64_t T,
             const float *norm_w, float eps, float *Y, int64_t ldy, int epilogue, int leg, void *ws,
             int64_t ws_bytes, void *stream) {
    int64_t n_w = 0;
    int st = check_sizes(qtype, n, k, T, epilogue, leg, &n_w);
    if (st != PF_OK) return st;
    if (ldy < n || (T > 0 && ldy > kMax31 / T)) return PF_E_SHAPE;
    if (!(eps >= 0.f) || !std::isfinite(eps)) return PF_E_SHAPE;
    if (T == 0) return PF_OK;  // an empty batch is a no-op
    if (!W || !X || !Y || !norm_w) return PF_E_NULL;
    if (!aligned16(W) || !aligned16(X) || !aligned16(Y) || !aligned16(norm_w)) return PF_E_ALIGN;
    const int64_t w_bytes = w_bytes_of(qtype, n_w, k);
    const int64_t x_bytes = T * k * 4, y_bytes = ((T - 1) * ldy + n) * 4, nw_bytes = k * 4;
    if (overlap(Y, y_bytes, X, x_bytes) || overlap(Y, y_bytes, W, w_bytes) ||
        overlap(Y, y_bytes, norm_w, nw_bytes))
        return PF_E_ALIAS;
    const int use = auto_path(qtype, k, T, epilogue, leg);
    const int64_t need = rms_ws_need(qtype, n, k, T, epilogue, leg, use);
    if (!ws || ws_bytes < need || !aligned16(ws)) return PF_E_WORKSPACE;
    if (overlap(ws, need, W, w_bytes) || overlap(ws, need, X, x_bytes) || overlap(ws, need, Y, y_bytes) ||
        overlap(ws, need, norm_w, nw_bytes))
        return PF_E_WORKSPACE;

    pf::GemmArgs a;
    a.qtype = qtype;
    a.epilogue = epilogue;
    a.W = static_cast<const uint8_t *>(W);
    a.X = X;
    a.Y = Y;
    a.n = (int)n;
    a.ldy = (int)ldy;
    a.k = (int)k;
    a.T = (int)T;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    float *inv = static_cast<float *>(ws);
    uint8_t *rest = static_cast<uint8_t *>(ws) + round256(T * 4);
    hipError_t err = pf::launch_rms_inv(X, a.T, a.k, eps, inv, s);
    if (err != hipSuccess) return PF_E_LAUNCH;
    if (rms_fused(qtype, k, T, leg, use)) {
        a.norm_inv = inv;
        a.norm_w = norm_w;
        err = pf::launch_gemm_f16_ws(a, rest, s);
    } else {
        float *Xn = reinterpret_cast<float *>(rest);
        err = pf::launch_rms_apply(X, inv, norm_w, Xn, a.T, a.k, s);
        if (err != hipSuccess) return PF_E_LAUNCH;
        a.X = Xn;
        if (is_xq(qtype))
            err = use == PF_PATH_GEMV ? pf::launch_xq_gemv(a, s) : pf::launch_xq_gemm(a, leg == PF_LEG_F16, nullptr, s);
        else
            err = use == PF_PATH_GEMV ? launch_gemv_q(a, leg, s) : pf::launch_gemm_f32(a, s);
    }
    return err == hipSuccess ? PF_OK : PF_E_LAUNCH;
}

int dequant_check(int qtype, const void *W, int64_t rows, int64_t k, const void *out, int out_elem) {
    if (block_bytes(qtype) < 0) return PF_E_QTYPE;
    const int be = block_elems(qtype);
    if (rows < 1 || k < be || k % be != 0) return PF_E_SHAPE;
    if (k > kMax31 / rows || (rows * (k / be)) > kMax31 / block_bytes(qtype)) return PF_E_SHAPE;
    if (!W || !out) return PF_E_NULL;
    if (!aligned16(W) || !aligned16(out)) return PF_E_ALIGN;
    if (overlap(out, rows * k * out_elem, W, w_bytes_of(qtype, rows, k))) return PF_E_ALIAS;
    return PF_OK;
}

}  // namespace

extern "C" {

int pf_gemm(int qtype, const void *W_blocks, int64_t n, int64_t k, const float *X, int64_t T,
            float *Y, int epilogue, int leg, void *stream) {
    return gemm_impl(qtype, W_blocks, n, k, X, T, Y, n, epilogue, leg, stream, PF_PATH_AUTO, WS_NONE,
                     nullptr, 0);
}

int pf_gemm_noalloc(int qtype, const void *W_blocks, int64_t n, int64_t k, const float *X, int64_t T,
                    float *Y, int epilogue, int leg, void *stream) {
    return gemm_impl(qtype, W_blocks, n, k, X, T, Y, n, epilogue, leg, stream, PF_PATH_AUTO, WS_STATIC,
                     nullptr, 0);
}

int pf_gemm_ex(int qtype, const void *W_blocks, int64_t n, int64_t k, const float *X, int64_t T,
               float *Y, int64_t ldy, int epilogue, int leg, void *workspace,
               int64_t workspace_bytes, void *stream) {
    const bool with_ws = workspace != nullptr || workspace_bytes != 0;
    return gemm_impl(qtype, W_blocks, n, k, X, T, Y, ldy, epilogue, leg, stream, PF_PATH_AUTO,
                     with_ws ? WS_CALLER : WS_NONE, workspace, workspace_bytes);
}

int pf_gemm_ws(int qtype, const void *W_blocks, int64_t n, int64_t k, const float *X, int64_t T,
               float *Y, int epilogue, int leg, void *workspace, int64_t workspace_bytes,
               void *stream) {
    return gemm_impl(qtype, W_blocks, n, k, X, T, Y, n, epilogue, leg, stream, PF_PATH_AUTO, WS_CALLER,
                     workspace, workspace_bytes);
}

int pf_gemm_rmsnorm(int qtype, const void *W_blocks, int64_t n, int64_t k, const float *X, int64_t T,
                    const float *norm_w, float eps, float *Y, int64_t ldy, int epilogue, int leg,
                    void *workspace, int64_t workspace_bytes, void *stream) {
    return rms_impl(qtype, W_blocks, n, k, X, T, norm_w, eps, Y, ldy, epilogue, leg, workspace,
                    workspace_bytes, stream);
}

int pf_lm_head_argmax(int qtype, const void *W_blocks, int64_t n, int64_t k, const float *x,
                      float *logits, int32_t *token, void *stream) {
    int64_t n_w = 0;
    const int st = check_sizes(qtype, n, k, 1, PF_PLAIN, PF_LEG_F32, &n_w);
    if (st != PF_OK) return st;
    if (!W_blocks || !x || !logits || !token) return PF_E_NULL;
    if (!aligned16(W_blocks) || !aligned16(x) || !aligned16(logits) ||
        (reinterpret_cast<uintptr_t>(token) & 3u) != 0)
        return PF_E_ALIGN;
    const int64_t w_bytes = w_bytes_of(qtype, n_w, k), x_bytes = k * 4, l_bytes = n * 4;
    if (overlap(logits, l_bytes, W_blocks, w_bytes) || overlap(logits, l_bytes, x, x_bytes) ||
        overlap(token, 4, logits, l_bytes) || overlap(token, 4, W_blocks, w_bytes) ||
        overlap(token, 4, x, x_bytes))
        return PF_E_ALIAS;
    pf::GemmArgs a;
    a.qtype = qtype;
    a.epilogue = PF_PLAIN;
    a.W = static_cast<const uint8_t *>(W_blocks);
    a.X = x;
    a.Y = logits;
    a.n = (int)n;
    a.ldy = (int)n;
    a.k = (int)k;
    a.T = 1;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if ((is_xq(qtype) ? pf::launch_xq_gemv(a, s) : pf::launch_gemv(a, s)) != hipSuccess) return PF_E_LAUNCH;
    return pf::launch_argmax(logits, (int)n, token, s) == hipSuccess ? PF_OK : PF_E_LAUNCH;
}

int pf_prepare_x(int qtype, int64_t k, const float *X, int64_t T, void *workspace, int64_t workspace_bytes,
                 void *stream) {
    if (block_bytes(qtype) < 0) return PF_E_QTYPE;
    if (T < 0 || k < 256 || k % 256 != 0 || (T > 0 && k > kMax31 / T)) return PF_E_SHAPE;
    // the further types have a prepared form where the f16 GEMMs take them
    if (is_xq(qtype) && T > 0 && !pf::f16_takes_xq(qtype, (int)T, (int)k)) return PF_E_QTYPE;
    if (T == 0) return PF_OK;
    if (!X) return PF_E_NULL;
    if (!aligned16(X)) return PF_E_ALIGN;
    const int64_t need = (T + 31) / 32 * 32 * k * 2;
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return PF_E_WORKSPACE;
    if (overlap(workspace, need, X, T * k * 4)) return PF_E_WORKSPACE;
    pf::GemmArgs a;
    a.qtype = qtype;
    a.epilogue = PF_PLAIN;
    a.W = nullptr;
    a.X = X;
    a.Y = nullptr;
    a.n = 1;
    a.ldy = 1;
    a.k = (int)k;
    a.T = (int)T;
    return pf::launch_prepare_x_f16(a, workspace, static_cast<hipStream_t>(stream)) == hipSuccess
               ? PF_OK
               : PF_E_LAUNCH;
}

int pf_gemm_prepared(int qtype, const void *W_blocks, int64_t n, int64_t k, int64_t T, float *Y, int64_t ldy,
                     int epilogue, void *workspace, int64_t workspace_bytes, void *stream) {
    int64_t n_w = 0;
    const int st = check_sizes(qtype, n, k, T, epilogue, PF_LEG_F16, &n_w);
    if (st != PF_OK) return st;
    // the further types' own GEMM reads f32 X: a prepared form only where the f16 GEMMs
    // take them
    if (is_xq(qtype) && T > 0 && !pf::f16_takes_xq(qtype, (int)T, (int)k)) return PF_E_QTYPE;
    if (ldy < n || (T > 0 && ldy > kMax31 / T)) return PF_E_SHAPE;
    // where pf_gemm_ws would run the GEMV (which reads f32 X) there is no prepared form
    if (T > 0 && auto_path(qtype, k, T, epilogue, PF_LEG_F16) != PF_PATH_GEMM) return PF_E_PATH;
    if (T == 0) return PF_OK;
    if (!W_blocks || !Y) return PF_E_NULL;
    if (!aligned16(W_blocks) || !aligned16(Y)) return PF_E_ALIGN;
    const int64_t w_bytes = w_bytes_of(qtype, n_w, k), y_bytes = ((T - 1) * ldy + n) * 4;
    if (overlap(Y, y_bytes, W_blocks, w_bytes)) return PF_E_ALIAS;
    const int64_t need = pf::f16_ws_bytes(qtype, (int)T, (int)n, (int)k, epilogue);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return PF_E_WORKSPACE;
    if (overlap(workspace, need, W_blocks, w_bytes) || overlap(workspace, need, Y, y_bytes))
        return PF_E_WORKSPACE;
    pf::GemmArgs a;
    a.qtype = qtype;
    a.epilogue = epilogue;
    a.W = static_cast<const uint8_t *>(W_blocks);
    a.X = nullptr;
    a.Y = Y;
    a.n = (int)n;
    a.ldy = (int)ldy;
    a.k = (int)k;
    a.T = (int)T;
    return pf::launch_gemm_f16_prepared(a, workspace, static_cast<hipStream_t>(stream)) == hipSuccess
               ? PF_OK
               : PF_E_LAUNCH;
}

int64_t pf_rmsnorm_workspace_bytes(int qtype, int64_t n, int64_t k, int64_t T, int epilogue, int leg) {
    int64_t n_w = 0;
    const int st = check_sizes(qtype, n, k, T, epilogue, leg, &n_w);
    if (st != PF_OK) return -st;
    return rms_ws_need(qtype, n, k, T, epilogue, leg, auto_path(qtype, k, T, epilogue, leg));
}

int64_t pf_workspace_bytes(int qtype, int64_t n, int64_t k, int64_t T, int epilogue, int leg) {
    int64_t n_w = 0;
    const int st = check_sizes(qtype, n, k, T, epilogue, leg, &n_w);
    if (st != PF_OK) return -st;
    if (T == 0) return 0;
    return ws_need(qtype, n, k, T, epilogue, leg, auto_path(qtype, k, T, epilogue, leg));
}

int pf_gemm_path(int qtype, const void *W_blocks, int64_t n, int64_t k, const float *X,
                 int64_t T, float *Y, int epilogue, int leg, void *stream, int path) {
    return gemm_impl(qtype, W_blocks, n, k, X, T, Y, n, epilogue, leg, stream, path, WS_NONE, nullptr, 0);
}

int pf_select_path(int qtype, int64_t n, int64_t k, int64_t T, int epilogue, int leg) {
    int64_t n_w = 0;
    const int st = check_sizes(qtype, n, k, T, epilogue, leg, &n_w);
    if (st != PF_OK) return -st;
    if (T == 0) return 0;
    return auto_path(qtype, k, T, epilogue, leg);
}

int pf_dequant_f32(int qtype, const void *W_blocks, int64_t rows, int64_t k, float *out,
                   void *stream) {
    const int st = dequant_check(qtype, W_blocks, rows, k, out, 4);
    if (st != PF_OK) return st;
    const hipError_t err =
        is_xq(qtype) ? pf::launch_xq_dequant(qtype, static_cast<const uint8_t *>(W_blocks), (int)rows, (int)k, out,
                                             false, static_cast<hipStream_t>(stream))
                     : pf::launch_dequant_f32(qtype, static_cast<const uint8_t *>(W_blocks), (int)rows, (int)k, out,
                                              static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PF_OK : PF_E_LAUNCH;
}

int pf_dequant_f16(int qtype, const void *W_blocks, int64_t rows, int64_t k, uint16_t *out,
                   void *stream) {
    const int st = dequant_check(qtype, W_blocks, rows, k, out, 2);
    if (st != PF_OK) return st;
    const hipError_t err =
        is_xq(qtype) ? pf::launch_xq_dequant(qtype, static_cast<const uint8_t *>(W_blocks), (int)rows, (int)k, out,
                                             true, static_cast<hipStream_t>(stream))
                     : pf::launch_dequant_f16(qtype, static_cast<const uint8_t *>(W_blocks), (int)rows, (int)k, out,
                                              static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PF_OK : PF_E_LAUNCH;
}

int64_t pf_weight_bytes(int qtype, int64_t rows, int64_t k) {
    const int bb = block_bytes(qtype);
    if (bb < 0) return -PF_E_QTYPE;
    if (rows < 0 || k < 0 || k % block_elems(qtype) != 0) return -PF_E_SHAPE;
    return w_bytes_of(qtype, rows, k);
}

const char *pf_strerror(int status) {
    switch (status) {
    case PF_OK: return "PF_OK: success";
    case PF_E_NULL: return "PF_E_NULL: a required pointer is NULL";
    case PF_E_QTYPE: return "PF_E_QTYPE: unknown block type";
    case PF_E_EPILOGUE: return "PF_E_EPILOGUE: unknown epilogue";
    case PF_E_LEG: return "PF_E_LEG: unknown leg";
    case PF_E_SHAPE: return "PF_E_SHAPE: unsupported shape";
    case PF_E_ALIGN: return "PF_E_ALIGN: pointer not 16-byte aligned";
    case PF_E_ALIAS: return "PF_E_ALIAS: output overlaps an input";
    case PF_E_LAUNCH: return "PF_E_LAUNCH: kernel launch failed";
    case PF_E_PATH: return "PF_E_PATH: unknown path or GEMV with T > 8";
    case PF_E_WORKSPACE: return "PF_E_WORKSPACE: workspace missing, too small, misaligned or overlapping";
    case PF_E_SCRATCH: return "PF_E_SCRATCH: the call needs more than the static scratch holds";
    default: return "unknown status";
    }
}

}  // extern "C"
