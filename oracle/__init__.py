"""CPU oracle for the quantized-weight prefill GEMM — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product (the HIP library and its Python
binding) never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, no FMA contraction). This
module only marshals numpy arrays through ctypes. See ``oracle.c`` for the
passages each function follows. ``tolerance.py`` holds the pass/fail rules. The
batched RMSNorm prologue (``rmsnorm``) and the GEMM on its fp64 output
(``matmul_f64``) are plain numpy fp64 here.
"""
import ctypes
import os

import numpy as np

from . import build as _build

Q4_0, Q8_0, F16, Q4_K, Q5_K, Q6_K, IQ4_XS = 0, 1, 2, 3, 4, 5, 6
PLAIN, RESIDUAL, GATE_UP_SWIGLU = 0, 1, 2
BLOCK_BYTES = {Q4_0: 18, Q8_0: 34, F16: 64, Q4_K: 144, Q5_K: 176, Q6_K: 210, IQ4_XS: 136}
BLOCK_ELEMS = {Q4_0: 32, Q8_0: 32, F16: 32, Q4_K: 256, Q5_K: 256, Q6_K: 256, IQ4_XS: 256}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = _build.LIB
    if not os.path.exists(path):
        _build.build()
    lib = ctypes.CDLL(path)
    i64, u16 = ctypes.c_int64, ctypes.c_uint16
    P = ctypes.c_void_p
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_fp16_to_f64.argtypes = [u16]
    lib.oracle_fp16_to_f64.restype = ctypes.c_double
    lib.oracle_f32_to_fp16_rne.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_fp16_rne.restype = u16
    lib.oracle_fp16_decode_array.argtypes = [P, i64, P]
    lib.oracle_f32_to_fp16_array.argtypes = [P, i64, P]
    lib.oracle_block_bytes.argtypes = [ctypes.c_int]
    lib.oracle_block_bytes.restype = ctypes.c_int
    lib.oracle_dequant_f32.argtypes = [ctypes.c_int, P, i64, i64, P]
    lib.oracle_dequant_f16.argtypes = [ctypes.c_int, P, i64, i64, P]
    lib.oracle_matmul.argtypes = [ctypes.c_int, P, i64, i64, P, i64, P]
    lib.oracle_matmul_sampled.argtypes = [ctypes.c_int, P, i64, i64, P, i64, P, P, i64, P]
    lib.oracle_row_norms.argtypes = [ctypes.c_int, P, i64, i64, P]
    lib.oracle_silu.argtypes = [ctypes.c_double]
    lib.oracle_silu.restype = ctypes.c_double
    lib.oracle_epilogue.argtypes = [ctypes.c_int, P, i64, i64, P, P]
    lib.oracle_gemm.argtypes = [ctypes.c_int, P, i64, i64, P, i64, P, ctypes.c_int, P]
    _lib = lib
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def num_threads():
    """OpenMP threads the oracle runs on."""
    return int(_load().oracle_num_threads())


def fp16_to_f64(h):
    """Decode binary16 bit patterns (uint16 array) to fp64, from the definition."""
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float64)
    _load().oracle_fp16_decode_array(_ptr(h), h.size, _ptr(out))
    return out


def f32_to_fp16(x):
    """Round f32 values to binary16 bit patterns (RNE), from the definition."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().oracle_f32_to_fp16_array(_ptr(x), x.size, _ptr(out))
    return out


def _check_blocks(qtype, W, rows, k):
    W = _c(W, np.uint8).reshape(-1)
    be = BLOCK_ELEMS[qtype]
    need = rows * (k // be) * BLOCK_BYTES[qtype]
    if k % be or W.size < need:
        raise ValueError("weight buffer does not hold %d rows of k=%d" % (rows, k))
    return W


def dequant_f32(qtype, W, rows, k):
    """W_hat [rows][k] f32: the exact decode of each block."""
    W = _check_blocks(qtype, W, rows, k)
    out = np.empty((rows, k), np.float32)
    _load().oracle_dequant_f32(qtype, _ptr(W), rows, k, _ptr(out))
    return out


def dequant_f16(qtype, W, rows, k):
    """f16-leg weights [rows][k] as binary16 bit patterns: RNE(decode)."""
    W = _check_blocks(qtype, W, rows, k)
    out = np.empty((rows, k), np.uint16)
    _load().oracle_dequant_f16(qtype, _ptr(W), rows, k, _ptr(out))
    return out


def matmul(qtype, W, rows, k, X):
    """fp64 X . W_hat^T, shape [T][rows]."""
    W = _check_blocks(qtype, W, rows, k)
    X = _c(X, np.float32).reshape(-1, k)
    T = X.shape[0]
    out = np.empty((T, rows), np.float64)
    _load().oracle_matmul(qtype, _ptr(W), rows, k, _ptr(X), T, _ptr(out))
    return out


def matmul_sampled(qtype, W, rows, k, X, ti, ri):
    """fp64 sum_k W_hat[ri[i]][k] * X[ti[i]][k] for chosen pairs."""
    W = _check_blocks(qtype, W, rows, k)
    X = _c(X, np.float32).reshape(-1, k)
    ti = _c(ti, np.int64)
    ri = _c(ri, np.int64)
    if ti.shape != ri.shape:
        raise ValueError("index arrays differ in shape")
    if ti.size and (ti.min() < 0 or ti.max() >= X.shape[0] or ri.min() < 0 or ri.max() >= rows):
        raise ValueError("sample index out of range")
    out = np.empty(ti.shape, np.float64)
    _load().oracle_matmul_sampled(qtype, _ptr(W), rows, k, _ptr(X), X.shape[0],
                                  _ptr(ti), _ptr(ri), ti.size, _ptr(out))
    return out


def row_norms(qtype, W, rows, k):
    """||W_hat[r]||_2 in fp64."""
    W = _check_blocks(qtype, W, rows, k)
    out = np.empty(rows, np.float64)
    _load().oracle_row_norms(qtype, _ptr(W), rows, k, _ptr(out))
    return out


def silu(g):
    """Textbook SiLU g / (1 + e^-g) in fp64 (scalar or array)."""
    lib = _load()
    g = np.asarray(g, np.float64)
    return np.vectorize(lib.oracle_silu, otypes=[np.float64])(g)


def epilogue(epi, acc, n, R=None):
    """Apply an epilogue to fp64 products acc [T][rows]; returns Y [T][n] fp64."""
    acc = _c(acc, np.float64)
    T = acc.shape[0]
    rows = 2 * n if epi == GATE_UP_SWIGLU else n
    if acc.shape != (T, rows):
        raise ValueError("acc shape %r does not match n=%d" % (acc.shape, n))
    if epi == RESIDUAL:
        R = _c(R, np.float32).reshape(T, n)
    Y = np.empty((T, n), np.float64)
    _load().oracle_epilogue(epi, _ptr(acc), T, n, _ptr(R) if R is not None else None, _ptr(Y))
    return Y


def gemm(qtype, W, n, k, X, epi, R=None):
    """The whole method in fp64: epilogue(X . W_hat^T). W has 2n rows for SWIGLU."""
    rows = 2 * n if epi == GATE_UP_SWIGLU else n
    W = _check_blocks(qtype, W, rows, k)
    X = _c(X, np.float32).reshape(-1, k)
    T = X.shape[0]
    if epi == RESIDUAL:
        R = _c(R, np.float32).reshape(T, n)
    Y = np.empty((T, n), np.float64)
    _load().oracle_gemm(qtype, _ptr(W), n, k, _ptr(X), T,
                        _ptr(R) if R is not None else None, epi, _ptr(Y))
    return Y


def rmsnorm(X, w, eps):
    """Batched RMSNorm in fp64: row t of X divided by sqrt(mean_j X[t][j]^2 + eps),
    then multiplied by the norm weight w[j] element by element. The pages name the
    step (`batched_rmsnorm_into(x, norm_weight, out, hidden, rows, eps)` on the page
    "aprender-serve 0.70.2 - src/gguf/cuda/forward_qwen35_cuda_prefill.rs", before
    the QKV and gate/up projections) but print no formula; this is the textbook
    definition with eps inside the square root."""
    X = np.asarray(X, np.float64)
    w = np.asarray(w, np.float64).reshape(1, -1)
    ms = np.mean(X * X, axis=1, keepdims=True)
    return X / np.sqrt(ms + eps) * w


def matmul_f64(qtype, W, rows, k, X64):
    """fp64 X64 . W_hat^T for fp64 activations [T][k] (an RMSNorm output, which f32
    would round), with W_hat the exact block decode (dequant_f32); the product is
    numpy's fp64 matrix multiply."""
    Wh = dequant_f32(qtype, W, rows, k).astype(np.float64)
    return np.asarray(X64, np.float64).reshape(-1, k) @ Wh.T


def argmax_last(logits):
    """The greedy token of a logit row: the index of its largest value, the largest
    such index when several are equal (-0 and +0 are equal). The page
    "oxibonsai-kernels 0.1.4 - src/gpu_backend/cuda_q_std_prefill.rs" picks it on
    the host with Rust's Iterator::max_by over partial_cmp, which returns the last
    of equal maxima. Plain Python over the values as given (no rounding)."""
    best_i, best_v = 0, None
    for i, v in enumerate(np.asarray(logits).reshape(-1).tolist()):
        if best_v is None or v >= best_v:
            best_i, best_v = i, v
    return best_i
