"""Python binding of libpfgemm (the C ABI in include/pf_gemm.h).

Argument marshalling only: every step of the method runs in the library's gfx950
kernels. PyTorch supplies device memory and the current stream. The binding has
no fallback: if the built library is missing it raises.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpfgemm.so")

PF_Q4_0, PF_Q8_0, PF_F16, PF_Q4_K, PF_Q5_K, PF_Q6_K, PF_IQ4_XS = 0, 1, 2, 3, 4, 5, 6
PF_PLAIN, PF_RESIDUAL, PF_GATE_UP_SWIGLU = 0, 1, 2
PF_LEG_F32, PF_LEG_F16 = 0, 1
PF_PATH_AUTO, PF_PATH_GEMM, PF_PATH_GEMV = 0, 1, 2
PF_GEMV_MAX_T = 8
(PF_OK, PF_E_NULL, PF_E_QTYPE, PF_E_EPILOGUE, PF_E_LEG, PF_E_SHAPE, PF_E_ALIGN,
 PF_E_ALIAS, PF_E_LAUNCH, PF_E_PATH, PF_E_WORKSPACE, PF_E_SCRATCH) = range(12)
PF_NOALLOC_SCRATCH_BYTES = 64 << 20

BLOCK_BYTES = {PF_Q4_0: 18, PF_Q8_0: 34, PF_F16: 64, PF_Q4_K: 144, PF_Q5_K: 176, PF_Q6_K: 210,
               PF_IQ4_XS: 136}
BLOCK_ELEMS = {PF_Q4_0: 32, PF_Q8_0: 32, PF_F16: 32, PF_Q4_K: 256, PF_Q5_K: 256, PF_Q6_K: 256,
               PF_IQ4_XS: 256}
QTYPES = {"q4_0": PF_Q4_0, "q8_0": PF_Q8_0, "f16": PF_F16, "q4_k": PF_Q4_K, "q5_k": PF_Q5_K,
          "q6_k": PF_Q6_K, "iq4_xs": PF_IQ4_XS}
EPILOGUES = {"plain": PF_PLAIN, "residual": PF_RESIDUAL, "swiglu": PF_GATE_UP_SWIGLU}
LEGS = {"f32": PF_LEG_F32, "f16": PF_LEG_F16}

# Every symbol include/pf_gemm.h declares (include/pf_probe.h adds the benchmark's
# pf_probe_read and pf_probe_read_sink_words).
EXPORTS = ("pf_gemm", "pf_gemm_path", "pf_workspace_bytes", "pf_gemm_ws", "pf_gemm_ex",
           "pf_gemm_rmsnorm", "pf_rmsnorm_workspace_bytes", "pf_lm_head_argmax", "pf_prepare_x",
           "pf_gemm_prepared", "pf_select_path", "pf_gemm_noalloc",
           "pf_dequant_f32",
           "pf_dequant_f16", "pf_weight_bytes", "pf_strerror")


class PfError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s: %s" % (what, strerror(status)))


_lib = None


def load():
    """Load libpfgemm.so (built in-tree by build.py); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libpfgemm.so is not built (run quantized_weight_prefill_gguf_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, P = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
    lib.pf_gemm.argtypes = [i32, P, i64, i64, P, i64, P, i32, i32, P]
    lib.pf_gemm.restype = i32
    lib.pf_gemm_noalloc.argtypes = [i32, P, i64, i64, P, i64, P, i32, i32, P]
    lib.pf_gemm_noalloc.restype = i32
    lib.pf_gemm_path.argtypes = [i32, P, i64, i64, P, i64, P, i32, i32, P, i32]
    lib.pf_gemm_path.restype = i32
    lib.pf_workspace_bytes.argtypes = [i32, i64, i64, i64, i32, i32]
    lib.pf_workspace_bytes.restype = i64
    lib.pf_gemm_ws.argtypes = [i32, P, i64, i64, P, i64, P, i32, i32, P, i64, P]
    lib.pf_gemm_ws.restype = i32
    lib.pf_gemm_ex.argtypes = [i32, P, i64, i64, P, i64, P, i64, i32, i32, P, i64, P]
    lib.pf_gemm_ex.restype = i32
    lib.pf_gemm_rmsnorm.argtypes = [i32, P, i64, i64, P, i64, P, ctypes.c_float, P, i64, i32, i32, P,
                                    i64, P]
    lib.pf_gemm_rmsnorm.restype = i32
    lib.pf_rmsnorm_workspace_bytes.argtypes = [i32, i64, i64, i64, i32, i32]
    lib.pf_rmsnorm_workspace_bytes.restype = i64
    lib.pf_lm_head_argmax.argtypes = [i32, P, i64, i64, P, P, P, P]
    lib.pf_lm_head_argmax.restype = i32
    lib.pf_prepare_x.argtypes = [i32, i64, P, i64, P, i64, P]
    lib.pf_prepare_x.restype = i32
    lib.pf_gemm_prepared.argtypes = [i32, P, i64, i64, i64, P, i64, i32, P, i64, P]
    lib.pf_gemm_prepared.restype = i32
    lib.pf_select_path.argtypes = [i32, i64, i64, i64, i32, i32]
    lib.pf_select_path.restype = i32
    lib.pf_dequant_f32.argtypes = [i32, P, i64, i64, P, P]
    lib.pf_dequant_f32.restype = i32
    lib.pf_dequant_f16.argtypes = [i32, P, i64, i64, P, P]
    lib.pf_dequant_f16.restype = i32
    lib.pf_weight_bytes.argtypes = [i32, i64, i64]
    lib.pf_weight_bytes.restype = i64
    lib.pf_strerror.argtypes = [i32]
    lib.pf_strerror.restype = ctypes.c_char_p
    # the benchmark's read floor (include/pf_probe.h)
    lib.pf_probe_read.argtypes = [P, i64, P, P]
    lib.pf_probe_read.restype = i32
    lib.pf_probe_read_sink_words.argtypes = []
    lib.pf_probe_read_sink_words.restype = i64
    _lib = lib
    return lib


def strerror(status):
    return load().pf_strerror(status).decode()


def weight_bytes(qtype, rows, k):
    return load().pf_weight_bytes(qtype, rows, k)


def select_path(qtype, n, k, T, epilogue, leg):
    return load().pf_select_path(qtype, n, k, T, epilogue, leg)


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev_ptr(t, name):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return ctypes.c_void_p(t.data_ptr())


def y_view_ldy(Y, T, n):
    """ldy of a [T][n] float32 view Y whose rows may lie ldy >= n floats apart: the
    elements of a row must be adjacent (stride 1) whenever a row has more than one,
    whatever T is, since the library writes n consecutive floats per row. Raises
    ValueError otherwise. Checks the view only (not the device)."""
    if Y.dim() != 2 or tuple(Y.shape) != (T, n):
        raise ValueError("Y must be a [T][n] view, got shape %s" % (tuple(Y.shape),))
    if n > 1 and Y.stride(1) != 1:
        raise ValueError("Y must have unit stride within rows")
    return Y.stride(0) if T > 1 else n


def workspace_bytes(qtype, n, k, T, epilogue, leg):
    """Bytes of workspace gemm_ws needs (0 if none; negative status on bad sizes)."""
    return load().pf_workspace_bytes(qtype, n, k, T, epilogue, leg)


def _check_gemm_args(qtype, W, n, k, X, Y, epilogue):
    import torch
    if X.dtype != torch.float32 or Y.dtype != torch.float32 or W.dtype != torch.uint8:
        raise TypeError("X and Y must be float32 and W uint8")
    T = X.numel() // k if k > 0 else 0
    if X.numel() != T * k or Y.numel() != T * n:
        raise ValueError("X must hold T*k and Y T*n elements")
    rows = 2 * n if epilogue == PF_GATE_UP_SWIGLU else n
    need = load().pf_weight_bytes(qtype, rows, k)
    if need >= 0 and W.numel() < need:
        raise ValueError("W holds %d bytes, %d needed" % (W.numel(), need))
    return T


def gemm_ws(qtype, W, n, k, X, Y, epilogue, leg, workspace, stream=None):
    """gemm with a caller workspace (a device tensor of at least workspace_bytes()
    bytes, or None when that is 0); see pf_gemm_ws."""
    T = _check_gemm_args(qtype, W, n, k, X, Y, epilogue)
    if workspace is None:
        ws, ws_bytes = ctypes.c_void_p(0), 0
    else:
        ws, ws_bytes = _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size()
    st = load().pf_gemm_ws(qtype, _dev_ptr(W, "W"), n, k, _dev_ptr(X, "X"), T, _dev_ptr(Y, "Y"),
                           epilogue, leg, ws, ws_bytes, _stream_handle(stream))
    if st != PF_OK:
        raise PfError(st, "pf_gemm_ws")
    return Y


def gemm_ex(qtype, W, n, k, X, Y, epilogue, leg, workspace=None, stream=None):
    """gemm / gemm_ws into a strided Y (see pf_gemm_ex): Y is a float32 device view
    [T][n] whose rows may lie ldy >= n floats apart (unit stride within a row), e.g.
    a column range of a wider buffer. workspace None runs as gemm."""
    import torch
    T = X.numel() // k if k > 0 else 0
    if X.dtype != torch.float32 or Y.dtype != torch.float32 or W.dtype != torch.uint8:
        raise TypeError("X and Y must be float32 and W uint8")
    if X.numel() != T * k or not X.is_contiguous():
        raise ValueError("X must be a contiguous [T][k] tensor")
    if not Y.is_cuda:
        raise ValueError("Y must be a device tensor")
    ldy = y_view_ldy(Y, T, n)
    rows = 2 * n if epilogue == PF_GATE_UP_SWIGLU else n
    need = load().pf_weight_bytes(qtype, rows, k)
    if need >= 0 and W.numel() < need:
        raise ValueError("W holds %d bytes, %d needed" % (W.numel(), need))
    if workspace is None:
        ws, ws_bytes = ctypes.c_void_p(0), 0
    else:
        ws, ws_bytes = _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size()
    st = load().pf_gemm_ex(qtype, _dev_ptr(W, "W"), n, k, _dev_ptr(X, "X"), T, ctypes.c_void_p(Y.data_ptr()),
                           ldy, epilogue, leg, ws, ws_bytes, _stream_handle(stream))
    if st != PF_OK:
        raise PfError(st, "pf_gemm_ex")
    return Y


def rmsnorm_workspace_bytes(qtype, n, k, T, epilogue, leg):
    """Bytes of workspace gemm_rmsnorm needs (negative status on bad sizes)."""
    return load().pf_rmsnorm_workspace_bytes(qtype, n, k, T, epilogue, leg)


def gemm_rmsnorm(qtype, W, n, k, X, norm_w, eps, Y, epilogue, leg, workspace, stream=None):
    """Y = epilogue(RMSNorm(X; norm_w, eps) . W_hat^T) (see pf_gemm_rmsnorm). norm_w is
    a float32 device tensor of k values; Y a [T][n] device view as in gemm_ex; the
    workspace a device tensor of at least rmsnorm_workspace_bytes() bytes."""
    import torch
    T = X.numel() // k if k > 0 else 0
    if X.dtype != torch.float32 or Y.dtype != torch.float32 or W.dtype != torch.uint8 or \
            norm_w.dtype != torch.float32:
        raise TypeError("X, Y and norm_w must be float32 and W uint8")
    if X.numel() != T * k or norm_w.numel() != k:
        raise ValueError("X must hold T*k and norm_w k elements")
    if not Y.is_cuda:
        raise ValueError("Y must be a device tensor")
    ldy = y_view_ldy(Y, T, n)
    rows = 2 * n if epilogue == PF_GATE_UP_SWIGLU else n
    need = load().pf_weight_bytes(qtype, rows, k)
    if need >= 0 and W.numel() < need:
        raise ValueError("W holds %d bytes, %d needed" % (W.numel(), need))
    if workspace is None:
        ws, ws_bytes = ctypes.c_void_p(0), 0
    else:
        ws, ws_bytes = _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size()
    st = load().pf_gemm_rmsnorm(qtype, _dev_ptr(W, "W"), n, k, _dev_ptr(X, "X"), T,
                                _dev_ptr(norm_w, "norm_w"), float(eps), ctypes.c_void_p(Y.data_ptr()),
                                ldy, epilogue, leg, ws, ws_bytes, _stream_handle(stream))
    if st != PF_OK:
        raise PfError(st, "pf_gemm_rmsnorm")
    return Y


def lm_head_argmax(qtype, W, n, k, x, logits, token, stream=None):
    """logits[n] = x[k] . W_hat^T and token[0] = the largest index among its maxima
    (see pf_lm_head_argmax). x, logits: float32 device tensors; token: an int32
    device tensor of at least one element."""
    import torch
    if x.dtype != torch.float32 or logits.dtype != torch.float32 or W.dtype != torch.uint8 or \
            token.dtype != torch.int32:
        raise TypeError("x and logits must be float32, W uint8, token int32")
    if x.numel() != k or logits.numel() != n or token.numel() < 1:
        raise ValueError("x must hold k, logits n and token at least one element")
    need = load().pf_weight_bytes(qtype, n, k)
    if need >= 0 and W.numel() < need:
        raise ValueError("W holds %d bytes, %d needed" % (W.numel(), need))
    st = load().pf_lm_head_argmax(qtype, _dev_ptr(W, "W"), n, k, _dev_ptr(x, "x"), _dev_ptr(logits, "logits"),
                                  _dev_ptr(token, "token"), _stream_handle(stream))
    if st != PF_OK:
        raise PfError(st, "pf_lm_head_argmax")
    return token


def prepare_x(qtype, k, X, workspace, stream=None):
    """X [T][k] (float32 device) rounded to binary16 into the workspace for
    gemm_prepared (see pf_prepare_x)."""
    import torch
    T = X.numel() // k if k > 0 else 0
    if X.dtype != torch.float32 or X.numel() != T * k:
        raise ValueError("X must be float32 [T][k]")
    st = load().pf_prepare_x(qtype, k, _dev_ptr(X, "X"), T, _dev_ptr(workspace, "workspace"),
                             workspace.numel() * workspace.element_size(), _stream_handle(stream))
    if st != PF_OK:
        raise PfError(st, "pf_prepare_x")
    return workspace


def gemm_prepared(qtype, W, n, k, T, Y, epilogue, workspace, stream=None):
    """The f16-leg GEMM on a prepare_x copy in the workspace (see pf_gemm_prepared); Y
    a [T][n] float32 device view as in gemm_ex."""
    import torch
    if Y.dtype != torch.float32 or W.dtype != torch.uint8:
        raise TypeError("Y must be float32 and W uint8")
    if not Y.is_cuda:
        raise ValueError("Y must be a device tensor")
    ldy = y_view_ldy(Y, T, n)
    rows = 2 * n if epilogue == PF_GATE_UP_SWIGLU else n
    need = load().pf_weight_bytes(qtype, rows, k)
    if need >= 0 and W.numel() < need:
        raise ValueError("W holds %d bytes, %d needed" % (W.numel(), need))
    st = load().pf_gemm_prepared(qtype, _dev_ptr(W, "W"), n, k, T, ctypes.c_void_p(Y.data_ptr()), ldy, epilogue,
                                 _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                 _stream_handle(stream))
    if st != PF_OK:
        raise PfError(st, "pf_gemm_prepared")
    return Y


def gemm(qtype, W, n, k, X, Y, epilogue, leg, stream=None, path=PF_PATH_AUTO):
    """Y[T][n] = epilogue(X[T][k] . W_hat^T) on the device (see pf_gemm).

    W: uint8 device tensor of blocks; X, Y: float32 device tensors [T][k], [T][n].
    """
    T = _check_gemm_args(qtype, W, n, k, X, Y, epilogue)
    lib = load()
    st = lib.pf_gemm_path(qtype, _dev_ptr(W, "W"), n, k, _dev_ptr(X, "X"), T, _dev_ptr(Y, "Y"),
                          epilogue, leg, _stream_handle(stream), path)
    if st != PF_OK:
        raise PfError(st, "pf_gemm")
    return Y


def gemm_noalloc(qtype, W, n, k, X, Y, epilogue, leg, stream=None):
    """gemm_ws in the library's static device scratch: no workspace argument and no
    allocation (see pf_gemm_noalloc; calls that overlap on one GPU race)."""
    T = _check_gemm_args(qtype, W, n, k, X, Y, epilogue)
    st = load().pf_gemm_noalloc(qtype, _dev_ptr(W, "W"), n, k, _dev_ptr(X, "X"), T, _dev_ptr(Y, "Y"),
                                epilogue, leg, _stream_handle(stream))
    if st != PF_OK:
        raise PfError(st, "pf_gemm_noalloc")
    return Y


def dequant_f32(qtype, W, rows, k, out, stream=None):
    """out[rows][k] (float32 device tensor) = the exact block decode of W."""
    import torch
    if out.dtype != torch.float32 or out.numel() != rows * k:
        raise ValueError("out must be float32 with rows*k elements")
    st = load().pf_dequant_f32(qtype, _dev_ptr(W, "W"), rows, k, _dev_ptr(out, "out"),
                               _stream_handle(stream))
    if st != PF_OK:
        raise PfError(st, "pf_dequant_f32")
    return out


def dequant_f16(qtype, W, rows, k, out, stream=None):
    """out[rows][k] (int16/uint16 device tensor of binary16 bits) = RNE_fp16(decode)."""
    if out.element_size() != 2 or out.numel() != rows * k:
        raise ValueError("out must have 2-byte elements, rows*k of them")
    st = load().pf_dequant_f16(qtype, _dev_ptr(W, "W"), rows, k, _dev_ptr(out, "out"),
                               _stream_handle(stream))
    if st != PF_OK:
        raise PfError(st, "pf_dequant_f16")
    return out
