"""Parity harness: run the GPU path through the C ABI and judge it with the oracle.

Small problems are checked on every output against the full fp64 oracle. Full-size
problems are checked on sampled outputs that the oracle computes one by one.
"""
import numpy as np

import oracle
from oracle import tolerance
from quantized_weight_prefill_gguf_amd import synth

LEG_NAME = {0: "f32", 1: "f16"}


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_gpu(pf, qtype, W, n, k, X, epi, leg, R=None, path=0, stream=None, Wd=None, Xd=None,
            workspace=False):
    """Y on the device via pf.gemm (or pf.gemm_ws with a NaN-filled workspace of
    exactly the size it asks for, when workspace is True); returns the numpy result."""
    import torch
    T = X.shape[0]
    Wd = to_dev(W) if Wd is None else Wd
    Xd = to_dev(X) if Xd is None else Xd
    if epi == oracle.RESIDUAL:
        Yd = to_dev(R.astype(np.float32))
    else:
        Yd = torch.full((T, n), float("nan"), dtype=torch.float32, device="cuda")
    if workspace:
        need = pf.workspace_bytes(qtype, n, k, T, epi, leg)
        assert need >= 0
        ws = torch.full((max(need, 16) // 2,), -1, dtype=torch.int16, device="cuda") if need else None
        pf.gemm_ws(qtype, Wd, n, k, Xd, Yd, epi, leg, ws, stream=stream)
    else:
        pf.gemm(qtype, Wd, n, k, Xd, Yd, epi, leg, stream=stream, path=path)
    torch.cuda.synchronize()
    return Yd.cpu().numpy()


def _rows_subset(qtype, W, k, rows):
    """Bytes of the listed weight rows, concatenated (rows are contiguous in W)."""
    rb = (k // synth.BLOCK_ELEMS[qtype]) * synth.BLOCK_BYTES[qtype]
    W2 = np.asarray(W, np.uint8).reshape(-1, rb)
    return np.ascontiguousarray(W2[rows]).reshape(-1)


def check(qtype, W, n, k, X, Y, epi, leg, R=None, samples=None, rng_seed=0):
    """Judge Y against the oracle. samples=None: every output; else the number of
    random (t, r) pairs (plus the last token row and last column). Returns
    (ok, metric) where metric is the normalised error (PLAIN/RESIDUAL) or the
    first-order ratio (SWIGLU)."""
    T = X.shape[0]
    legn = LEG_NAME[leg]
    xn = np.linalg.norm(X.astype(np.float64), axis=1)
    if samples is None:
        ti, ri = np.meshgrid(np.arange(T), np.arange(n), indexing="ij")
        ti, ri = ti.reshape(-1), ri.reshape(-1)
    else:
        rng = np.random.default_rng(rng_seed)
        ti = np.concatenate([rng.integers(0, T, samples), np.full(n, T - 1), np.arange(T)])
        ri = np.concatenate([rng.integers(0, n, samples), np.arange(n), np.full(T, n - 1)])
    y = np.asarray(Y, np.float64).reshape(T, n)[ti, ri]
    if epi == oracle.GATE_UP_SWIGLU:
        ur = np.unique(ri)
        sub_g = _rows_subset(qtype, W, k, ur)
        sub_u = _rows_subset(qtype, W, k, ur + n)
        pos = np.searchsorted(ur, ri)
        g = oracle.matmul_sampled(qtype, sub_g, ur.size, k, X, ti, pos)
        u = oracle.matmul_sampled(qtype, sub_u, ur.size, k, X, ti, pos)
        gn = oracle.row_norms(qtype, sub_g, ur.size, k)[pos]
        un = oracle.row_norms(qtype, sub_u, ur.size, k)[pos]
        return tolerance.swiglu_check_elems(y, g, u, gn * xn[ti], un * xn[ti], legn)
    ur = np.unique(ri)
    sub = _rows_subset(qtype, W, k, ur)
    pos = np.searchsorted(ur, ri)
    acc = oracle.matmul_sampled(qtype, sub, ur.size, k, X, ti, pos)
    wn = oracle.row_norms(qtype, sub, ur.size, k)[pos]
    ref = acc + (np.asarray(R, np.float64).reshape(T, n)[ti, ri] if epi == oracle.RESIDUAL else 0.0)
    return tolerance.check_linear_elems(y, ref, wn * xn[ti], legn)
