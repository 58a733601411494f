"""GPU parity of pf_gemm_rmsnorm (the projection with its batched RMSNorm prologue)
against the fp64 CPU oracle: Xn = oracle.rmsnorm(X, w, eps) in fp64, then the GEMM
on Xn in fp64 (oracle.matmul_f64), judged by the usual bars with ||Xn_t|| as the
activation norm. Every kernel family: the GEMV (both legs), the f32 GEMM, the f16
GEMM below 256 rows and the cooperative kernel (with and without a K split), and a
strided Y.
"""
import numpy as np
import pytest

import oracle
from oracle import tolerance
from quantized_weight_prefill_gguf_amd import synth
from tests import parity
from tests.test_gpu_parity import acts, weight

pytestmark = pytest.mark.gpu

Q4_0, Q8_0 = synth.Q4_0, synth.Q8_0
PLAIN, RESIDUAL, SWIGLU = oracle.PLAIN, oracle.RESIDUAL, oracle.GATE_UP_SWIGLU
F32, F16 = 0, 1
EPS = 1e-6


def norm_weight(k, wid):
    return np.random.default_rng([wid, 9]).uniform(0.5, 1.5, k).astype(np.float32)


def run_and_check(gpu, qtype, n, k, T, epi, leg, wid, pad=0):
    import torch
    rows = 2 * n if epi == SWIGLU else n
    W = weight(qtype, n, k, epi == SWIGLU, wid)
    X = acts(T, k, wid, row_scale=True)
    w = norm_weight(k, wid)
    R = acts(T, n, wid, synth.TENSOR_R) if epi == RESIDUAL else None
    print("case rmsnorm qtype=%d n=%d k=%d T=%d epi=%d leg=%d pad=%d" % (qtype, n, k, T, epi, leg, pad),
          flush=True)
    big = torch.full((T, n + pad), float("nan"), dtype=torch.float32, device="cuda")
    Y = big[:, :n]
    if R is not None:
        Y.copy_(torch.from_numpy(R).cuda())
    need = gpu.rmsnorm_workspace_bytes(qtype, n, k, T, epi, leg)
    assert need > 0
    ws = torch.full((need // 2,), -1, dtype=torch.int16, device="cuda")
    Xd = parity.to_dev(X)
    gpu.gemm_rmsnorm(qtype, parity.to_dev(W), n, k, Xd, torch.from_numpy(w).cuda(), EPS, Y, epi, leg, ws)
    torch.cuda.synchronize()
    host = big.cpu().numpy()
    Yh = host[:, :n].copy()
    assert np.array_equal(Xd.cpu().numpy(), X), "X was modified"
    if pad:
        assert np.all(np.isnan(host[:, n:])), "columns past n written"
    Xn = oracle.rmsnorm(X, w, EPS)
    acc = oracle.matmul_f64(qtype, W, rows, k, Xn)
    norms = oracle.row_norms(qtype, W, rows, k)
    xn = np.linalg.norm(Xn, axis=1)
    legn = "f32" if leg == F32 else "f16"
    if epi == SWIGLU:
        ok, err = tolerance.swiglu_check(Yh, acc[:, :n], acc[:, n:], norms[:n], norms[n:], xn, legn)
    else:
        ref = oracle.epilogue(epi, acc, n, R)
        ok, err = tolerance.check_linear(Yh, ref, norms, xn, legn)
    assert ok, "parity failed: metric %.3e" % err


@pytest.mark.parametrize("epi", [PLAIN, RESIDUAL, SWIGLU])
@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
@pytest.mark.parametrize("T,leg", [(3, F32), (6, F16), (40, F32), (40, F16), (300, F16)])
def test_rmsnorm_families(gpu, qtype, epi, T, leg):
    run_and_check(gpu, qtype, 200, 768, T, epi, leg, wid=300 + T + 10 * epi + qtype)


@pytest.mark.parametrize("epi", [PLAIN, RESIDUAL])
def test_rmsnorm_split_k_strided(gpu, epi):
    """The cooperative kernel's K split behind the norm, into a strided Y."""
    run_and_check(gpu, Q4_0, 1001, 3072, 300, epi, F16, wid=350 + epi, pad=7)


def test_rmsnorm_ffn_gate_up(gpu):
    """The gate/up SwiGLU shape at T = 512 (Q4_0 4096 -> 2 x 12288), sampled by the
    full parity check on a column block."""
    run_and_check(gpu, Q4_0, 1536, 4096, 512, SWIGLU, F16, wid=360)
