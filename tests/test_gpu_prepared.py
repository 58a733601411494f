"""GPU checks of pf_prepare_x + pf_gemm_prepared: the same kernels as pf_gemm_ws in two
calls, whose K splits store partial sums that a second kernel adds in a fixed order,
so the result must equal pf_gemm_ws bit for bit at every T. One prepared copy of X
serves several projections (q, k and v weights of different widths) in a row, and the
copy is left intact by the GEMMs.
"""
import numpy as np
import pytest

import oracle
from quantized_weight_prefill_gguf_amd import synth
from tests import parity
from tests.test_gpu_parity import acts, weight

pytestmark = pytest.mark.gpu

Q4_0, Q8_0 = synth.Q4_0, synth.Q8_0
PLAIN, RESIDUAL, SWIGLU = oracle.PLAIN, oracle.RESIDUAL, oracle.GATE_UP_SWIGLU
F16 = 1


def ws_for(gpu, qtype, n, k, T, epi):
    import torch
    need = gpu.workspace_bytes(qtype, n, k, T, epi, F16)
    return torch.full((need // 2,), -1, dtype=torch.int16, device="cuda")


@pytest.mark.parametrize("epi", [PLAIN, RESIDUAL, SWIGLU])
@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
@pytest.mark.parametrize("T,n,k", [(40, 200, 768), (300, 1001, 3072), (512, 384, 1024)])
def test_prepared_equals_ws(gpu, qtype, epi, T, n, k):
    import torch
    wid = 600 + T + epi
    W = parity.to_dev(weight(qtype, n, k, epi == SWIGLU, wid))
    X = acts(T, k, wid)
    R = acts(T, n, wid, synth.TENSOR_R) if epi == RESIDUAL else None
    print("case prepared qtype=%d n=%d k=%d T=%d epi=%d" % (qtype, n, k, T, epi), flush=True)
    Y0 = parity.run_gpu(gpu, qtype, None, n, k, X, epi, F16, R=R, Wd=W, workspace=True)
    ws = ws_for(gpu, qtype, n, k, T, epi)
    Y = torch.from_numpy(R.copy()).cuda() if R is not None else \
        torch.full((T, n), float("nan"), dtype=torch.float32, device="cuda")
    gpu.prepare_x(qtype, k, parity.to_dev(X), ws)
    gpu.gemm_prepared(qtype, W, n, k, T, Y, epi, ws)
    torch.cuda.synchronize()
    check(qtype, W, n, k, X, Y.cpu().numpy(), Y0, epi, R)


def check(qtype, Wd, n, k, X, Y, Y0, epi, R=None):
    assert np.array_equal(Y.view(np.uint32), Y0.view(np.uint32))


# F16 up to 128 rows keeps its own GEMM, which has no prepared form
FURTHER = [(q, T, n) for q in (synth.Q4_K, synth.Q5_K, synth.IQ4_XS, synth.Q6_K, synth.F16)
           for T, n in ((40, 200), (300, 200), (520, 150)) if q != synth.F16 or T > 128]


@pytest.mark.parametrize("epi", [PLAIN, RESIDUAL, SWIGLU])
@pytest.mark.parametrize("qtype,T,n", FURTHER)
def test_prepared_equals_ws_further_types(gpu, qtype, T, n, epi):
    """The further types where pf_gemm_ws runs them on the f16 GEMMs (the 4-wave kernel at
    40 rows; the cooperative kernel above, F16 only there): the prepared form gives
    pf_gemm_ws's bits."""
    import torch
    k = 1024
    wid = 630 + T + epi + 7 * qtype
    rows = 2 * n if epi == SWIGLU else n
    W = parity.to_dev(synth.quantize(qtype, synth.weights_f32(rows, k, workload_id=wid)))
    X = acts(T, k, wid)
    R = acts(T, n, wid, synth.TENSOR_R) if epi == RESIDUAL else None
    print("case prepared further qtype=%d n=%d T=%d epi=%d" % (qtype, n, T, epi), flush=True)
    Y0 = parity.run_gpu(gpu, qtype, None, n, k, X, epi, F16, R=R, Wd=W, workspace=True)
    ws = ws_for(gpu, qtype, n, k, T, epi)
    Y = torch.from_numpy(R.copy()).cuda() if R is not None else \
        torch.full((T, n), float("nan"), dtype=torch.float32, device="cuda")
    gpu.prepare_x(qtype, k, parity.to_dev(X), ws)
    gpu.gemm_prepared(qtype, W, n, k, T, Y, epi, ws)
    torch.cuda.synchronize()
    check(qtype, W, n, k, X, Y.cpu().numpy(), Y0, epi, R)


@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
@pytest.mark.parametrize("T", [64, 512])
def test_one_copy_many_projections(gpu, qtype, T):
    import torch
    k = 2048
    parts = [(1024, 610), (256, 611), (256, 612)]
    X = acts(T, k, 613)
    Xd = parity.to_dev(X)
    need = max(gpu.workspace_bytes(qtype, n, k, T, PLAIN, F16) for n, _ in parts)
    ws = torch.full((need // 2,), -1, dtype=torch.int16, device="cuda")
    gpu.prepare_x(qtype, k, Xd, ws)
    torch.cuda.synchronize()
    xcopy = ws[: (T + 31) // 32 * 32 * k].clone()
    print("case one-copy qtype=%d T=%d" % (qtype, T), flush=True)
    for n, wid in parts:
        W = parity.to_dev(weight(qtype, n, k, False, wid))
        Y = torch.full((T, n), float("nan"), dtype=torch.float32, device="cuda")
        gpu.gemm_prepared(qtype, W, n, k, T, Y, PLAIN, ws)
        torch.cuda.synchronize()
        Y0 = parity.run_gpu(gpu, qtype, None, n, k, X, PLAIN, F16, Wd=W, workspace=True)
        check(qtype, W, n, k, X, Y.cpu().numpy(), Y0, PLAIN)
    assert torch.equal(ws[: xcopy.numel()], xcopy), "the prepared copy was overwritten"


@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
@pytest.mark.parametrize("epi", [PLAIN, RESIDUAL, SWIGLU])
def test_prepared_few_rows(gpu, qtype, epi):
    """Five rows: every epilogue runs the GEMM on the prepared copy (the family
    pf_gemm_ws picks there on the f16 leg), bit for bit as pf_gemm_ws; where pf_gemm_ws
    runs the GEMV (PLAIN at 2 rows, SwiGLU at 4) there is no prepared form and the call
    is refused."""
    import torch
    n, k, T = 300, 1024, 5
    wid = 650 + epi + qtype
    W_np = weight(qtype, n, k, epi == SWIGLU, wid)
    Wd = parity.to_dev(W_np)
    X = acts(T, k, wid)
    R = acts(T, n, wid, synth.TENSOR_R) if epi == RESIDUAL else None
    print("case prepared-few qtype=%d T=%d epi=%d" % (qtype, T, epi), flush=True)
    ws = ws_for(gpu, qtype, n, k, T, epi)
    gpu.prepare_x(qtype, k, parity.to_dev(X), ws)
    Y = torch.from_numpy(R.copy()).cuda() if R is not None else \
        torch.full((T, n), float("nan"), dtype=torch.float32, device="cuda")
    gpu.gemm_prepared(qtype, Wd, n, k, T, Y, epi, ws)
    torch.cuda.synchronize()
    Y0 = parity.run_gpu(gpu, qtype, None, n, k, X, epi, F16, R=R, Wd=Wd, workspace=True)
    check(qtype, Wd, n, k, X, Y.cpu().numpy(), Y0, epi)
    ok, err = parity.check(qtype, W_np, n, k, X, Y.cpu().numpy(), epi, F16, R=R)
    assert ok, "parity failed: metric %.3e" % err
    # the GEMV's row counts: refused before anything is enqueued
    tg = 4 if epi == SWIGLU else 2
    Yg = torch.zeros((tg, n), dtype=torch.float32, device="cuda")
    with pytest.raises(gpu.PfError):
        gpu.gemm_prepared(qtype, Wd, n, k, tg, Yg, epi, ws)
