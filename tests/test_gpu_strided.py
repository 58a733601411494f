"""GPU parity of pf_gemm_ex: the GEMM into a strided Y (rows ldy >= n floats apart),
through every kernel family, against the fp64 CPU oracle to the usual bars; the
columns between Y's rows keep their bits; and a fused projection (q, k and v
weights stacked row-wise, the fused QKV GEMM of the page "oxibonsai-kernels 0.1.4 -
src/gpu_backend/cuda_q_std_prefill.rs") in one call, its output placed inside wider
rows (the `ldc >= n` of `qwen35_project_rows` on the page "aprender-serve 0.70.2 -
src/cuda/executor/gdn_prefill_ops.rs").
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
F32, F16 = 0, 1
SENTINEL = 0x7FC0_1234  # a NaN pattern no kernel writes


def run_strided(gpu, qtype, W, n, k, X, epi, leg, R=None, pad_left=16, pad_right=36,
                use_ws=False):
    """Y as columns [pad_left, pad_left + n) of a [T][pad_left + n + pad_right] buffer
    filled with SENTINEL (R there for RESIDUAL); returns (Y view, whole buffer) on
    the host after the call."""
    import torch
    T = X.shape[0]
    ldy = pad_left + n + pad_right
    big = torch.full((T, ldy), 0, dtype=torch.int32, device="cuda")
    big.fill_(SENTINEL)
    big = big.view(torch.float32)
    view = big[:, pad_left:pad_left + n]
    if R is not None:
        view.copy_(torch.from_numpy(R.astype(np.float32)).cuda())
    ws = None
    if use_ws:
        need = gpu.workspace_bytes(qtype, n, k, T, epi, leg)
        if need > 0:
            ws = torch.full((need // 2,), -1, dtype=torch.int16, device="cuda")
    gpu.gemm_ex(qtype, parity.to_dev(W), n, k, parity.to_dev(X), view, epi, leg, workspace=ws)
    torch.cuda.synchronize()
    host = big.cpu().numpy()
    return host[:, pad_left:pad_left + n].copy(), host, ldy, pad_left


def check_gaps(host, pad_left, n):
    bits = host.view(np.uint32)
    assert np.all(bits[:, :pad_left] == SENTINEL), "columns before Y written"
    assert np.all(bits[:, pad_left + n:] == SENTINEL), "columns after Y written"


# (T, leg, workspace): the GEMV, the f32 GEMM, the f16 GEMM without and with a
# workspace below 256 rows, and the cooperative kernel (T >= 256) with a workspace.
FAMILIES = [(3, F32, False), (8, F16, False), (40, F32, False), (40, F16, False),
            (40, F16, True), (300, F16, True)]


@pytest.mark.parametrize("epi", [PLAIN, RESIDUAL, SWIGLU])
@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
@pytest.mark.parametrize("T,leg,use_ws", FAMILIES)
def test_strided_y(gpu, qtype, epi, T, leg, use_ws):
    n, k = 200, 768
    wid = 200 + T + 10 * epi + qtype
    W = weight(qtype, n, k, epi == SWIGLU, wid)
    X = acts(T, k, wid)
    R = acts(T, n, wid, synth.TENSOR_R) if epi == RESIDUAL else None
    print("case strided qtype=%d n=%d k=%d T=%d epi=%d leg=%d ws=%d" % (qtype, n, k, T, epi, leg,
                                                                       use_ws), flush=True)
    Y, host, ldy, left = run_strided(gpu, qtype, W, n, k, X, epi, leg, R=R, use_ws=use_ws)
    ok, err = parity.check(qtype, W, n, k, X, Y, epi, leg, R=R)
    assert ok, "parity failed: metric %.3e" % err
    check_gaps(host, left, n)


@pytest.mark.parametrize("epi", [PLAIN, RESIDUAL])
def test_strided_y_split_k(gpu, epi):
    """The cooperative kernel's K split (partial sums, then the sum kernel) into a
    strided Y: narrow n, long k."""
    n, k, T = 1001, 3072, 300
    wid = 240 + epi
    W = weight(Q4_0, n, k, False, wid)
    X = acts(T, k, wid)
    R = acts(T, n, wid, synth.TENSOR_R) if epi == RESIDUAL else None
    need = gpu.workspace_bytes(Q4_0, n, k, T, epi, F16)
    assert need > 320 * k * 2   # the call splits k
    print("case strided-split n=%d k=%d T=%d epi=%d" % (n, k, T, epi), flush=True)
    Y, host, ldy, left = run_strided(gpu, Q4_0, W, n, k, X, epi, F16, R=R, pad_left=4, pad_right=3,
                                     use_ws=True)
    ok, err = parity.check(Q4_0, W, n, k, X, Y, epi, F16, R=R)
    assert ok, "parity failed: metric %.3e" % err
    check_gaps(host, left, n)


@pytest.mark.parametrize("T,leg,use_ws", [(5, F32, False), (64, F16, True), (300, F16, True)])
@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
def test_fused_qkv(gpu, qtype, T, leg, use_ws):
    """q (512 rows), k (128) and v (128) weights stacked in one buffer: one call gives
    Y[:, :512], Y[:, 512:640], Y[:, 640:] equal (to the leg's bar) to the oracle of
    each weight alone; the output sits inside rows of 832 floats."""
    k = 1024
    parts = [("q", 512, 260), ("k", 128, 261), ("v", 128, 262)]
    Ws = [weight(qtype, rows, k, False, wid) for _, rows, wid in parts]
    W = np.concatenate(Ws)
    n = sum(rows for _, rows, _ in parts)
    X = acts(T, k, 263)
    print("case fused-qkv qtype=%d T=%d leg=%d ws=%d" % (qtype, T, leg, use_ws), flush=True)
    Y, host, ldy, left = run_strided(gpu, qtype, W, n, k, X, PLAIN, leg, pad_left=32, pad_right=32,
                                     use_ws=use_ws)
    check_gaps(host, left, n)
    c0 = 0
    for (name, rows, _), Wp in zip(parts, Ws):
        ok, err = parity.check(qtype, Wp, rows, k, X, Y[:, c0:c0 + rows].copy(), PLAIN, leg)
        assert ok, "%s part: metric %.3e" % (name, err)
        c0 += rows
