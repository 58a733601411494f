"""GPU parity on adversarial weight blocks (tests/edge_blocks.py): every byte value as
a code (Q8_0 -128 included), negative and zero scales, binary16 subnormal scales and
the largest scale each leg allows, through every kernel family, against the fp64
oracle on every output at the leg's bar. Zero-scale rows must come out exactly 0
(R for RESIDUAL).

The synthetic quantizer never makes these blocks (its Q8_0 codes stay in [-127, 127]
and its scales are positive normals), so this is the test of the kernels' own
decode paths on them: the GEMV's per-block algebra d (sum u x - c sum x) with
u = byte ^ 0x80, the cooperative kernel's per-unit decode, the 4-wave kernel's
per-fragment decode, the f32 GEMM's exact decode, and the fp16 MFMA fed subnormal
weights.
"""
import numpy as np
import pytest

import oracle
from quantized_weight_prefill_gguf_amd import synth
from tests import edge_blocks, parity

pytestmark = pytest.mark.gpu

Q4_0, Q8_0 = synth.Q4_0, synth.Q8_0
PLAIN, RESIDUAL, SWIGLU = oracle.PLAIN, oracle.RESIDUAL, oracle.GATE_UP_SWIGLU
F32, F16 = 0, 1
LEG_NAME = {F32: "f32", F16: "f16"}

# (label, leg, T, k, path, workspace): each reaches one kernel family.
FAMILIES = [
    ("f32_gemm", F32, 40, 768, 1, False),
    ("f16_row1_32", F16, 20, 768, 1, False),
    ("f16_row1_128", F16, 100, 768, 1, False),
    ("f16_tiles_T200", F16, 200, 768, 1, False),
    ("f16_ws_row1_32", F16, 20, 2560, 0, True),      # split K (SwiGLU: the scratch form)
    ("f16_ws_T200", F16, 200, 2560, 0, True),
    ("coop_256x192", F16, 300, 2560, 0, True),
    ("coop_512x96", F16, 600, 2560, 0, True),
]


def _run(gpu, qtype, n, k, T, epi, leg, path, workspace, seed):
    rows = 2 * n if epi == SWIGLU else n
    W = edge_blocks.weight(qtype, rows, k, LEG_NAME[leg], seed)
    X = synth.activations(T, k, workload_id=seed)
    R = synth.activations(T, n, workload_id=seed, tensor_id=synth.TENSOR_R) if epi == RESIDUAL else None
    Y = parity.run_gpu(gpu, qtype, W, n, k, X, epi, leg, R=R, path=path, workspace=workspace)
    ok, err = parity.check(qtype, W, n, k, X, Y, epi, leg, R=R)
    assert ok, "parity failed on adversarial blocks: metric %.3e" % err
    if epi != SWIGLU:
        # rows whose scale is +-0 in every block decode to zeros: exact 0 (or R)
        nscale = len(edge_blocks.scales(LEG_NAME[leg], qtype))
        for r in range(n):
            if r < 2 * nscale and edge_blocks.scales(LEG_NAME[leg], qtype)[r % nscale] == 0:
                want = R[:, r] if R is not None else np.zeros(T, np.float32)
                assert np.array_equal(Y[:, r], want), r
    return Y


@pytest.mark.parametrize("epi", [PLAIN, RESIDUAL, SWIGLU])
@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
@pytest.mark.parametrize("family", FAMILIES, ids=[f[0] for f in FAMILIES])
def test_edge_blocks_gemm_families(gpu, family, qtype, epi):
    label, leg, T, k, path, ws = family
    n = 40
    print("case edge %s qtype=%d epi=%d T=%d k=%d" % (label, qtype, epi, T, k), flush=True)
    if ws:
        assert gpu.select_path(qtype, n, k, T, epi, leg) == gpu.PF_PATH_GEMM
    _run(gpu, qtype, n, k, T, epi, leg, path, ws, seed=700 + 10 * qtype + epi + T)


@pytest.mark.parametrize("leg", [F32, F16])
@pytest.mark.parametrize("epi", [PLAIN, RESIDUAL, SWIGLU])
@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 6, 7, 8])
def test_edge_blocks_gemv(gpu, T, qtype, epi, leg):
    """The GEMV forced at every T it takes, both legs (it computes in f32 on both)."""
    print("case edge gemv qtype=%d epi=%d T=%d leg=%d" % (qtype, epi, T, leg), flush=True)
    _run(gpu, qtype, 40, 1024, T, epi, leg, 2, False, seed=800 + 10 * qtype + epi + T)


@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
def test_edge_blocks_lm_head(gpu, qtype):
    """pf_lm_head_argmax on adversarial rows: logits at the f32 bar, the token the
    oracle's greedy pick over the same f32 logits."""
    import torch
    from oracle import tolerance
    n, k = 333, 1024
    W = edge_blocks.weight(qtype, n, k, "f32", 900 + qtype)
    x = synth.activations(1, k, workload_id=900 + qtype).reshape(k)
    logits = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    token = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    print("case edge lm_head qtype=%d" % qtype, flush=True)
    gpu.lm_head_argmax(qtype, parity.to_dev(W), n, k, parity.to_dev(x), logits, token)
    torch.cuda.synchronize()
    lg, tok = logits.cpu().numpy(), int(token.cpu().numpy()[0])
    acc = oracle.matmul(qtype, W, n, k, x.reshape(1, k))
    ok, err = tolerance.check_linear(lg.reshape(1, n), acc, oracle.row_norms(qtype, W, n, k),
                                     np.linalg.norm(x.astype(np.float64)).reshape(1), "f32")
    assert ok, "logits parity failed: metric %.3e" % err
    assert tok == oracle.argmax_last(lg)
