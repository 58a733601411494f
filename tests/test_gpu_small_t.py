"""GPU parity of the f16-leg GEMM on short chunks (up to 128 token rows: one row tile
of 32, 64 or 128 rows with the four waves side by side): the model's projection
shapes (Q4_0 4096 -> 12288 and 4096 -> 2 x 12288 SwiGLU, Q8_0 12288 -> 4096 with the
residual), with X rounded inside the GEMM (pf_gemm) and once into a workspace
(pf_gemm_ws; SwiGLU there splits along K through its gate/up scratch), each split
along K where the epilogue allows, against the fp64 CPU oracle on sampled columns;
and the rows at each tile size's edge at a small shape, fully checked.
"""
import pytest

import oracle
from quantized_weight_prefill_gguf_amd import synth
from tests.test_gpu_parity import run_and_check
from tests.test_gpu_workspace import run_ws_and_check

pytestmark = pytest.mark.gpu

Q4_0, Q8_0 = synth.Q4_0, synth.Q8_0
PLAIN, RESIDUAL, SWIGLU = oracle.PLAIN, oracle.RESIDUAL, oracle.GATE_UP_SWIGLU
F16 = 1

SHAPES = [(Q4_0, 12288, 4096, PLAIN), (Q4_0, 12288, 4096, SWIGLU), (Q8_0, 4096, 12288, RESIDUAL)]


@pytest.mark.parametrize("ws", [False, True])
@pytest.mark.parametrize("T", [9, 16, 32, 48, 100, 128])
@pytest.mark.parametrize("qtype,n,k,epi", SHAPES)
def test_short_chunk_model_shapes(gpu, qtype, n, k, epi, T, ws):
    wid = 500 + T + 7 * epi
    if ws:
        run_ws_and_check(gpu, qtype, n, k, T, epi, F16, wid=wid, samples=96)
    else:
        run_and_check(gpu, qtype, n, k, T, epi, F16, wid=wid, samples=96)


@pytest.mark.parametrize("ws", [False, True])
@pytest.mark.parametrize("epi", [PLAIN, RESIDUAL, SWIGLU])
@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
@pytest.mark.parametrize("T", [31, 32, 33, 64, 65, 127, 128, 129])
def test_tile_edge_rows(gpu, qtype, epi, T, ws):
    n, k = 391, 2304
    wid = 540 + T + 3 * epi + qtype
    if ws:
        run_ws_and_check(gpu, qtype, n, k, T, epi, F16, wid=wid)
    else:
        run_and_check(gpu, qtype, n, k, T, epi, F16, wid=wid)


@pytest.mark.parametrize("qtype,n,k,epi,T", [(Q4_0, 12288, 4096, SWIGLU, 16), (Q8_0, 4096, 12288, RESIDUAL, 9),
                                             (Q4_0, 12288, 4096, PLAIN, 100)])
def test_workspace_path_deterministic(gpu, qtype, n, k, epi, T):
    """pf_gemm_ws splits K into partial sums in the workspace and adds them in a fixed
    order: two calls give the same bits."""
    import numpy as np
    from tests import parity
    from tests.test_gpu_parity import acts, weight
    wid = 580 + T + epi
    W = weight(qtype, n, k, epi == SWIGLU, wid)
    X = acts(T, k, wid)
    R = acts(T, n, wid, synth.TENSOR_R) if epi == RESIDUAL else None
    print("case ws-determinism qtype=%d n=%d k=%d T=%d epi=%d" % (qtype, n, k, T, epi), flush=True)
    Wd = parity.to_dev(W)
    Y1 = parity.run_gpu(gpu, qtype, None, n, k, X, epi, F16, R=R, Wd=Wd, workspace=True)
    Y2 = parity.run_gpu(gpu, qtype, None, n, k, X, epi, F16, R=R, Wd=Wd, workspace=True)
    assert np.array_equal(Y1.view(np.uint32), Y2.view(np.uint32))
