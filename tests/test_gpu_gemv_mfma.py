"""Parity of the matrix-core GEMV (f32 leg, 3 <= T <= 8; T = 1 and 2 run the vector-ALU
GEMV and are checked here too) on every output, against the fp64 oracle at the f32 bar.

Shapes pick each workgroup form the launcher can choose: for PLAIN and RESIDUAL four
compute waves of one row quad (n = 100) or two (n = 8200, and Q8_0 with more than four
tokens at n >= 12241, whose twelve-wave form does not fit in LDS), or twelve waves of
one quad (n = 12290, 16390); for SwiGLU four compute waves of two or four quads (n = 100,
8200) or twelve of two (n = 12290 with up to four tokens).
None is a multiple of the workgroup's rows, so the last workgroup is ragged.
k = 1280 is 20 block pairs per row: one full round of 16 pairs and a partial one;
k = 256 is a single partial round. T covers one and two token groups, full and ragged.
"""
import functools

import numpy as np
import pytest

import oracle
from quantized_weight_prefill_gguf_amd import synth
from tests import parity

pytestmark = pytest.mark.gpu

Q4_0, Q8_0 = synth.Q4_0, synth.Q8_0
PLAIN, RESIDUAL, SWIGLU = oracle.PLAIN, oracle.RESIDUAL, oracle.GATE_UP_SWIGLU
F32, F16 = 0, 1


@functools.lru_cache(maxsize=None)
def _weight(qtype, n, k, swiglu):
    if swiglu:
        return synth.gate_up_weight(qtype, n, k, workload_id=77)
    return synth.quantized_weight(qtype, n, k, workload_id=77)


def _case(gpu, qtype, n, k, T, epi, leg=0):
    W = _weight(qtype, n, k, epi == SWIGLU)
    X = synth.activations(T, k, workload_id=77)
    R = synth.activations(T, n, workload_id=77, tensor_id=synth.TENSOR_R) if epi == RESIDUAL else None
    assert gpu.select_path(qtype, n, k, T, epi, leg) == gpu.PF_PATH_GEMV
    print("case mfma-gemv qtype=%d n=%d k=%d T=%d epi=%d leg=%d" % (qtype, n, k, T, epi, leg), flush=True)
    Y = parity.run_gpu(gpu, qtype, W, n, k, X, epi, leg, R=R)
    ok, err = parity.check(qtype, W, n, k, X, Y, epi, leg, R=R)
    assert ok, "parity failed: metric %.3e" % err
    return W, X, R, Y


SHAPES = [(PLAIN, 100), (PLAIN, 8200), (PLAIN, 12290), (PLAIN, 16390),
          (RESIDUAL, 100), (RESIDUAL, 12290),
          (SWIGLU, 100), (SWIGLU, 8200), (SWIGLU, 12290)]


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
def test_every_token_count(gpu, qtype, T):
    for epi in (PLAIN, RESIDUAL, SWIGLU):
        _case(gpu, qtype, 100, 1280, T, epi)


@pytest.mark.parametrize("n", [100, 12290])
@pytest.mark.parametrize("T", [3, 4])
@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
def test_f16_leg_swiglu(gpu, qtype, T, n):
    """The f16 leg's GEMV (SwiGLU up to 4 rows) runs the same f32 kernel; its bar holds."""
    _case(gpu, qtype, n, 1280, T, SWIGLU, leg=F16)


@pytest.mark.parametrize("T", [1, 4, 5, 8])
@pytest.mark.parametrize("epi,n", SHAPES)
@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
def test_row_quads_and_ragged_rounds(gpu, qtype, epi, n, T):
    _case(gpu, qtype, n, 1280, T, epi)


@pytest.mark.parametrize("epi", [PLAIN, RESIDUAL, SWIGLU])
@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
def test_single_partial_round(gpu, qtype, epi):
    _case(gpu, qtype, 37, 256, 6, epi)


@pytest.mark.parametrize("k", [3072, 3328, 5120])
@pytest.mark.parametrize("T", [3, 4])
@pytest.mark.parametrize("epi", [PLAIN, RESIDUAL])
@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
def test_one_quad_many_rounds(gpu, qtype, epi, T, k):
    """Four compute waves of one row quad (4081 <= n <= 8160 at up to four tokens) over
    three, three and a quarter, and five rounds: the weight ring wraps and the last
    round is full or partial."""
    _case(gpu, qtype, 4100, k, T, epi)


@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
def test_bitwise_repeatable(gpu, qtype):
    W, X, R, Y = _case(gpu, qtype, 8200, 1280, 7, RESIDUAL)
    Y2 = parity.run_gpu(gpu, qtype, W, 8200, 1280, X, RESIDUAL, F32, R=R)
    assert np.array_equal(Y.view(np.uint32), Y2.view(np.uint32))
