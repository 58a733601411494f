"""CPU checks of the random edge-scale blocks the further-type parity tests use
(tests/xq_blocks.py): on the f16 leg's bound every decoded weight is binary16-finite
(|w| <= 65504), and the scale fields take both signs and the subnormal and zero
edge values."""
import numpy as np
import pytest

import oracle
from quantized_weight_prefill_gguf_amd import synth
from tests import xq_blocks

TYPES = [synth.F16, synth.Q4_K, synth.Q5_K, synth.Q6_K, synth.IQ4_XS]


@pytest.mark.parametrize("qtype", TYPES)
def test_f16_leg_bound_keeps_weights_finite(qtype):
    rows, k = 70, 2048
    W = xq_blocks.weight(qtype, rows, k, 600 + qtype, xq_blocks.TOP["f16"][qtype])
    w = oracle.dequant_f32(qtype, W, rows, k)
    assert np.all(np.isfinite(w)) and np.max(np.abs(w)) <= 65504.0


@pytest.mark.parametrize("qtype", [synth.Q4_K, synth.Q5_K, synth.Q6_K, synth.IQ4_XS])
def test_scale_fields_take_edge_values(qtype):
    rows, k = 70, 2048
    W = xq_blocks.weight(qtype, rows, k, 600 + qtype, xq_blocks.TOP["f16"][qtype])
    blk = W.reshape(rows * (k // 256), synth.BLOCK_BYTES[qtype])
    at = 208 if qtype == synth.Q6_K else 0
    d = blk[:, at].astype(np.uint16) | (blk[:, at + 1].astype(np.uint16) << 8)
    mag = d & 0x7FFF
    assert np.any(d >> 15) and np.any((d >> 15) == 0)
    for edge in (0x0001, 0x03FF, 0x0000):
        assert np.any(mag == edge), hex(edge)
