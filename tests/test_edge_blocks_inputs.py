"""The adversarial block generator (tests/edge_blocks.py) covers what its parity test
relies on, checked through the oracle's decode (CPU only)."""
import numpy as np
import pytest

import oracle
from quantized_weight_prefill_gguf_amd import synth
from tests import edge_blocks


@pytest.mark.parametrize("leg", ["f32", "f16"])
@pytest.mark.parametrize("qtype", [synth.Q4_0, synth.Q8_0])
def test_edge_blocks_cover_codes_scales_and_range(oracle_lib, qtype, leg):
    rows, k = 80, 2560
    B = synth.BLOCK_BYTES[qtype]
    W = edge_blocks.weight(qtype, rows, k, leg, 1234)
    blk = W.reshape(rows, k // 32, B)
    codes = blk[:, :, 2:]
    assert np.unique(codes).size == 256                     # every byte, 0x80 (-128) included
    d = blk[:, :, 0].astype(np.uint16) | (blk[:, :, 1].astype(np.uint16) << 8)
    for m in edge_blocks.scales(leg, qtype):
        for sgn in (0, 0x8000):
            assert np.any(d == (m | sgn)), hex(m | sgn)
    w16 = oracle.dequant_f16(qtype, W, rows, k).view(np.uint16)
    w32 = oracle.dequant_f32(qtype, W, rows, k)
    assert np.all(np.isfinite(w32))
    if leg == "f16":
        # RNE_fp16(d q) stays finite and reaches the largest finite binary16 value
        assert not np.any((w16 & 0x7C00) == 0x7C00)
        assert np.max(np.abs(w32)) == 65504.0
    else:
        assert np.max(np.abs(w32)) == 65504.0 * (8 if qtype == synth.Q4_0 else 128)
    # the fp16 weights include subnormals (the MFMA must take them as they are)
    assert np.any(((w16 & 0x7C00) == 0) & ((w16 & 0x3FF) != 0))
    # rows r % 7 == 5 (r < 14) have a zero scale in every block: all weights +-0
    for r in (5, 12):
        assert np.all(w32.reshape(rows, k)[r] == 0)
