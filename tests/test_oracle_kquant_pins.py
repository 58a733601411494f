"""Pins of the oracle's decode of the further GGUF weight types (F16, Q4_K, Q5_K,
Q6_K), CPU only: hand-worked blocks (tests/golden/k_quant_blocks.txt), the position
of every code bit as the layout places it (one bit at a time), the binary16 leg as
numpy's RNE of the f32 decode, and the GEMM on one-hot rows picking single weights.
"""
import numpy as np
import pytest

import oracle
from quantized_weight_prefill_gguf_amd import synth
from tests.golden import hex_bytes, load

QT = {"q4_k": synth.Q4_K, "q5_k": synth.Q5_K, "q6_k": synth.Q6_K, "f16": synth.F16}
RAMP = np.array([(i % 16) | ((15 - i % 16) << 4) for i in range(128)], np.uint8)


def _cases():
    cases, cur = [], None
    for key, val in load("k_quant_blocks.txt"):
        if key == "case":
            cur = {"name": val}
            cases.append(cur)
        else:
            cur[key] = val
    return cases


def _block(case):
    """The block bytes of a fixture case, field by field."""
    name = case["name"]
    if name == "f16":
        b = np.zeros(64, np.uint8)
        for i, h in enumerate(case["halves"].split()):
            v = int(h, 16)
            b[2 * i], b[2 * i + 1] = v & 0xFF, v >> 8
        return b
    if name == "q6_k":
        b = np.zeros(210, np.uint8)
        b[0:128] = RAMP
        b[128 + 5] = hex_bytes(case["qh5"])[0]
        b[192:208] = hex_bytes(case["scales"])
        b[208:210] = hex_bytes(case["d"])
        return b
    b = np.zeros(144 if name == "q4_k" else 176, np.uint8)
    b[0:2] = hex_bytes(case["d"])
    b[2:4] = hex_bytes(case["dmin"])
    b[4:16] = hex_bytes(case["scales"])
    if name == "q5_k":
        b[16 + 3] = hex_bytes(case["qh3"])[0]
        b[16 + 31] = hex_bytes(case["qh31"])[0]
        b[48:176] = RAMP
    else:
        b[16:144] = RAMP
    return b


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_hand_worked_blocks(oracle_lib, case):
    qt = QT[case["name"]]
    blk = _block(case)
    k = synth.BLOCK_ELEMS[qt]
    w = oracle_lib.dequant_f32(qt, blk, 1, k)[0]
    for pair in case["expect"].split():
        e, v = pair.split(":")
        want = np.float32(float(v))
        got = w[int(e)]
        assert got == want and np.signbit(got) == np.signbit(want), (case["name"], e, got, want)


def _unit_k_block(qt):
    """A K super-block whose every weight is exactly its code (Q4_K / Q5_K: d = 1,
    dmin = 0, all s_j = 1) or 1 x (code - 32) (Q6_K: d = 1, every scale 1)."""
    if qt == synth.Q6_K:
        b = np.zeros(210, np.uint8)
        b[192:208] = 1
        b[208:210] = [0x00, 0x3C]
        return b
    b = np.zeros(144 if qt == synth.Q4_K else 176, np.uint8)
    b[0:2] = [0x00, 0x3C]
    b[4:8] = 1           # s_0..3 = 1, and no top bits for s_4..7 / m_4..7
    b[12:16] = 1         # s_4..7 low nibble 1, m_4..7 low nibble 0
    return b


def test_q4_k_nibble_positions(oracle_lib):
    """qs[32 p + l]: its low nibble is element 64 p + l, its high nibble 64 p + 32 + l."""
    base = _unit_k_block(synth.Q4_K)
    for p in range(4):
        for l in range(32):
            for high, e in ((False, 64 * p + l), (True, 64 * p + 32 + l)):
                b = base.copy()
                b[16 + 32 * p + l] = 0x30 if high else 0x03
                w = oracle_lib.dequant_f32(synth.Q4_K, b, 1, 256)[0]
                want = np.zeros(256, np.float32)
                want[e] = 3.0
                assert np.array_equal(w, want), (p, l, high)


def test_q5_k_high_bit_positions(oracle_lib):
    """Bit b of qh[l] adds 16 to element 32 b + l, nothing else."""
    base = _unit_k_block(synth.Q5_K)
    for b_ in range(8):
        for l in range(32):
            b = base.copy()
            b[16 + l] = 1 << b_
            w = oracle_lib.dequant_f32(synth.Q5_K, b, 1, 256)[0]
            want = np.zeros(256, np.float32)
            want[32 * b_ + l] = 16.0
            assert np.array_equal(w, want), (b_, l)


def test_q6_k_code_positions(oracle_lib):
    """Element 128 h + 32 c + l: low 4 bits in ql[64 h + l + 32 (c % 2)] (low nibble for
    c < 2, high for c >= 2), top 2 bits at bits 2c, 2c+1 of qh[32 h + l]."""
    base = _unit_k_block(synth.Q6_K)
    zero = oracle_lib.dequant_f32(synth.Q6_K, base, 1, 256)[0]
    assert np.all(zero == -32.0)
    for h in range(2):
        for c in range(4):
            for l in range(32):
                e = 128 * h + 32 * c + l
                b = base.copy()
                b[64 * h + l + 32 * (c % 2)] = 0x50 if c >= 2 else 0x05   # low bits 5
                b[128 + 32 * h + l] = 2 << (2 * c)                         # top bits 2
                w = oracle_lib.dequant_f32(synth.Q6_K, b, 1, 256)[0]
                want = np.full(256, -32.0, np.float32)
                want[e] = 5 + 32 - 32
                assert np.array_equal(w, want), (h, c, l)


def test_k_scale_fields_round_trip(oracle_lib):
    """Every (s_j, m_j) in 0..63 placed by the packer is read back by the decode, with
    the other sub-blocks untouched (weights = s_j q - m_j on codes q = 1)."""
    rng = np.random.default_rng(3)
    for trial in range(64):
        s = rng.integers(0, 64, 8)
        m = rng.integers(0, 64, 8)
        b = np.zeros(144, np.uint8)
        b[0:2] = [0x00, 0x3C]
        b[2:4] = [0x00, 0x3C]
        b[4:16] = synth.pack_k_scales(s, m)
        b[16:144] = 0x11
        w = oracle_lib.dequant_f32(synth.Q4_K, b, 1, 256)[0].reshape(8, 32)
        assert np.array_equal(w, np.repeat((s - m).astype(np.float32)[:, None], 32, axis=1)), trial


@pytest.mark.parametrize("qt", [synth.F16, synth.Q4_K, synth.Q5_K, synth.Q6_K])
def test_f16_leg_is_rne_of_f32_decode(oracle_lib, qt):
    W = synth.quantize(qt, synth.weights_f32(37, 512, workload_id=31))
    w32 = oracle_lib.dequant_f32(qt, W, 37, 512)
    w16 = oracle_lib.dequant_f16(qt, W, 37, 512)
    assert np.array_equal(w16, w32.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("qt", [synth.F16, synth.Q4_K, synth.Q5_K, synth.Q6_K])
def test_one_hot_rows_pick_weights(oracle_lib, qt):
    rows, k = 9, 768
    W = synth.quantize(qt, synth.weights_f32(rows, k, workload_id=32))
    cols = [(7 * t + 3) % k for t in range(k // 3)]
    X = np.zeros((len(cols), k), np.float32)
    X[np.arange(len(cols)), cols] = 1.0
    y = oracle_lib.matmul(qt, W, rows, k, X)
    w = oracle_lib.dequant_f32(qt, W, rows, k)
    assert np.array_equal(y, w[:, cols].T.astype(np.float64))


@pytest.mark.parametrize("qt,bound", [(synth.Q4_K, 0.09), (synth.Q5_K, 0.045), (synth.Q6_K, 0.025),
                                      (synth.F16, 0.0005)])
def test_encoder_round_trip_error(oracle_lib, qt, bound):
    """The test-input encoders and the decode agree: N(0, 0.02) weights come back
    within the quantisation error the bit widths allow (relative RMS)."""
    w = synth.weights_f32(64, 2048, workload_id=33)
    d = oracle_lib.dequant_f32(qt, synth.quantize(qt, w), 64, 2048)
    rel = np.sqrt(np.mean((d - w) ** 2) / np.mean(w ** 2))
    assert rel < bound, rel
