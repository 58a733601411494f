"""Pins of the oracle's IQ4_XS decode, CPU only: hand-worked blocks
(tests/golden/iq4_xs_blocks.txt), each code against the grid the fixture lists, the
position of every scale bit and every code nibble as the layout places them (one at a
time), the binary16 leg as numpy's RNE of the f32 decode, the GEMM on one-hot rows
picking single weights, and the test-input encoder's round trip.
"""
import numpy as np
import pytest

import oracle
from quantized_weight_prefill_gguf_amd import synth
from tests.golden import hex_bytes, load

QT = synth.IQ4_XS
RAMP = np.array([(i % 16) | ((15 - i % 16) << 4) for i in range(128)], np.uint8)


def _fixture():
    grid, cases, cur = None, [], None
    for key, val in load("iq4_xs_blocks.txt"):
        if key == "grid":
            grid = np.array([float(v) for v in val.split()], np.float32)
        elif key == "case":
            cur = {"name": val}
            cases.append(cur)
        else:
            cur[key] = val
    return grid, cases


GRID, CASES = _fixture()


def _block(d=(0x00, 0x3C), scales_h=0, scales_l=(0, 0, 0, 0), qs=None):
    b = np.zeros(136, np.uint8)
    b[0:2] = d
    b[2] = scales_h & 0xFF
    b[3] = scales_h >> 8
    b[4:8] = scales_l
    b[8:136] = 0 if qs is None else qs
    return b


def _dequant(b):
    return oracle.dequant_f32(QT, b, 1, 256)[0]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c["name"])
def test_hand_worked_blocks(case):
    b = _block(d=tuple(hex_bytes(case["d"])), scales_h=int.from_bytes(hex_bytes(case["scales_h"]).tobytes(), "little"),
               scales_l=tuple(hex_bytes(case["scales_l"])), qs=RAMP)
    w = _dequant(b)
    for pair in case["expect"].split():
        e, v = pair.split(":")
        want = np.float32(float(v))
        got = w[int(e)]
        assert got == want and np.signbit(got) == np.signbit(want), (e, got, want)


def _ls33():
    """Every sub-block scale 33 (d (ls - 32) = d): low nibbles 1, top bits 2."""
    return 0xAAAA, (0x11, 0x11, 0x11, 0x11)


def test_each_code_selects_its_grid_value():
    sh, sl = _ls33()
    for code in range(16):
        qs = np.zeros(128, np.uint8)
        qs[0] = code                 # element 0
        qs[16 * 3 + 5] = code << 4   # element 32 * 3 + 16 + 5
        w = _dequant(_block(scales_h=sh, scales_l=sl, qs=qs))
        assert w[0] == GRID[code] and w[96 + 21] == GRID[code], code
        rest = np.delete(w, [0, 117])
        assert np.all(rest == GRID[0]), code   # every other code is 0


def test_grid_is_strictly_increasing_and_spans_the_nibble():
    assert GRID.size == 16 and np.all(np.diff(GRID) > 0)
    assert GRID[0] == -127 and GRID[-1] < 127


def test_scale_bit_positions():
    """Bit i of sub-block b's 6-bit scale sits in nibble b % 2 of scales_l[b / 2] (i < 4)
    or in bit 2b + i - 4 of scales_h (i >= 4); with every code 8 (grid value 1) a
    sub-block's weights equal d (ls - 32)."""
    qs = np.full(128, 0x88, np.uint8)
    for b in range(8):
        for i in range(6):
            sl = [0, 0, 0, 0]
            sh = 0
            if i < 4:
                sl[b // 2] = (1 << i) << (4 * (b % 2))
            else:
                sh = 1 << (2 * b + i - 4)
            w = _dequant(_block(scales_h=sh, scales_l=tuple(sl), qs=qs)).reshape(8, 32)
            want = np.full((8, 32), -32.0, np.float32)
            want[b] = (1 << i) - 32
            assert np.array_equal(w, want), (b, i)


def test_code_nibble_positions():
    """qs[16 b + j]: its low nibble is element 32 b + j, its high nibble 32 b + 16 + j."""
    sh, sl = _ls33()
    base = np.full(128, 0x88, np.uint8)   # code 8 everywhere: grid 1
    for b in range(8):
        for j in range(16):
            for high in (False, True):
                qs = base.copy()
                qs[16 * b + j] = 0x8F if not high else 0xF8   # code 15 (113) in one nibble
                w = _dequant(_block(scales_h=sh, scales_l=sl, qs=qs))
                want = np.ones(256, np.float32)
                want[32 * b + 16 * high + j] = 113.0
                assert np.array_equal(w, want), (b, j, high)


def test_f16_leg_is_rne_of_f32_decode():
    W = synth.quantize(QT, synth.weights_f32(37, 512, workload_id=31))
    w32 = oracle.dequant_f32(QT, W, 37, 512)
    w16 = oracle.dequant_f16(QT, W, 37, 512)
    assert np.array_equal(w16, w32.astype(np.float16).view(np.uint16))


def test_one_hot_rows_pick_weights():
    rows, k = 9, 768
    W = synth.quantize(QT, synth.weights_f32(rows, k, workload_id=32))
    cols = [(7 * t + 3) % k for t in range(k // 3)]
    X = np.zeros((len(cols), k), np.float32)
    X[np.arange(len(cols)), cols] = 1.0
    y = oracle.matmul(QT, W, rows, k, X)
    w = oracle.dequant_f32(QT, W, rows, k)
    assert np.array_equal(y, w[:, cols].T.astype(np.float64))


def test_encoder_round_trip_error():
    """The test-input encoder and the decode agree: N(0, 0.02) weights come back within
    the error a 16-level non-linear grid allows (relative RMS)."""
    w = synth.weights_f32(64, 2048, workload_id=33)
    d = oracle.dequant_f32(QT, synth.quantize(QT, w), 64, 2048)
    rel = np.sqrt(np.mean((d - w) ** 2) / np.mean(w ** 2))
    assert rel < 0.11, rel
