"""Pins of the CPU oracle to things other than itself (runs without a GPU).

Each test ties one part of the oracle to the block definitions, a library routine,
a closed form or a printed worked example, so that a dropped term, a wrong sign or
index, or a transposed operand in the oracle fails here.
"""
import numpy as np
import pytest
import torch

from quantized_weight_prefill_gguf_amd import synth
from tests.golden import floats, hex_bytes, load

Q4_0, Q8_0 = synth.Q4_0, synth.Q8_0


# --------------------------------------------------------------------------- fp16

def test_fp16_decode_exhaustive_against_numpy(oracle_lib):
    """All 65,536 binary16 patterns decode as numpy.float16 does."""
    h = np.arange(65536, dtype=np.uint16)
    got = oracle_lib.fp16_to_f64(h)
    ref = h.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _f32_neighbours(x):
    x = np.asarray(x, np.float32)
    up = np.nextafter(x, np.float32(np.inf))
    dn = np.nextafter(x, np.float32(-np.inf))
    return np.concatenate([x, up, dn])


def test_fp16_encode_against_numpy():
    """RNE to binary16: every fp16 value, every halfway tie and +-1 f32 ulp around
    both, the subnormal range, the overflow threshold and random magnitudes."""
    import oracle
    h = np.arange(65536, dtype=np.uint16)
    v = h.view(np.float16)
    fin = np.isfinite(v)
    vals = v[fin].astype(np.float32)
    # exact fp16 values map to themselves (including -0.0)
    assert np.array_equal(oracle.f32_to_fp16(vals), h[fin])
    # halfway points between consecutive positive fp16 values are exact in f32
    pos = np.sort(np.unique(np.abs(v[fin].astype(np.float64))))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)
    probe = _f32_neighbours(np.concatenate([mids, -mids, vals]))
    rng = np.random.default_rng(7)
    rand = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 12, 200000))).astype(np.float32)
    extra = np.array([65504, 65519.996, 65520, 65536, 1e9, 2.0 ** -24, 2.0 ** -25,
                      2.0 ** -25 * 1.0000001, 2.0 ** -26, 1e-30, 0.0], np.float32)
    probe = np.concatenate([probe, rand, _f32_neighbours(extra), -extra])
    ref = probe.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f32_to_fp16(probe), ref)


# --------------------------------------------------------------------------- decode

def _golden_blocks(name):
    items = load(name)
    qtype = {"q4_0": Q4_0, "q8_0": Q8_0}[dict(items)["qtype"]]
    cases = []
    cur = {}
    for key, val in items:
        if key == "block_hex":
            cur = {"block": hex_bytes(val)}
        elif key == "values":
            cur["values"] = floats(val)
        elif key == "sum":
            cur["sum"] = float(val)
            cases.append(cur)
    return qtype, cases


@pytest.mark.parametrize("name", ["q4_0_nibble_order.txt", "q8_0_sign.txt"])
def test_decode_hand_worked_blocks(oracle_lib, name):
    """Hand-worked blocks decode to the printed values, bit for bit (signed zeros too)."""
    qtype, cases = _golden_blocks(name)
    assert cases
    for c in cases:
        got = oracle_lib.dequant_f32(qtype, c["block"], 1, 32)[0]
        assert np.array_equal(got.view(np.uint32), c["values"].view(np.uint32)), (got, c["values"])
        assert float(np.sum(got.astype(np.float64))) == c["sum"]


def test_decode_one_hot_picks_single_weight(oracle_lib):
    """x = e_0 gives -8 d and x = e_16 gives 7 d for the nibble-order block."""
    qtype, cases = _golden_blocks("q4_0_nibble_order.txt")
    blk = cases[0]["block"]
    for idx, expect in [(0, -8.0), (16, 7.0), (15, 7.0), (31, -8.0)]:
        x = np.zeros((1, 32), np.float32)
        x[0, idx] = 1.0
        y = oracle_lib.matmul(qtype, blk, 1, 32, x)
        assert y[0, 0] == expect


def test_zero_weight_block_from_page(oracle_lib):
    """The page's zero-weight Q4_0 blocks give Y = 0, R, 0 for the three epilogues."""
    items = dict(load("q4_0_zero_weight_batch12.txt"))
    blk = hex_bytes(items["block_hex"])
    T, k, n = int(items["T"]), int(items["k"]), int(items["n"])
    W = np.tile(blk, n * (k // 32))
    W2 = np.tile(blk, 2 * n * (k // 32))
    X = np.full((T, k), float(items["x_fill"]), np.float32)
    R = synth.activations(T, n, tensor_id=synth.TENSOR_R)
    assert np.all(oracle_lib.gemm(Q4_0, W, n, k, X, oracle_lib.PLAIN) == float(items["expected_plain"]))
    assert np.array_equal(oracle_lib.gemm(Q4_0, W, n, k, X, oracle_lib.RESIDUAL, R), R.astype(np.float64))
    assert np.all(oracle_lib.gemm(Q4_0, W2, n, k, X, oracle_lib.GATE_UP_SWIGLU) == float(items["expected_swiglu"]))
    assert np.array_equal(W[: 18 * 4], synth.zero_q4_0(4, 32))


SCALES = [  # binary16 bits, value written out by hand
    (0x3C00, 1.0), (0xBC00, -1.0), (0x0001, 2.0 ** -24), (0x03FF, 1023 * 2.0 ** -24),
    (0x0400, 2.0 ** -14), (0x7BFF, 65504.0), (0x0000, 0.0), (0x8000, -0.0),
    (0x3555, 0.333251953125), (0xC800, -8.0),
]


@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
def test_decode_scale_handling(oracle_lib, qtype):
    """Every element equals float32(d) * float32(integer) with d written by hand;
    the product is exact in f32, so the bits (and the sign of zero) are fixed."""
    rng = np.random.default_rng(3)
    for bits, dval in SCALES:
        if qtype == Q4_0:
            q = rng.integers(0, 16, 32)
            q[:2] = [8, 0]
            qs = (q[:16] | (q[16:] << 4)).astype(np.uint8)
            ints = q - 8
        else:
            q = rng.integers(-128, 128, 32)
            q[:3] = [0, -128, 127]
            qs = q.astype(np.int8).view(np.uint8)
            ints = q
        blk = np.concatenate([np.array([bits & 0xFF, bits >> 8], np.uint8), qs])
        got = oracle_lib.dequant_f32(qtype, blk, 1, 32)[0]
        exp = np.float32(dval) * ints.astype(np.float32)
        assert np.array_equal(got.view(np.uint32), exp.view(np.uint32)), (hex(bits), got, exp)


@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
def test_dequant_f16_is_rne_of_f32_decode(oracle_lib, qtype):
    """The f16-leg weights are numpy's RNE float16 cast of the exact f32 decode."""
    W = synth.quantized_weight(qtype, 64, 256, workload_id=99)
    f32 = oracle_lib.dequant_f32(qtype, W, 64, 256)
    f16 = oracle_lib.dequant_f16(qtype, W, 64, 256)
    assert np.array_equal(f16, f32.astype(np.float16).view(np.uint16))


# --------------------------------------------------------------------------- quantizer

@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
def test_quantizer_round_trip_bounds(oracle_lib, qtype):
    rows, k = 64, 4096
    w = synth.weights_f32(rows, k, workload_id=98)
    W = synth.quantize(qtype, w)
    bb = synth.BLOCK_BYTES[qtype]
    assert W.size == rows * (k // 32) * bb
    blocks = W.reshape(rows, k // 32, bb)
    d = blocks[..., 0:2].copy().view(np.uint16)[..., 0].view(np.float16).astype(np.float64)
    what = oracle_lib.dequant_f32(qtype, W, rows, k).reshape(rows, k // 32, 32).astype(np.float64)
    wb = w.reshape(rows, k // 32, 32).astype(np.float64)
    err = np.abs(wb - what)
    ad = np.abs(d)[..., None]
    slack = 1e-5
    if qtype == Q8_0:
        assert np.all(err <= ad * (0.5 + slack))
        # the largest element maps to |q| = 127
        q = blocks[..., 2:].view(np.int8)
        assert np.all(np.max(np.abs(q.astype(np.int32)), axis=2) == 127)
    else:
        ratio = wb / d[..., None]
        inner = ratio <= 7.5
        assert np.all(err[inner] <= np.broadcast_to(ad, err.shape)[inner] * (0.5 + slack))
        assert np.all(err <= ad * 1.005)
        # the largest-magnitude element maps to nibble 0 (value -8 d)
        idx = np.argmax(np.abs(wb), axis=2)
        qv = np.take_along_axis(what, idx[..., None], axis=2)[..., 0]
        assert np.array_equal(qv, -8.0 * d)
    # idempotence: re-encoding the decoded weight reproduces the bytes
    again = synth.quantize(qtype, what.reshape(rows, k).astype(np.float32))
    assert np.array_equal(again, W)


# --------------------------------------------------------------------------- GEMM

def _blocks_from_codes(qtype, q, d16):
    """Pack integer codes q [rows][k] and fp16 scales d16 [rows][k/32] into blocks,
    following the GGUF block layout directly (independent of the oracle)."""
    rows, k = q.shape
    nb = k // 32
    qb = q.reshape(rows, nb, 32)
    sc = d16.astype(np.float16).view(np.uint16)
    lo = (sc & 0xFF).astype(np.uint8)[..., None]
    hi = (sc >> 8).astype(np.uint8)[..., None]
    if qtype == Q4_0:
        qs = (qb[..., :16] | (qb[..., 16:] << 4)).astype(np.uint8)
    else:
        qs = qb.astype(np.int8).view(np.uint8)
    return np.concatenate([lo, hi, qs], axis=2).reshape(-1)


def _random_codes(qtype, rows, k, seed):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 16, (rows, k)) if qtype == Q4_0 else rng.integers(-128, 128, (rows, k))
    d16 = (rng.uniform(0.5, 2.0, (rows, k // 32)) * 0.01).astype(np.float16)
    d16[0, 0] = -d16[0, 0]
    ints = q - 8 if qtype == Q4_0 else q
    w = (d16.astype(np.float64).repeat(32, axis=1) * ints)  # exact value of each weight
    return _blocks_from_codes(qtype, q, d16), w


@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
def test_gemm_identity_activations(oracle_lib, qtype):
    """X = I (T = k = 256) gives Y[t][r] = w_hat[r][t] exactly: pins orientation."""
    n, k = 40, 256
    W, w = _random_codes(qtype, n, k, 11)
    Y = oracle_lib.matmul(qtype, W, n, k, np.eye(k, dtype=np.float32))
    assert np.array_equal(Y, w.T)


@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
def test_gemm_rotated_one_hot(oracle_lib, qtype):
    n, k, T = 24, 512, 37
    W, w = _random_codes(qtype, n, k, 12)
    X = np.zeros((T, k), np.float32)
    cols = (7 * np.arange(T) + 3) % k
    X[np.arange(T), cols] = 1.0
    Y = oracle_lib.matmul(qtype, W, n, k, X)
    assert np.array_equal(Y, w[:, cols].T)


@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
@pytest.mark.parametrize("T,n,k", [(1, 1, 32), (5, 7, 64), (33, 17, 256), (64, 64, 320)])
def test_gemm_brute_force_against_numpy(oracle_lib, qtype, T, n, k):
    """The oracle's loops against numpy's fp64 matmul of weights built from codes."""
    W, w = _random_codes(qtype, n, k, 100 + T + n + k)
    X = synth.activations(T, k, workload_id=97)
    Y = oracle_lib.matmul(qtype, W, n, k, X)
    ref = X.astype(np.float64) @ w.T
    scale = np.outer(np.linalg.norm(X.astype(np.float64), axis=1), np.linalg.norm(w, axis=1))
    assert np.all(np.abs(Y - ref) <= 1e-13 * scale + 1e-300)
    # sampled entries agree bit for bit with the full product
    ti = np.arange(T).repeat(n)
    ri = np.tile(np.arange(n), T)
    assert np.array_equal(oracle_lib.matmul_sampled(qtype, W, n, k, X, ti, ri), Y.reshape(-1))
    assert np.allclose(oracle_lib.row_norms(qtype, W, n, k), np.linalg.norm(w, axis=1), rtol=1e-14)


def test_epilogues(oracle_lib):
    T, n, k = 9, 48, 256
    W, w = _random_codes(Q4_0, n, k, 21)
    X = synth.activations(T, k, workload_id=96)
    R = synth.activations(T, n, workload_id=96, tensor_id=synth.TENSOR_R)
    plain = oracle_lib.gemm(Q4_0, W, n, k, X, oracle_lib.PLAIN)
    res = oracle_lib.gemm(Q4_0, W, n, k, X, oracle_lib.RESIDUAL, R)
    assert np.array_equal(plain, oracle_lib.matmul(Q4_0, W, n, k, X))
    assert np.all(np.abs(res - (R.astype(np.float64) + plain)) <= 2.0 ** -52 * np.abs(res))
    # gate rows first, then up rows; fused == two plain products then silu(g) * u
    Wg, wg = _random_codes(Q4_0, n, k, 22)
    Wu, wu = _random_codes(Q4_0, n, k, 23)
    fused = oracle_lib.gemm(Q4_0, np.concatenate([Wg, Wu]), n, k, X, oracle_lib.GATE_UP_SWIGLU)
    g = oracle_lib.matmul(Q4_0, Wg, n, k, X)
    u = oracle_lib.matmul(Q4_0, Wu, n, k, X)
    ref = torch.nn.functional.silu(torch.from_numpy(g)).numpy() * u
    assert np.all(np.abs(fused - ref) <= 4 * 2.0 ** -52 * np.abs(ref))
    # swapping gate and up changes the answer (the operand order matters)
    swapped = oracle_lib.gemm(Q4_0, np.concatenate([Wu, Wg]), n, k, X, oracle_lib.GATE_UP_SWIGLU)
    assert not np.allclose(swapped, fused)


def test_linearity(oracle_lib):
    """Y(X1 + X2) = Y(X1) + Y(X2) with X1 + X2 exact in f32."""
    T, n, k = 6, 20, 256
    W, _ = _random_codes(Q8_0, n, k, 31)
    rng = np.random.default_rng(5)
    X1 = (rng.integers(-32, 33, (T, k)) / 8).astype(np.float32)
    X2 = (rng.integers(-32, 33, (T, k)) / 8).astype(np.float32)
    Y12 = oracle_lib.matmul(Q8_0, W, n, k, X1 + X2)
    Y1 = oracle_lib.matmul(Q8_0, W, n, k, X1)
    Y2 = oracle_lib.matmul(Q8_0, W, n, k, X2)
    scale = np.abs(Y1) + np.abs(Y2) + 1e-30
    assert np.all(np.abs(Y12 - (Y1 + Y2)) <= 1e-14 * scale)


def test_silu_against_torch(oracle_lib):
    g = np.linspace(-30, 30, 2001)
    ours = oracle_lib.silu(g)
    ref = torch.nn.functional.silu(torch.from_numpy(g)).numpy()
    assert np.all(np.abs(ours - ref) <= 4 * 2.0 ** -52 * np.abs(ref) + 1e-300)
    assert oracle_lib.silu(0.0) == 0.0


# --------------------------------------------------------------------------- RMSNorm

def test_rmsnorm_hand_worked(oracle_lib):
    """x = (3, 4), w = (1, 2), eps = 0: mean square 12.5, so x / sqrt(12.5) * w =
    (3 sqrt(2) / 5, 8 sqrt(2) / 5)."""
    got = oracle_lib.rmsnorm(np.array([[3.0, 4.0]]), np.array([1.0, 2.0]), 0.0)
    assert np.allclose(got, [[3 * np.sqrt(2) / 5, 8 * np.sqrt(2) / 5]], rtol=1e-15, atol=0)


def test_rmsnorm_eps_inside_the_root(oracle_lib):
    """A row of ones with eps = 3: 1 / sqrt(1 + 3) = 0.5 exactly (eps added after the
    square root would give 0.25; a sum instead of a mean, 1 / sqrt(4 + 3))."""
    got = oracle_lib.rmsnorm(np.ones((1, 4)), np.array([1.0, -2.0, 4.0, 0.5]), 3.0)
    assert np.array_equal(got, [[0.5, -1.0, 2.0, 0.25]])


def test_rmsnorm_closed_forms(oracle_lib):
    rng = np.random.default_rng(5)
    X = rng.normal(0, 1, (6, 256))
    w = rng.uniform(0.5, 1.5, 256)
    # a constant row c: c / |c| * w exactly when eps = 0
    C = np.outer([2.5, -0.75], np.ones(256))
    assert np.array_equal(oracle_lib.rmsnorm(C, w, 0.0), np.outer([1.0, -1.0], w))
    # invariant to a positive row scale when eps = 0
    assert np.allclose(oracle_lib.rmsnorm(3.7 * X, w, 0.0), oracle_lib.rmsnorm(X, w, 0.0), rtol=1e-14)
    # unit weight, eps = 0: every row has mean square 1
    ms = np.mean(oracle_lib.rmsnorm(X, np.ones(256), 0.0) ** 2, axis=1)
    assert np.allclose(ms, 1.0, rtol=1e-14)
    # a zero row stays zero for eps > 0
    assert np.array_equal(oracle_lib.rmsnorm(np.zeros((1, 256)), w, 1e-6), np.zeros((1, 256)))
    # the weight multiplies column by column (a transposed w would not broadcast here)
    Xn1 = oracle_lib.rmsnorm(X, np.ones(256), 1e-6)
    assert np.allclose(oracle_lib.rmsnorm(X, w, 1e-6), Xn1 * w[None, :], rtol=1e-15)


@pytest.mark.parametrize("qtype", [Q4_0, Q8_0])
def test_matmul_f64_against_c_oracle(oracle_lib, qtype):
    """On f32-representable activations the numpy fp64 product equals the C oracle's
    (both exact products, fp64 sums; differences are sum-order rounding only)."""
    n, k, T = 40, 512, 7
    W = synth.quantized_weight(qtype, n, k, workload_id=77)
    X = synth.activations(T, k, workload_id=77)
    a = oracle_lib.matmul_f64(qtype, W, n, k, X.astype(np.float64))
    b = oracle_lib.matmul(qtype, W, n, k, X)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------- argmax

def test_argmax_last_hand_cases(oracle_lib):
    am = oracle_lib.argmax_last
    assert am([1.0]) == 0
    assert am([0.5, 2.0, -3.0]) == 1
    assert am([2.0, 1.0, 2.0, 0.0]) == 2          # equal maxima: the last one
    assert am([-5.0, -1.0, -1.0, -7.0]) == 2      # all negative
    assert am([0.0, -0.0]) == 1                    # -0 == +0: a tie
    assert am([-0.0, 0.0]) == 1
    assert am(np.array([3, 9, 9, 9, 1], np.float32)) == 3


def test_argmax_last_against_numpy(oracle_lib):
    """Distinct values: numpy.argmax; with a planted tie, the later index."""
    rng = np.random.default_rng(11)
    x = rng.normal(0, 1, 1000).astype(np.float32)
    assert oracle_lib.argmax_last(x) == int(np.argmax(x))
    i = int(np.argmax(x))
    x[900 if i < 900 else 10] = x[i]
    assert oracle_lib.argmax_last(x) == max(i, 900 if i < 900 else 10)
