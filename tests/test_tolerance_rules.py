"""The pass/fail rules: what they accept and what they reject (CPU only).

Correct fp32 arithmetic must pass the f32 bound with a wide margin; a 10-bit input
shortcut, a dropped term, a sign slip or swapped gate/up operands must fail. These
plant the mistakes in CPU emulations built on the oracle's products.
"""
import numpy as np
import pytest

from oracle import tolerance
from quantized_weight_prefill_gguf_amd import synth

Q4_0, Q8_0 = synth.Q4_0, synth.Q8_0


def _round_mantissa(a, bits):
    """Round f32 values to `bits` explicit mantissa bits, nearest-even (emulation)."""
    a = np.asarray(a, np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    drop = 23 - bits
    half = np.uint64(1 << (drop - 1))
    lsb = (u >> np.uint64(drop)) & np.uint64(1)
    u = (u + half - np.uint64(1) + lsb) >> np.uint64(drop) << np.uint64(drop)
    return u.astype(np.uint32).view(np.float32)


@pytest.fixture(scope="module")
def case(oracle_lib):
    T, n, k = 64, 64, 4096
    W = synth.quantized_weight(Q4_0, n, k, workload_id=95)
    X = synth.activations(T, k, workload_id=95)
    w = oracle_lib.dequant_f32(Q4_0, W, n, k)
    ref = oracle_lib.matmul(Q4_0, W, n, k, X)
    wn = oracle_lib.row_norms(Q4_0, W, n, k)
    xn = np.linalg.norm(X.astype(np.float64), axis=1)
    return dict(T=T, n=n, k=k, W=W, X=X, w=w, ref=ref, wn=wn, xn=xn)


def _f32_sequential(X, w):
    """fp32 products, fp32 running sum in ascending k (one rounding per step)."""
    prods = (X[:, None, :] * w[None, :, :]).astype(np.float32)
    return np.add.accumulate(prods, axis=2, dtype=np.float32)[..., -1]


def test_true_fp32_accumulation_passes_with_margin(case):
    Y = _f32_sequential(case["X"], case["w"])
    ok, err = tolerance.check_linear(Y, case["ref"], case["wn"], case["xn"], "f32")
    assert ok and err < 1e-6, err


def test_tf32_like_inputs_fail_f32_leg(case):
    Y = _round_mantissa(case["X"], 10).astype(np.float64) @ _round_mantissa(case["w"], 10).astype(np.float64).T
    ok, err = tolerance.check_linear(Y, case["ref"], case["wn"], case["xn"], "f32")
    assert not ok and err > 1e-5, err


def test_fp16_inputs_pass_f16_leg_only(case):
    xh = case["X"].astype(np.float16).astype(np.float64)
    wh = case["w"].astype(np.float16).astype(np.float64)
    Y = (xh @ wh.T).astype(np.float32)
    ok16, err = tolerance.check_linear(Y, case["ref"], case["wn"], case["xn"], "f16")
    ok32, _ = tolerance.check_linear(Y, case["ref"], case["wn"], case["xn"], "f32")
    assert ok16 and not ok32, err


def test_dropped_term_fails(case):
    X = case["X"].copy()
    X[:, 1234] = 0.0  # one term of every dot product left out
    Y = X.astype(np.float64) @ case["w"].astype(np.float64).T
    ok, err = tolerance.check_linear(Y, case["ref"], case["wn"], case["xn"], "f32")
    assert not ok, err


def test_zero_denominator_needs_exact_result(case):
    ref = case["ref"].copy()
    wn = case["wn"].copy()
    ref[:, 3] = 0.0
    wn[3] = 0.0
    Y = ref.astype(np.float32).astype(np.float64)
    assert tolerance.check_linear(Y, ref, wn, case["xn"], "f32")[0]
    Y[5, 3] = 1e-30
    assert not tolerance.check_linear(Y, ref, wn, case["xn"], "f32")[0]


def test_residual_sign_slip_fails(case):
    R = synth.activations(case["T"], case["n"], workload_id=95, tensor_id=synth.TENSOR_R)
    good = R.astype(np.float64) + case["ref"]
    bad = (R.astype(np.float64) - case["ref"]).astype(np.float32)
    assert tolerance.check_linear(good.astype(np.float32), good, case["wn"], case["xn"], "f32")[0]
    assert not tolerance.check_linear(bad, good, case["wn"], case["xn"], "f16")[0]


def test_swiglu_interval(oracle_lib):
    T, n, k = 32, 48, 4096
    W = synth.gate_up_weight(Q4_0, n, k, workload_id=94)
    X = synth.activations(T, k, workload_id=94)
    acc = oracle_lib.matmul(Q4_0, W, 2 * n, k, X)
    g, u = acc[:, :n], acc[:, n:]
    norms = oracle_lib.row_norms(Q4_0, W, 2 * n, k)
    gn, un = norms[:n], norms[n:]
    xn = np.linalg.norm(X.astype(np.float64), axis=1)
    w = oracle_lib.dequant_f32(Q4_0, W, 2 * n, k)
    # fp32 sums, fp32 silu and product: passes the f32 rule
    a32 = _f32_sequential(X, w)
    g32, u32 = a32[:, :n], a32[:, n:]
    y32 = (g32 / (np.float32(1) + np.exp(-g32)) * u32).astype(np.float32)
    ok, ratio = tolerance.swiglu_check(y32, g, u, gn, un, xn, "f32")
    assert ok and ratio < 0.1, ratio
    # fp16 inputs: pass the f16 rule, fail the f32 rule
    ah = X.astype(np.float16).astype(np.float64) @ w.astype(np.float16).astype(np.float64).T
    gh, uh = ah[:, :n], ah[:, n:]
    yh = (gh / (1 + np.exp(-gh)) * uh).astype(np.float32)
    assert tolerance.swiglu_check(yh, g, u, gn, un, xn, "f16")[0]
    assert not tolerance.swiglu_check(yh, g, u, gn, un, xn, "f32")[0]
    # gate and up swapped: fails even the f16 rule
    ys = (u / (1 + np.exp(-u)) * g).astype(np.float32)
    assert not tolerance.swiglu_check(ys, g, u, gn, un, xn, "f16")[0]
    # a non-finite value fails
    y_bad = y32.copy()
    y_bad[0, 0] = np.nan
    assert not tolerance.swiglu_check(y_bad, g, u, gn, un, xn, "f16")[0]


def test_silu_range_is_exact_on_intervals():
    rng = np.random.default_rng(0)
    a = rng.uniform(-6, 4, 2000)
    b = a + rng.uniform(0, 3, 2000)
    lo, hi = tolerance.silu_range(a, b)
    grid = a[:, None] + (b - a)[:, None] * np.linspace(0, 1, 4001)[None, :]
    s = grid / (1 + np.exp(-grid))
    assert np.all(lo <= s.min(axis=1) + 1e-15)
    assert np.all(hi >= s.max(axis=1) - 1e-15)
    assert np.all(s.min(axis=1) - lo <= 1e-6)
    assert abs(tolerance.G_STAR + 1.2784645427610738) < 1e-12


def test_f32_output_rounding_is_admitted_and_nothing_more():
    """A residual far larger than the product's norms: the exact sum rounded once to
    f32 passes (no f32 value is nearer), the next f32 value beyond the interval's
    outward rounding fails, and so does a dropped product."""
    rng = np.random.default_rng(5)
    R = rng.standard_normal(4000)
    acc = rng.standard_normal(4000) * 1e-6          # |acc| << ulp(R)
    den = np.full(4000, 1e-6)                       # tau den = 1e-11 on the f32 leg
    ref = R + acc
    y = ref.astype(np.float32).astype(np.float64)
    assert np.max(np.abs(y - ref) / den) > 1e-5      # the old |Y - Y_ref| <= tau D fails it
    assert tolerance.check_linear_elems(y, ref, den, "f32")[0]
    hi = tolerance.f32_up(ref + 1e-5 * den)
    over = np.nextafter(hi.astype(np.float32), np.float32(np.inf)).astype(np.float64)
    for i in range(0, 4000, 397):
        y2 = y.copy()
        y2[i] = over[i]
        assert not tolerance.check_linear_elems(y2, ref, den, "f32")[0], i
    assert not tolerance.check_linear_elems(R.astype(np.float32), ref, np.full(4000, 1e-9), "f32")[0]


def test_f32_bounds_are_the_neighbouring_f32_values():
    v = np.array([1.0, 1.0 + 2.0 ** -30, -1.0 - 2.0 ** -30, 1e-50, -1e-50, 3e38 * 1.2])
    lo, hi = tolerance.f32_down(v), tolerance.f32_up(v)
    assert list(lo[:3]) == [1.0, 1.0, np.nextafter(np.float32(-1.0), np.float32(-2))]
    assert list(hi[:3]) == [1.0, np.nextafter(np.float32(1.0), np.float32(2)), -1.0]
    assert lo[3] == 0.0 and hi[3] == 2.0 ** -149 and lo[4] == -(2.0 ** -149) and hi[4] == 0.0
    assert lo[5] == np.finfo(np.float32).max and hi[5] == np.inf


def test_swiglu_f32_underflow_is_admitted():
    """g = -115.8 with a large u: any f32 silu(g) is 0 (e^-g overflows), so Y = 0 must
    pass although silu(g) u = -1.4e-42 is an f32 subnormal; the allowance is
    2^-120 (|u| + tau U) = 1.8e-30 here, so 1e-28 fails, and away from underflow
    nothing changes."""
    g = np.array([-115.84, -115.84, 3.0, -2.0])
    u = np.array([2.45433e6, 2.45433e6, 5.0, 7.0])
    gden = np.array([4.7e3, 4.7e3, 10.0, 10.0])
    uden = np.array([9.4e7, 9.4e7, 10.0, 10.0])
    yref = g / (1 + np.exp(-g)) * u
    ok, _ = tolerance.swiglu_check_elems(np.array([0.0, -0.0, yref[2], yref[3]]), g, u, gden, uden, "f32")
    assert ok
    bad = np.array([0.0, 1e-28, yref[2], yref[3]])
    assert not tolerance.swiglu_check_elems(bad, g, u, gden, uden, "f32")[0]
    bad = np.array([0.0, 0.0, yref[2] * (1 + 1e-3), yref[3]])
    assert not tolerance.swiglu_check_elems(bad, g, u, gden, uden, "f32")[0]
