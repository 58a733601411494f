"""Pass/fail rules for comparing a GEMM result with the fp64 oracle.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Tolerances (normalised by the norms of the two operands of each dot product):

    e = max_{t,r} |Y[t][r] - Y_ref[t][r]| / (||w_hat_r||_2 * ||x_t||_2)

must not exceed 1e-5 on the f32 leg and 2e-3 on the f16 leg. The f32 bound is what
true fp32 accumulation of exact fp32 products meets with a wide margin, and what a
reduced-precision (10-bit) input shortcut fails; the page aprender-serve
gdn_prefill_ops.rs (module doc, group 1) asks for fp32 in and out with no TF32 on
that leg. The f16 leg rounds both inputs to binary16 and accumulates in fp32.

Zero denominators (an all-zero weight row or activation row): the result must
equal the oracle exactly (0 for PLAIN, R for RESIDUAL, 0 for SWIGLU).

GATE_UP_SWIGLU has no single weight row, so the linear tolerance is carried
through the epilogue as an interval: with G = ||w_gate_r|| ||x_t||,
U = ||w_up_r|| ||x_t|| and the leg's tau, Y must lie in the exact range of
silu(g') * u' over g' in [g - tau G, g + tau G], u' in [u - tau U, u + tau U],
widened by 4 * 2^-24 * |Y_ref| for the f32 evaluation of silu and the product.
silu(g) = g * sigma(g) falls on (-inf, g*] and rises on [g*, inf), so the range on
an interval is found from its end points and g*.
"""
import numpy as np

TOL = {"f32": 1e-5, "f16": 2e-3}


def _silu(g):
    with np.errstate(over="ignore", invalid="ignore"):
        return g / (1.0 + np.exp(-g))


def _silu_argmin():
    # silu'(g) = sigma(g) * (1 + g * (1 - sigma(g))); its only zero is the minimum.
    def dsilu(g):
        s = 1.0 / (1.0 + np.exp(-g))
        return s * (1.0 + g * (1.0 - s))
    lo, hi = -2.0, -1.0  # dsilu(-2) < 0 < dsilu(-1)
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if dsilu(mid) < 0:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


G_STAR = _silu_argmin()
SILU_MIN = float(_silu(np.float64(G_STAR)))


def silu_range(a, b):
    """Exact [min, max] of silu over [a, b] (elementwise arrays, a <= b)."""
    sa, sb = _silu(a), _silu(b)
    lo = np.minimum(sa, sb)
    hi = np.maximum(sa, sb)
    inside = (a <= G_STAR) & (G_STAR <= b)
    lo = np.where(inside, SILU_MIN, lo)
    return lo, hi


def linear_error_elems(Y, Y_ref, den):
    """Normalised error of PLAIN/RESIDUAL results on matching element arrays.

    den = ||w_hat_r|| * ||x_t|| for each element. Returns (max normalised error
    over elements with den > 0, whether every den == 0 element equals the oracle
    rounded to f32).
    """
    Y = np.asarray(Y, np.float64)
    Y_ref = np.asarray(Y_ref, np.float64)
    den = np.broadcast_to(np.asarray(den, np.float64), Y.shape)
    if not np.all(np.isfinite(Y)):
        return np.inf, False
    diff = np.abs(Y - Y_ref)
    nz = den > 0
    err = float(np.max(diff[nz] / den[nz])) if np.any(nz) else 0.0
    exact_ok = bool(np.all(Y[~nz] == Y_ref[~nz].astype(np.float32).astype(np.float64)))
    return err, exact_ok


def linear_error(Y, Y_ref, wnorm, xnorm):
    """linear_error_elems for full [T][n] results: wnorm [n], xnorm [T]."""
    den = np.outer(np.asarray(xnorm, np.float64), np.asarray(wnorm, np.float64))
    return linear_error_elems(Y, Y_ref, den)


def check_linear(Y, Y_ref, wnorm, xnorm, leg):
    err, exact_ok = linear_error(Y, Y_ref, wnorm, xnorm)
    return (err <= TOL[leg] and exact_ok), err


def check_linear_elems(Y, Y_ref, den, leg):
    err, exact_ok = linear_error_elems(Y, Y_ref, den)
    return (err <= TOL[leg] and exact_ok), err


def swiglu_check_elems(Y, g, u, gden, uden, leg):
    """Interval check for SWIGLU outputs on matching element arrays.

    g, u: fp64 oracle gate and up products; gden = ||w_gate_r|| ||x_t||,
    uden = ||w_up_r|| ||x_t||. Returns (pass, first-order diagnostic ratio).
    """
    tau = TOL[leg]
    Y = np.asarray(Y, np.float64)
    g = np.asarray(g, np.float64)
    u = np.asarray(u, np.float64)
    G = tau * np.broadcast_to(np.asarray(gden, np.float64), Y.shape)
    U = tau * np.broadcast_to(np.asarray(uden, np.float64), Y.shape)
    if not np.all(np.isfinite(Y)):
        return False, np.inf
    s_lo, s_hi = silu_range(g - G, g + G)
    u_lo, u_hi = u - U, u + U
    prods = np.stack([s_lo * u_lo, s_lo * u_hi, s_hi * u_lo, s_hi * u_hi])
    lo = prods.min(axis=0)
    hi = prods.max(axis=0)
    y_ref = _silu(g) * u
    widen = 4.0 * 2.0 ** -24 * np.abs(y_ref)
    ok = bool(np.all((Y >= lo - widen) & (Y <= hi + widen)))
    # First-order diagnostic: |dY| / (|silu'(g)| |u| G + |silu(g)| U) at tau = 1.
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-g))
    dsilu = s * (1.0 + g * (1.0 - s))
    den = np.abs(dsilu) * np.abs(u) * G / tau + np.abs(_silu(g)) * U / tau
    diff = np.abs(Y - y_ref)
    nz = den > 0
    ratio = float(np.max(diff[nz] / den[nz])) if np.any(nz) else 0.0
    return ok, ratio


def swiglu_check(Y, g, u, gnorm, unorm, xnorm, leg):
    """swiglu_check_elems for full [T][n] results: gnorm, unorm [n], xnorm [T]."""
    xn = np.asarray(xnorm, np.float64)[:, None]
    return swiglu_check_elems(Y, g, u, xn * np.asarray(gnorm, np.float64)[None, :],
                              xn * np.asarray(unorm, np.float64)[None, :], leg)
