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


def linear_error(Y, Y_ref, wnorm, xnorm):
    """Normalised error of a PLAIN/RESIDUAL result.

    Y, Y_ref: [T][n]; wnorm: [n]; xnorm: [T]. Returns (max normalised error over
    elements with a nonzero denominator, all zero-denominator elements exact?).
    """
    Y = np.asarray(Y, np.float64)
    Y_ref = np.asarray(Y_ref, np.float64)
    den = np.outer(np.asarray(xnorm, np.float64), np.asarray(wnorm, np.float64))
    if not np.all(np.isfinite(Y)):
        return np.inf, False
    diff = np.abs(Y - Y_ref)
    nz = den > 0
    err = float(np.max(diff[nz] / den[nz])) if np.any(nz) else 0.0
    exact_ok = bool(np.all(Y[~nz] == Y_ref[~nz].astype(np.float32).astype(np.float64)))
    return err, exact_ok


def check_linear(Y, Y_ref, wnorm, xnorm, leg):
    err, exact_ok = linear_error(Y, Y_ref, wnorm, xnorm)
    return (err <= TOL[leg] and exact_ok), err


def swiglu_check(Y, g, u, gnorm, unorm, xnorm, leg):
    """Interval check for SWIGLU outputs.

    Y: [T][n] result; g, u: [T][n] fp64 oracle gate and up products; gnorm, unorm:
    [n] weight-row norms; xnorm: [T]. Returns (pass, first-order diagnostic ratio).
    """
    tau = TOL[leg]
    Y = np.asarray(Y, np.float64)
    g = np.asarray(g, np.float64)
    u = np.asarray(u, np.float64)
    xn = np.asarray(xnorm, np.float64)[:, None]
    G = tau * xn * np.asarray(gnorm, np.float64)[None, :]
    U = tau * xn * np.asarray(unorm, np.float64)[None, :]
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
    # First-order diagnostic: |dY| / (|silu'(g)| |u| G + |silu(g)| U).
    s = 1.0 / (1.0 + np.exp(-g))
    dsilu = s * (1.0 + g * (1.0 - s))
    den = np.abs(dsilu) * np.abs(u) * G / tau + np.abs(_silu(g)) * U / tau
    diff = np.abs(Y - y_ref)
    nz = den > 0
    ratio = float(np.max(diff[nz] / den[nz])) if np.any(nz) else 0.0
    return ok, ratio
