"""Pass/fail rules for comparing a GEMM result with the fp64 oracle.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Tolerances (normalised by the norms of the two operands of each dot product):

    e = max_{t,r} |Y[t][r] - Y_ref[t][r]| / (||w_hat_r||_2 * ||x_t||_2)

must not exceed 1e-5 on the f32 leg and 2e-3 on the f16 leg. The f32 bound is what
true fp32 accumulation of exact fp32 products meets with a wide margin, and what a
reduced-precision (10-bit) input shortcut fails; the page aprender-serve
gdn_prefill_ops.rs (module doc, group 1) asks for fp32 in and out with no TF32 on
that leg. The f16 leg rounds both inputs to binary16 and accumulates in fp32.

The output is f32 (the pages fix the projection's output type), so no result can
lie nearer to the exact value than the f32 numbers next to it. A PLAIN or RESIDUAL
element therefore passes iff it lies in [Y_ref - tau D, Y_ref + tau D] (D = the
norm product above) rounded outward to f32: from the largest f32 <= the lower end
to the smallest f32 >= the upper end. This differs from |Y - Y_ref| <= tau D only
where f32 cannot hold the interval: an element whose R dwarfs D (its sum R + acc
must round to an f32 ulp of R), or a product below the f32 range. The reported
metric stays max |Y - Y_ref| / D, a diagnostic.

Zero denominators (an all-zero weight row or activation row): the result must
equal the oracle exactly (0 for PLAIN, R for RESIDUAL, 0 for SWIGLU).

GATE_UP_SWIGLU has no single weight row, so the linear tolerance is carried
through the epilogue as an interval: with G = ||w_gate_r|| ||x_t||,
U = ||w_up_r|| ||x_t|| and the leg's tau, Y must lie in the exact range of
silu(g') * u' over g' in [g - tau G, g + tau G], u' in [u - tau U, u + tau U],
widened for the f32 evaluation of silu and the product: by 4 * 2^-24 * |Y_ref|,
and by 2^-120 * (|u| + tau U) for silu's own f32 range: below g = -88.72, e^-g
overflows f32 and silu(g) = g / (1 + e^-g) is 0, where the exact value is at most
88.72 e^-88.72 < 2^-120 in magnitude. silu(g) = g * sigma(g) falls on (-inf, g*]
and rises on [g*, inf), so the range on an interval is found from its end points
and g*. The widened range, too, is rounded outward to f32.
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


# |silu(g)| where e^-g overflows f32 (g = -ln(2^128)) is below this bound; an f32
# evaluation of silu may return 0 for anything smaller.
SILU_F32_FLOOR = 2.0 ** -120

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


def f32_down(v):
    """The largest f32 value <= v (fp64 array), as fp64."""
    v = np.asarray(v, np.float64)
    with np.errstate(over="ignore"):
        f = v.astype(np.float32)
    f = np.where(f.astype(np.float64) > v, np.nextafter(f, np.float32(-np.inf)), f)
    return f.astype(np.float64)


def f32_up(v):
    """The smallest f32 value >= v (fp64 array), as fp64."""
    return -f32_down(-np.asarray(v, np.float64))


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


def linear_fits_elems(Y, Y_ref, den, leg):
    """Whether every element with den > 0 lies in [Y_ref - tau den, Y_ref + tau den]
    rounded outward to f32."""
    Y = np.asarray(Y, np.float64)
    Y_ref = np.asarray(Y_ref, np.float64)
    den = np.broadcast_to(np.asarray(den, np.float64), Y.shape)
    nz = den > 0
    r = TOL[leg] * den[nz]
    return bool(np.all((Y[nz] >= f32_down(Y_ref[nz] - r)) & (Y[nz] <= f32_up(Y_ref[nz] + r))))


def check_linear(Y, Y_ref, wnorm, xnorm, leg):
    den = np.outer(np.asarray(xnorm, np.float64), np.asarray(wnorm, np.float64))
    return check_linear_elems(Y, Y_ref, den, leg)


def check_linear_elems(Y, Y_ref, den, leg):
    err, exact_ok = linear_error_elems(Y, Y_ref, den)
    if not np.isfinite(err):
        return False, err
    return (exact_ok and linear_fits_elems(Y, Y_ref, den, leg)), err


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
    widen = 4.0 * 2.0 ** -24 * np.abs(y_ref) + SILU_F32_FLOOR * (np.abs(u) + U)
    ok = bool(np.all((Y >= f32_down(lo - widen)) & (Y <= f32_up(hi + widen))))
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
