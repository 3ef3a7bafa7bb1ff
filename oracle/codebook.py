"""Lloyd-Max scalar codebooks for a rotated coordinate, N(0, 1/d).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

P1, section "Lloyd-Max 的两个最优性条件": a b-bit quantiser has 2^b levels
c_0 < ... < c_{2^b-1} and 2^b - 1 decision boundaries; it is optimal for a
density p when (1) every boundary is the midpoint of its two neighbouring
levels and (2) every level is the conditional mean of p over its cell, the
outer cells reaching to -inf and +inf.  The fixed point is found by
alternating the two conditions, starting from levels spread evenly over
[-3.5 sigma, 3.5 sigma] (same section).  The density is N(0, sigma^2) with
sigma^2 = 1/d (P1, section "旋转的关键定理" and "vLLM 的实现:数值积分而
不是解析解").

Two solvers:

* ``lloyd_max_exact``: the conditional mean of a Gaussian over (a, b) has the
  closed form  sigma * (phi(a/sigma) - phi(b/sigma)) / (Phi(b/sigma) - Phi(a/sigma))
  (phi, Phi: standard normal density and distribution).  Iterate in float64
  until no level moves by 1e-14 or more, then make the table exactly
  symmetric by mirroring the positive half (the page states the solution is
  symmetric about 0) and round to float32.  This is the default codebook.
* ``lloyd_max_page_trapz``: the numerical recipe of P1 ("vLLM 的实现:数值积分
  而不是解析解"), from the parameters the page gives: 200-trapezoid
  integrals, outer edges at +-10.5 sigma, tolerance 1e-10, at most 200
  iterations, returning the levels held when the loop stops.  The page does
  not say how its trapezoid rule is formed; the composite rule with 200
  equal panels is the reading taken.

A third codebook, ``lloyd_max_beta``: the exact marginal of one coordinate of
a uniformly random unit vector in R^d, the density of a rotated, normalised
key coordinate when the rotation is uniformly random (P3, kwkr.cn news
555717, section on the random orthogonal rotation: a scaled Beta law on
[-1, 1] that is nearly N(0, 1/d) in high dimension).  Its density is
  f(x) = C (1 - x^2)^a on [-1, 1],  a = (d - 3) / 2,
  C = Gamma(d/2) / (sqrt(pi) Gamma((d - 1)/2)).
The cell mass comes from the regularised incomplete Beta function,
P(|X| < x) = I_{x^2}(1/2, a + 1), and the first moment has the closed form
integral of x f(x) over (l, u) = C ((1 - l^2)^(a+1) - (1 - u^2)^(a+1)) / (2 (a + 1)).
The same fixed point as ``lloyd_max_exact``, with the outer cells ending at
-1 and +1.

Midpoints are formed from the sorted float32 levels in float32, as the page's
device set-up does (P1, section "vLLM 内置的 Lloyd-Max 码本"):
m_i = (c_i + c_{i+1}) / 2.
"""

import math

import numpy as np

EXACT_TOL = 1e-14
EXACT_MAX_ITER = 100000


def _std_pdf(z):
    if math.isinf(z):
        return 0.0
    return math.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)


def _std_mass(a, b):
    """P(a < Z < b) for a standard normal Z, taken from the tail that keeps
    full relative precision (complementary error function)."""
    if a >= 0.0:
        return 0.5 * (math.erfc(a / math.sqrt(2.0)) - math.erfc(b / math.sqrt(2.0)))
    if b <= 0.0:
        return 0.5 * (math.erfc(-b / math.sqrt(2.0)) - math.erfc(-a / math.sqrt(2.0)))
    return 1.0 - 0.5 * math.erfc(-a / math.sqrt(2.0)) - 0.5 * math.erfc(b / math.sqrt(2.0))


def gaussian_cell_mean(a, b, sigma):
    """E[X | a < X < b] for X ~ N(0, sigma^2); a may be -inf, b may be +inf."""
    za, zb = a / sigma, b / sigma
    return sigma * (_std_pdf(za) - _std_pdf(zb)) / _std_mass(za, zb)


def _initial_levels(n_levels, sigma):
    lo, hi = -3.5 * sigma, 3.5 * sigma
    return [lo + (hi - lo) * (i + 0.5) / n_levels for i in range(n_levels)]


def lloyd_max_exact(d, bits, tol=EXACT_TOL, max_iter=EXACT_MAX_ITER):
    """Fixed point of the two Lloyd-Max conditions for N(0, 1/d), float64.

    Returns (levels_f64 (symmetrised), iterations used).
    """
    n = 2 ** bits
    sigma = math.sqrt(1.0 / d)
    c = _initial_levels(n, sigma)
    for it in range(1, max_iter + 1):
        edges = [-math.inf] + [(c[i] + c[i + 1]) / 2.0 for i in range(n - 1)] + [math.inf]
        new = [gaussian_cell_mean(edges[i], edges[i + 1], sigma) for i in range(n)]
        delta = max(abs(new[i] - c[i]) for i in range(n))
        c = new
        if delta < tol:
            break
    else:
        raise RuntimeError("Lloyd-Max fixed point did not converge")
    pos = c[n // 2:]
    levels = [-v for v in reversed(pos)] + list(pos)
    return np.array(levels, dtype=np.float64), it


# The page's numerical recipe, from the parameters its text states: levels
# start evenly spread over +-3.5 sigma; the outer cells end at +-10.5 sigma
# (three times that spread) instead of +-inf; each cell's mass and first
# moment come from the composite trapezoid rule on 200 equal panels; the
# iteration stops as soon as an update would move no level by 1e-10 or more
# (keeping the levels it had), or after 200 updates.
PAGE_PANELS = 200
PAGE_OUTER_SIGMAS = 10.5
PAGE_TOL = 1e-10
PAGE_MAX_ITER = 200


def _gauss_density(x, var):
    return math.exp(-x * x / (2.0 * var)) / math.sqrt(2.0 * math.pi * var)


def trapezoid_cell_moments(a, b, var, panels=PAGE_PANELS):
    """(mass, first moment) of N(0, var) over [a, b] by the composite
    trapezoid rule on `panels` equal panels: nodes x_j = a + j h, weight h
    (h / 2 at the two ends); both sums taken in node order."""
    h = (b - a) / panels
    mass = 0.0
    first = 0.0
    for j in range(panels + 1):
        x = a + j * h
        fx = _gauss_density(x, var)
        if j == 0 or j == panels:
            fx = 0.5 * fx
        mass += fx
        first += x * fx
    return mass * h, first * h


def lloyd_max_page_trapz(d, bits, max_iter=PAGE_MAX_ITER, tol=PAGE_TOL):
    """The page's numerical recipe (see the comment above).  Returns
    (levels_f64, updates tried, converged flag).  Every cell has positive
    mass for these parameters, so each update is a plain ratio."""
    var = 1.0 / d
    outer = PAGE_OUTER_SIGMAS * math.sqrt(var)
    levels = _initial_levels(2 ** bits, math.sqrt(var))
    for it in range(1, max_iter + 1):
        bounds = [-outer] + [(u + w) / 2.0 for u, w in zip(levels, levels[1:])] + [outer]
        means = []
        for a, b in zip(bounds, bounds[1:]):
            mass, first = trapezoid_cell_moments(a, b, var)
            means.append(first / mass)
        if max(abs(m - c) for m, c in zip(means, levels)) < tol:
            return np.array(levels, dtype=np.float64), it, True
        levels = means
    return np.array(levels, dtype=np.float64), max_iter, False


def _beta_cdf(x, a):
    """P(X <= x) for the sphere marginal with exponent a (x in [-1, 1])."""
    from scipy.special import betainc
    if x <= -1.0:
        return 0.0
    if x >= 1.0:
        return 1.0
    half = 0.5 * betainc(0.5, a + 1.0, x * x)
    return 0.5 + half if x >= 0 else 0.5 - half


def _beta_mass(l, u, a):
    """P(l < X < u), from the tail nearer the cell for full relative precision."""
    from scipy.special import betainc
    if l >= 0.0:
        return 0.5 * (betainc(0.5, a + 1.0, u * u) - betainc(0.5, a + 1.0, l * l))
    if u <= 0.0:
        return 0.5 * (betainc(0.5, a + 1.0, l * l) - betainc(0.5, a + 1.0, u * u))
    return _beta_cdf(u, a) - _beta_cdf(l, a)


def beta_cell_mean(l, u, d):
    """E[X | l < X < u] for the sphere marginal in dimension d."""
    a = (d - 3) / 2.0
    logC = math.lgamma(d / 2.0) - 0.5 * math.log(math.pi) - math.lgamma((d - 1) / 2.0)
    m1 = math.exp(logC) * ((1.0 - l * l) ** (a + 1.0) - (1.0 - u * u) ** (a + 1.0)) / (2.0 * (a + 1.0))
    return m1 / _beta_mass(l, u, a)


def lloyd_max_beta(d, bits, tol=EXACT_TOL, max_iter=EXACT_MAX_ITER):
    """Fixed point of the Lloyd-Max conditions for the sphere marginal in
    dimension d (d >= 3), float64.  Returns (levels_f64 (symmetrised), iterations)."""
    n = 2 ** bits
    # the page's even spread over +-3.5 sigma, or over the support (-1, 1)
    # when that is narrower (small d)
    c = _initial_levels(n, min(math.sqrt(1.0 / d), 1.0 / 3.5))
    for it in range(1, max_iter + 1):
        edges = [-1.0] + [(c[i] + c[i + 1]) / 2.0 for i in range(n - 1)] + [1.0]
        new = [beta_cell_mean(edges[i], edges[i + 1], d) for i in range(n)]
        delta = max(abs(new[i] - c[i]) for i in range(n))
        c = new
        if delta < tol:
            break
    else:
        raise RuntimeError("Lloyd-Max fixed point did not converge")
    pos = c[n // 2:]
    levels = [-v for v in reversed(pos)] + list(pos)
    return np.array(levels, dtype=np.float64), it


def beta_mse_per_coord(levels, d):
    """Mean squared error per coordinate of a quantiser with the given sorted
    levels (midpoint boundaries) under the sphere marginal, by quadrature."""
    from scipy.integrate import quad
    a = (d - 3) / 2.0
    C = math.exp(math.lgamma(d / 2.0) - 0.5 * math.log(math.pi) - math.lgamma((d - 1) / 2.0))
    lv = list(levels)
    edges = [-1.0] + [(lv[i] + lv[i + 1]) / 2.0 for i in range(len(lv) - 1)] + [1.0]
    tot = 0.0
    for i, c in enumerate(lv):
        tot += quad(lambda x: (x - c) ** 2 * C * (1.0 - x * x) ** a, edges[i], edges[i + 1],
                    epsabs=1e-16, epsrel=1e-12, limit=200)[0]
    return tot


def midpoints_f32(levels_f32):
    """Decision boundaries from sorted float32 levels, in float32."""
    c = np.sort(np.asarray(levels_f32, dtype=np.float32))
    return ((c[:-1] + c[1:]) / np.float32(2.0)).astype(np.float32)


def codebook(d, bits, mode="exact"):
    """(centroids_f32, midpoints_f32) for a d-dimensional rotated coordinate."""
    if mode == "exact":
        levels, _ = lloyd_max_exact(d, bits)
    elif mode == "page_trapz":
        levels, _, _ = lloyd_max_page_trapz(d, bits)
    elif mode == "beta":
        levels, _ = lloyd_max_beta(d, bits)
    else:
        raise ValueError(mode)
    c32 = levels.astype(np.float32)
    return c32, midpoints_f32(c32)
