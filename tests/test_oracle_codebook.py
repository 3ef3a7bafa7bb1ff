"""Pins for the oracle's Lloyd-Max codebook for N(0, 1/d).

* 1-bit closed form: the optimal two-level quantiser of N(0, s^2) has levels
  +-s*sqrt(2/pi) (the conditional mean of a half-normal).
* Max (1960) classic table, scaled by 1/sqrt(d) (tests/golden).
* The pages' printed d = 128 levels (P1, section "vLLM 内置的 Lloyd-Max 码本").
* Both optimality conditions of P1, section "Lloyd-Max 的两个最优性条件",
  checked by numerical quadrature (scipy), independent of the closed form.
* Distortion below the page's high-rate approximation (P1, section "3-bit
  和 4-bit 的码本长什么样": NMSE about (sqrt(3) pi / 2) 2^-2b).
"""

import math

import numpy as np
import pytest
from scipy import integrate

from oracle import codebook as cb
from conftest import load_golden


@pytest.mark.parametrize("d", [64, 128, 256])
def test_one_bit_closed_form(d):
    lv, _ = cb.lloyd_max_exact(d, 1)
    want = math.sqrt(2.0 / math.pi) / math.sqrt(d)
    assert abs(lv[1] - want) < 1e-15 and lv[0] == -lv[1]


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_matches_max_1960_table(bits):
    tab = load_golden("lloyd_max_unit_gaussian.json")["positive_levels"][str(bits)]
    lv, _ = cb.lloyd_max_exact(128, bits)
    pos = lv[len(lv) // 2:] * math.sqrt(128)
    for got, txt in zip(pos, tab):
        unit = 10.0 ** -len(txt.split(".")[1])      # one unit of the last printed digit
        assert abs(got - float(txt)) <= unit * 1.0001


@pytest.mark.parametrize("bits", [3, 4])
def test_matches_page_printed_levels(bits):
    g = load_golden("codebook_d128_page.json")
    c32, _ = cb.codebook(128, bits)
    pos = c32[len(c32) // 2:].astype(np.float64)
    # printed to 4 decimals with sigma rounded to 0.0884: allow 1.5e-4
    assert np.max(np.abs(pos - np.array(g["positive_levels"][str(bits)]))) < 1.5e-4
    assert abs(pos[-1] - g["outermost_approx"][str(bits)]) < 1.5e-3


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d", [64, 128])
def test_optimality_conditions_by_quadrature(d, bits):
    lv, _ = cb.lloyd_max_exact(d, bits)
    sigma = 1.0 / math.sqrt(d)
    pdf = lambda x: math.exp(-x * x / (2 * sigma * sigma)) / (sigma * math.sqrt(2 * math.pi))
    edges = [-np.inf] + [(lv[i] + lv[i + 1]) / 2 for i in range(len(lv) - 1)] + [np.inf]
    for i in range(len(lv)):
        a, b = edges[i], edges[i + 1]
        num = integrate.quad(lambda x: x * pdf(x), a, b, epsabs=1e-15, epsrel=1e-13, limit=200)[0]
        den = integrate.quad(pdf, a, b, epsabs=1e-15, epsrel=1e-13, limit=200)[0]
        assert abs(num / den - lv[i]) < 1e-12


@pytest.mark.parametrize("bits", [3, 4])
def test_symmetry_and_midpoints_float32(bits):
    c, m = cb.codebook(128, bits)
    n = len(c)
    assert np.array_equal(c.view(np.uint32), (-c[::-1]).view(np.uint32))
    assert np.all(np.diff(c) > 0)
    assert len(m) == n - 1
    centre = m[n // 2 - 1]
    assert centre == 0.0 and not np.signbit(centre)
    assert np.array_equal(m, ((c[:-1] + c[1:]) / np.float32(2)).astype(np.float32))
    assert np.all((m > c[:-1]) & (m < c[1:]))


@pytest.mark.parametrize("bits,mse_d", [(3, 0.0345), (4, 0.00950)])
def test_distortion_below_high_rate_bound(bits, mse_d):
    d = 128
    c, m = cb.codebook(d, bits)
    rng = np.random.default_rng(bits)
    x = rng.standard_normal(2_000_000) / math.sqrt(d)
    idx = np.searchsorted(m.astype(np.float64), x, side="right")
    err = ((x - c.astype(np.float64)[idx]) ** 2).mean() * d
    high_rate = math.sqrt(3) * math.pi / 2 * 2.0 ** (-2 * bits)
    assert err < high_rate
    assert abs(err - mse_d) / mse_d < 0.02


def test_page_recipe_reading():
    """The page's trapezoid recipe converges for 3 bits but not within its
    200-iteration cap for 4 bits; either way it lands next to the fixed point."""
    l3, it3, conv3 = cb.lloyd_max_page_trapz(128, 3)
    l4, it4, conv4 = cb.lloyd_max_page_trapz(128, 4)
    assert conv3 and it3 < 200
    assert (not conv4) and it4 == 200
    for bits, lt in ((3, l3), (4, l4)):
        le, _ = cb.lloyd_max_exact(128, bits)
        assert np.max(np.abs(lt - le) / np.abs(le)) < 1e-3


# ---------------------------------------------------------------------------
# exact sphere-marginal (Beta) codebook
# ---------------------------------------------------------------------------


def test_beta_codebook_matches_printed_d128_b3():
    g = load_golden("codebook_beta_d128_b3_page.json")
    lv, _ = cb.lloyd_max_beta(g["head_dim"], g["bits"])
    assert np.max(np.abs(lv - np.array(g["centroids"]))) <= 0.5 * 10.0 ** -g["printed_decimals"] + 1e-12
    mse = cb.beta_mse_per_coord(lv, g["head_dim"])
    assert abs(mse - g["mse_per_coord"]) <= 0.005e-4
    assert abs(mse * g["head_dim"] - g["mse_total"]) <= 0.005e-2


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_beta_codebook_d3_is_the_uniform_quantiser(bits):
    # d = 3: the marginal of a uniform point on the sphere S^2 is uniform on
    # [-1, 1] (Archimedes), whose Lloyd-Max quantiser is the uniform one
    lv, _ = cb.lloyd_max_beta(3, bits)
    n = 2 ** bits
    want = -1.0 + (2 * np.arange(n) + 1) / n
    assert np.max(np.abs(lv - want)) < 1e-12


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bits", [3, 4])
def test_beta_codebook_fixed_point(d, bits):
    lv, _ = cb.lloyd_max_beta(d, bits)
    assert np.array_equal(lv, -lv[::-1])
    edges = [-1.0] + list((lv[:-1] + lv[1:]) / 2) + [1.0]
    # each level is its cell's mean, by an independent quadrature of the density
    from scipy.integrate import quad
    a = (d - 3) / 2.0
    for i, c in enumerate(lv):
        m0 = quad(lambda x: (1 - x * x) ** a, edges[i], edges[i + 1], epsabs=0, epsrel=1e-13, limit=200)[0]
        m1 = quad(lambda x: x * (1 - x * x) ** a, edges[i], edges[i + 1], epsabs=0, epsrel=1e-13, limit=200)[0]
        assert abs(m1 / m0 - c) < 1e-11 * max(1.0, abs(c)) + 1e-13


def test_beta_codebook_tends_to_gaussian():
    # the marginal tends to N(0, 1/d); the levels' relative gap shrinks like 1/d
    gaps = []
    for d in (128, 1024, 8192):
        g, _ = cb.lloyd_max_exact(d, 3)
        b, _ = cb.lloyd_max_beta(d, 3)
        gaps.append(np.max(np.abs(g - b) / np.abs(g)))
    assert gaps[0] > gaps[1] > gaps[2]
    assert gaps[2] < 2e-4
    assert 4 < gaps[0] / gaps[1] < 16


def test_beta_codebook_lower_mse_than_gaussian_on_sphere():
    # the codebook made for the true marginal distorts less under it
    for bits in (3, 4):
        g, _ = cb.lloyd_max_exact(128, bits)
        b, _ = cb.lloyd_max_beta(128, bits)
        assert cb.beta_mse_per_coord(b, 128) < cb.beta_mse_per_coord(g, 128)


def test_page_recipe_levels_near_the_printed_table():
    """The page's recipe lands within its own quadrature bias (200 panels over
    cells reaching +-10.5 sigma) of the levels the page prints: 3e-4."""
    g = load_golden("codebook_d128_page.json")
    for bits in (3, 4):
        lt, _, _ = cb.lloyd_max_page_trapz(g["head_dim"], bits)
        pos = lt[len(lt) // 2:]
        assert np.max(np.abs(pos - np.array(g["positive_levels"][str(bits)]))) < 3e-4


@pytest.mark.parametrize("a,b", [(-10.5, -2.0), (-0.3, 0.7), (1.1, 10.5)])
def test_trapezoid_cell_moments_within_the_rule_error_bound(a, b):
    """The composite trapezoid rule against the closed forms of a Gaussian
    cell's mass and first moment, within the rule's bound (b - a) h^2 / 12
    max|f''| (f'' of the density and of x times the density are below
    0.5 and 0.8 over R for unit variance)."""
    var = 1.0
    mass, first = cb.trapezoid_cell_moments(a, b, var)
    want_mass = 0.5 * (math.erf(b / math.sqrt(2)) - math.erf(a / math.sqrt(2)))
    want_first = (math.exp(-a * a / 2) - math.exp(-b * b / 2)) / math.sqrt(2 * math.pi)
    h = (b - a) / cb.PAGE_PANELS
    assert abs(mass - want_mass) <= (b - a) * h * h / 12 * 0.5
    assert abs(first - want_first) <= (b - a) * h * h / 12 * 0.8
