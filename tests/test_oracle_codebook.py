"""Pins for the oracle's Lloyd-Max codebooks (CPU only).

The codebook is the Lloyd-Max quantizer of the rotated-coordinate law
(blog.hotdry.top, random rotation + scalar quantisation section; a2a-mcp.org,
stage 1).  Pinned by: the d = 3 case (uniform law, uniform quantizer), the
1-bit closed form, the Gaussian limit (Max 1960), the optimality conditions
checked by independent quadrature, and the numbers the pages print.
"""
import math

import numpy as np
import pytest
from scipy import integrate, special

from oracle import tq_oracle as o


@pytest.mark.parametrize("bp", [1, 2, 3, 4])
def test_d3_is_uniform_quantizer(bp):
    # A coordinate of a uniform point on S^2 is Uniform[-1, 1] (Archimedes).
    K = 2 ** bp
    c, t = o.lloyd_max(3, K)
    want = -1 + (2 * np.arange(K) + 1) / K
    assert np.max(np.abs(c - want)) < 1e-10
    # per-vector error d * (1/3) (1/K)^2 * ... = 4^-bp for the uniform grid on [-1,1]
    assert abs(o.codebook_distortion(3, c, t) - 4.0 ** -bp) < 1e-10


@pytest.mark.parametrize("d", [3, 16, 128, 200, 1000])
def test_one_bit_closed_form(d):
    c, t = o.lloyd_max(d, 2)
    exact = math.exp(math.lgamma(d / 2) - math.lgamma((d + 1) / 2)) / math.sqrt(math.pi)
    assert abs(c[1] - exact) < 1e-12 and abs(c[0] + exact) < 1e-12
    assert t[0] == 0.0
    assert abs(o.codebook_distortion(d, c, t) - (1 - d * exact ** 2)) < 1e-11


@pytest.mark.parametrize("d", [128, 200])
def test_one_bit_page_value(d, golden):
    # page prints +-sqrt(2/(pi d)), the Gaussian limit; the exact Beta-law
    # centroid differs by O(1/d) relative.
    c, _ = o.lloyd_max(d, 2)
    page = math.sqrt(2 / (math.pi * d))
    assert abs(c[1] - page) / page < 1 / (2 * d)


@pytest.mark.parametrize("d,bp", [(5, 2), (16, 3), (128, 2), (128, 4), (200, 3)])
def test_optimality_conditions_by_quadrature(d, bp):
    # Independent of the closed-form moment and of betainc: plain adaptive
    # quadrature of the unnormalised density (1-x^2)^((d-3)/2).
    K = 2 ** bp
    c, t = o.lloyd_max(d, K)
    assert np.allclose(t, 0.5 * (c[1:] + c[:-1]), atol=1e-15)
    w = lambda x: (1 - x * x) ** ((d - 3) / 2)
    edges = np.concatenate(([-1.0], t, [1.0]))
    for k in range(K):
        m0, _ = integrate.quad(w, edges[k], edges[k + 1], epsabs=0, epsrel=1e-13, limit=200)
        m1, _ = integrate.quad(lambda x: x * w(x), edges[k], edges[k + 1], epsabs=0, epsrel=1e-13, limit=200)
        assert abs(m1 / m0 - c[k]) < 1e-10 / math.sqrt(d)


def test_symmetric_and_sorted():
    for d in (7, 128):
        for bp in (1, 2, 3, 4):
            c, t = o.lloyd_max(d, 2 ** bp)
            assert np.all(np.diff(c) > 0)
            assert np.array_equal(c, -c[::-1])


@pytest.mark.parametrize("bp", [1, 2, 3, 4])
def test_gaussian_limit_matches_max_table(bp, golden):
    # d * (per-coordinate error) -> Max's Gaussian value as d -> oo; the gap
    # is O(1/d), so extrapolate linearly in 1/d from d = 512 and 1024.
    want = golden["books"]["gaussian_lloyd_max_mse"]["values"][str(bp)]
    D = {}
    for d in (512, 1024):
        c, t = o.lloyd_max(d, 2 ** bp, tol=1e-11)
        D[d] = o.codebook_distortion(d, c, t)
    extrap = 2 * D[1024] - D[512]
    # the table is printed to 4 significant figures
    assert abs(extrap - want) / want < 5e-4
    assert abs(D[1024] - want) < abs(D[512] - want)


@pytest.mark.parametrize("bp", [1, 2, 3, 4])
def test_page_distortion_values(bp, golden):
    # The page prints 0.36 / 0.117 / 0.03 / 0.009; those are rounded (the last
    # two to one significant figure).  Accept half a unit of the last printed
    # digit plus 2% of the printed value.
    printed = golden["pages"]["mse_per_unit_vector"]["values"][str(bp)]
    s = repr(printed)
    ulp = 10.0 ** -(len(s.split(".")[1]))
    c, t = o.lloyd_max(128, 2 ** bp)
    D = o.codebook_distortion(128, c, t)
    assert abs(D - printed) <= 0.5 * ulp + 0.02 * printed


def test_four_times_per_bit_and_bound(golden):
    # each bit cuts the error by about 4x; the error stays between the
    # Shannon-type bound 4^-b' and sqrt(3) pi / 2 times it.
    ratio = golden["pages"]["distortion_ratio_to_lower_bound"]["value"]
    Ds = []
    for bp in (1, 2, 3, 4):
        c, t = o.lloyd_max(128, 2 ** bp)
        D = o.codebook_distortion(128, c, t)
        Ds.append(D)
        assert 4.0 ** -bp <= D <= math.sqrt(3) * math.pi / 2 * 4.0 ** -bp
        assert D / 4.0 ** -bp < ratio + 0.05
    for a, b in zip(Ds, Ds[1:]):
        assert 3.0 < a / b < 4.0


def test_cosine_at_three_bits(golden):
    # by the centroid condition E<u, u_hat> = E||u_hat||^2 = 1 - D, so the
    # cosine is sqrt(1 - D)
    c, t = o.lloyd_max(128, 8)
    D = o.codebook_distortion(128, c, t)
    assert math.sqrt(1 - D) >= golden["pages"]["cosine_3bit"]["value"] - 5e-4


def test_one_bit_gaussian_limit_closed_form():
    # d * E|X|^2-type limit: 1 - 2/pi for the 1-bit Gaussian quantizer
    D = {}
    for d in (512, 1024):
        c, t = o.lloyd_max(d, 2)
        D[d] = o.codebook_distortion(d, c, t)
    assert abs((2 * D[1024] - D[512]) - (1 - 2 / math.pi)) < 1e-6


def test_distortion_formula_by_quadrature():
    d, K = 64, 8
    c, t = o.lloyd_max(d, K)
    edges = np.concatenate(([-1.0], t, [1.0]))
    tot = 0.0
    for k in range(K):
        v, _ = integrate.quad(lambda x: (x - c[k]) ** 2 * o.beta_density(x, d),
                              edges[k], edges[k + 1], epsabs=0, epsrel=1e-12, limit=200)
        tot += v
    assert abs(d * tot - o.codebook_distortion(d, c, t)) < 1e-10
