"""Pins of the oracle's Lloyd-Max codebook ("OrbitQuant" abstract: one
Lloyd-Max codebook for the fixed, known marginal of a rotated coordinate;
the marginal read as N(0, 1) in the normalized basis)."""
import math

import numpy as np
import pytest
from scipy import integrate
from scipy.stats import norm

from oracle import oracle as orc
from tests._golden import rows


def test_two_level_closed_form():
    lv, th = orc.lloyd_max_gaussian(2)
    assert abs(lv[1] - math.sqrt(2 / math.pi)) < 1e-13
    assert abs(lv[0] + math.sqrt(2 / math.pi)) < 1e-13 and th[0] == 0.0


@pytest.mark.parametrize("L", [2, 4, 8, 16])
def test_optimality_conditions_by_quadrature(L):
    # independent numerical integration (scipy quad on the normal density):
    # each level is the conditional mean of its cell (centroid condition),
    # each threshold the midpoint of its neighbours (nearest-neighbour condition)
    lv, th = orc.lloyd_max_gaussian(L)
    edges = [-np.inf, *th, np.inf]
    for i in range(L):
        a, b = edges[i], edges[i + 1]
        m1 = integrate.quad(lambda z: z * norm.pdf(z), a, b, epsabs=1e-14, epsrel=1e-13)[0]
        m0 = norm.cdf(b) - norm.cdf(a) if b <= 0 else norm.sf(a) - norm.sf(b)
        assert abs(m1 / m0 - lv[i]) < 1e-9, (L, i)
    assert np.allclose(th, (lv[:-1] + lv[1:]) / 2, atol=0, rtol=0)
    assert np.allclose(lv, -lv[::-1], atol=1e-14)


def test_two_level_mse():
    lv, _ = orc.lloyd_max_gaussian(2)
    mse = integrate.quad(lambda z: (abs(z) - lv[1]) ** 2 * norm.pdf(z), -np.inf, np.inf)[0]
    assert abs(mse - (1 - 2 / math.pi)) < 1e-10


def test_max_1960_table():
    for L, pos in rows("lloyd_max_gaussian.txt"):
        L = int(L)
        want = [float(v) for v in pos.split()]
        lv, _ = orc.lloyd_max_gaussian(L)
        got = lv[L // 2:]
        for w, g in zip(want, got):
            digits = len(str(w).replace(".", "").lstrip("0"))
            assert abs(g - w) <= 0.6 * 10 ** (math.floor(math.log10(abs(w))) - digits + 1), (L, w, g)


def test_bf16_codebook_is_rounded_book():
    # each decode level is one of the two bf16 neighbours of the fp64 level,
    # the nearer one; the book stays symmetric and ascending
    for L in (4, 16):
        lv, _ = orc.lloyd_max_gaussian(L)
        bk = orc.codebook_bf16(L).astype(np.float64)
        assert np.all(np.diff(bk) > 0) and np.array_equal(bk, -bk[::-1])
        for x, c in zip(lv, bk):
            m, e = math.frexp(x)
            ulp = 2.0 ** (e - 8)
            assert abs(c - x) <= ulp / 2
            assert (c / ulp) == round(c / ulp)
    assert orc.round_to_bf16(1.0 + 2 ** -8) == 1.0          # tie to even
    assert orc.round_to_bf16(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6
