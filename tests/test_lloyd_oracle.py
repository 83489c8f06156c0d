"""Pins of the Lloyd-Max fitting oracle (oracle/lloyd.py).

fit_gaussian is pinned to the textbook optimum quantisers of a unit
Gaussian (Max 1960, tests/golden/max1960_gaussian.txt) and to the page's
3-bit table (the "hardcoded fast-path table" of turboquant-tables.ts);
fit_samples is pinned by hand-computed small cases (including the tie rule
and empty levels), exact invariances (sample order, scaling by 2) and by
converging, on a large seeded N(0,1) sample, to fit_gaussian -- two
independent evaluations of the same iteration."""
import math
import os

import numpy as np
import pytest

import oracle as O
from oracle import lloyd as L

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "max1960_gaussian.txt")


def max_tables():
    out = {}
    for ln in open(GOLDEN):
        if ln.startswith("#") or not ln.strip():
            continue
        n, rest = ln.split(":")
        outs, thr = rest.split("|")
        pos = [float(v) for v in outs.split()]
        t = [float(v) for v in thr.split()]
        c = np.array([-v for v in pos[::-1]] + pos)
        b = np.array([-v for v in t[::-1]] + ([0.0] if int(n) % 2 == 0 else []) + t)
        out[int(n)] = (c, b)
    return out


@pytest.mark.parametrize("levels", [2, 4, 8, 16])
def test_gaussian_fit_matches_max_1960(levels):
    c, b = L.fit_gaussian(np.linspace(-2.0, 2.0, levels), 2000)
    mc, mb = max_tables()[levels]
    np.testing.assert_allclose(c, mc, atol=1.5e-3, rtol=5e-4)
    np.testing.assert_allclose(b, mb, atol=1.5e-3, rtol=5e-4)
    if levels == 2:
        assert abs(c[1] - math.sqrt(2.0 / math.pi)) < 1e-12


def test_gaussian_fit_matches_page_3bit_table():
    c, b = L.fit_gaussian(np.linspace(-2.0, 2.0, 8), 2000)
    pc, pb = O.lloyd_max(3)
    np.testing.assert_allclose(c, pc, atol=1e-5)
    np.testing.assert_allclose(b, pb, atol=1e-5)


def test_samples_small_cases_by_hand():
    # two clusters: one iteration lands on the cluster means and stays
    c, b = L.fit_samples(np.array([-3, -1, 1, 3], np.float32), [-0.5, 0.5], 5)
    np.testing.assert_array_equal(c, [-2.0, 2.0])
    np.testing.assert_array_equal(b, [0.0])
    # a sample exactly on a boundary goes to the lower level
    c, _ = L.fit_samples(np.array([-1, 0, 1], np.float32), [-1.0, 1.0], 1)
    np.testing.assert_array_equal(c, [-0.5, 1.0])
    # a level with no samples keeps its centroid
    c, _ = L.fit_samples(np.array([1, 2, 3, 4], np.float32), [-5.0, 1.0, 4.0], 1)
    assert c[0] == -5.0
    np.testing.assert_array_equal(c[1:], [1.5, 3.5])   # boundaries -2, 2.5: {1, 2} and {3, 4}
    # zero iterations return the start
    c, b = L.fit_samples(np.array([0.5], np.float32), [-1.0, 1.0], 0)
    np.testing.assert_array_equal(c, [-1.0, 1.0])
    np.testing.assert_array_equal(b, [0.0])


def test_samples_exact_invariances():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(20000).astype(np.float32)
    init = np.linspace(-2, 2, 8)
    c1, b1 = L.fit_samples(x, init, 30)
    c2, b2 = L.fit_samples(rng.permutation(x), init, 30)     # order independent, exactly
    np.testing.assert_array_equal(c1, c2)
    c3, b3 = L.fit_samples(2 * x, 2 * init, 30)              # scaling by 2 commutes, exactly
    np.testing.assert_array_equal(c3, 2 * c1)
    np.testing.assert_array_equal(b3, 2 * b1)


def test_fixed_point_shift_rule():
    assert L.fixed_point_shift(np.zeros(1, np.float32)) == 40
    # |x| < 2^3 and 2^20 samples: s = 62 - 21 - 3
    x = np.zeros(1 << 20, np.float32)
    x[0] = 7.5
    assert L.fixed_point_shift(x) == 38
    assert L.fixed_point_shift(np.array([np.inf], np.float32)) == -1
    assert L.fixed_point_shift(np.array([np.nan], np.float32)) == -1
    assert L.fixed_point_shift(np.array([2.0 ** 70], np.float32)) == -1


@pytest.mark.parametrize("levels", [4, 8])
def test_samples_converge_to_density_fit(levels):
    x = np.random.default_rng(11).standard_normal(1 << 18).astype(np.float32)
    init = np.linspace(-2.0, 2.0, levels)
    c, b = L.fit_samples(x, init, 300)
    g, gb = L.fit_gaussian(init, 2000)
    # sampling error of the level means over ~2^18 / levels samples; the
    # outer levels (a few percent of the mass, long tails) move the most
    np.testing.assert_allclose(c[1:-1], g[1:-1], atol=2e-2)
    np.testing.assert_allclose(c, g, atol=3e-2)
    np.testing.assert_allclose(b, gb, atol=2e-2)
