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


# ---------------------------------------------------------------------------
# Independent pins of the fixed-point sums. The fit's definition is the plain
# Lloyd iteration of the tables page (header of LLOYD_MAX: an iterative
# Lloyd-Max fit, 500 iterations): each centroid becomes the mean of the samples
# in its cell. fit_samples takes those means over the integers rint(x * 2^s),
# so each centroid may differ from the exact cell mean by at most half a unit
# 2^-(s+1) (every sample moves by at most that much, and so does their mean),
# plus the two binary64 roundings of converting and dividing the sum. The tests
# below hold fit_samples to that bound against exact rational means and against
# a plain binary64 Lloyd iteration written without fixed point, and check that
# the integer sums cannot overflow int64 at the largest sample count and
# magnitude the shift admits.
# ---------------------------------------------------------------------------

import importlib.util  # noqa: E402
from fractions import Fraction  # noqa: E402


def plain_lloyd(samples, init, iterations):
    """Lloyd's iteration in plain binary64: midpoint boundaries, a sample goes
    to the number of boundaries strictly below it, each centroid becomes the
    correctly rounded sum of its cell (math.fsum) divided by the count; a cell
    with no sample keeps its centroid. Returns the centroids and, per
    iteration, the cell sizes (for checking that two runs saw the same cells)."""
    xs = np.sort(np.asarray(samples, np.float32).astype(np.float64))
    c = np.array(init, np.float64)
    sizes = []
    for _ in range(iterations):
        b = (c[:-1] + c[1:]) * 0.5
        # cell k holds the samples in (b[k-1], b[k]]: those at or below b[k] and above b[k-1]
        edges = np.concatenate([[0], np.searchsorted(xs, b, side="right"), [xs.size]])
        new = c.copy()
        for k in range(c.size):
            seg = xs[edges[k]:edges[k + 1]]
            if seg.size:
                new[k] = math.fsum(seg) / seg.size
        sizes.append(np.diff(edges))
        c = new
    return c, sizes


def cell_sizes(samples, c):
    b = (np.asarray(c)[:-1] + np.asarray(c)[1:]) * 0.5
    k = np.searchsorted(b, np.asarray(samples, np.float32).astype(np.float64), side="left")
    return np.bincount(k, minlength=len(c))


def half_unit_bound(s, c):
    """|fit - exact cell mean| <= 2^-(s+1) from the rounded integers, plus a
    few binary64 ulps of the centroid for the conversion and the division."""
    return 2.0 ** -(s + 1) + 4.0 * np.spacing(np.abs(np.asarray(c, np.float64)))


def sample_sets():
    rng = np.random.default_rng(2024)
    yield "normal", rng.standard_normal(1 << 15).astype(np.float32)
    yield "student_t3", rng.standard_t(3, 1 << 14).astype(np.float32)
    yield "uniform", rng.uniform(-3.0, 3.0, 1 << 14).astype(np.float32)
    # values with bits below 2^-s: small magnitudes next to one large one
    small = (rng.standard_normal(1 << 14) * 1e-6).astype(np.float32)
    small[0] = np.float32(900.0)
    yield "mixed_scale", small


def lockstep_compare(fit, x, init, iterations):
    """Run fit_samples and the plain iteration side by side; require the same
    cells at every step and centroids within the half-unit bound."""
    s = L.fixed_point_shift(x)
    assert s >= 0
    c_fit = np.array(init, np.float64)
    c_plain = np.array(init, np.float64)
    for it in range(iterations):
        assert np.array_equal(cell_sizes(x, c_fit), cell_sizes(x, c_plain)), f"cells differ at iteration {it}"
        c_fit, _ = fit(x, c_fit, 1)
        c_plain, _ = plain_lloyd(x, c_plain, 1)
        err = np.abs(c_fit - c_plain)
        assert np.all(err <= half_unit_bound(s, c_plain)), (it, float(err.max()), s)
    return c_fit, c_plain


@pytest.mark.parametrize("levels", [4, 16])
def test_fit_samples_equals_plain_lloyd_within_half_unit(levels):
    """500 iterations (the page's count) on four sample sets: the fixed-point
    fit follows the plain binary64 Lloyd iteration cell for cell, each
    centroid within 2^-(s+1) plus rounding of the exact cell mean."""
    for name, x in sample_sets():
        init = np.linspace(-2.0, 2.0, levels) * (1e-6 if name == "mixed_scale" else 1.0)
        c_fit, c_plain = lockstep_compare(L.fit_samples, x, init, 500)
        # and the 500-iteration fit in one call equals the stepped one exactly
        c_once, _ = L.fit_samples(x, init, 500)
        np.testing.assert_array_equal(c_once, c_fit, err_msg=name)


def adversarial_quarter_units(n=4096, seed=5):
    """Samples whose scaled values x * 2^s all sit three quarters of a unit
    above an integer, next to one large sample that fixes the shift: rounding
    to nearest moves each by +1/4 unit, a floor would move each by -3/4."""
    rng = np.random.default_rng(seed)
    base = np.zeros(n, np.float32)
    base[0] = np.float32(6.5)
    s = L.fixed_point_shift(base)
    m = rng.integers(1, 1 << 12, n)
    x = ((4 * m + 3).astype(np.float64) * 2.0 ** -(s + 2)).astype(np.float32)
    x[0] = np.float32(6.5)
    assert L.fixed_point_shift(x) == s
    assert np.all(x[1:].astype(np.float64) * 2.0 ** (s + 2) == (4 * m[1:] + 3))
    return x, s


def check_means_against_fractions(fit):
    x, s = adversarial_quarter_units()
    init = np.array([0.0, 1e-3, 5.0])  # cells: (-inf, 5e-4], (5e-4, 2.5005], (2.5005, inf)
    c, _ = fit(x, init, 1)
    b = (init[:-1] + init[1:]) / 2
    k = np.searchsorted(b, x.astype(np.float64), side="left")
    for lev in range(3):
        cell = [Fraction(float(v)) for v in x[k == lev]]
        if not cell:
            continue
        exact = sum(cell, Fraction(0)) / len(cell)
        assert abs(Fraction(float(c[lev])) - exact) <= Fraction(1, 2 ** (s + 1)) + Fraction(4 * float(np.spacing(c[lev]))), lev


def test_fixed_point_means_within_half_unit_of_exact_rationals():
    check_means_against_fractions(L.fit_samples)


def check_worst_case_sums_fit_int64(shift):
    """For sample counts up to 2^26 and magnitudes just below each power of
    two, every sample at the largest magnitude: the sum of rint(x * 2^s) as a
    Python integer stays below 2^63, and so does int64 accumulation."""
    for n in (1, 3, 1 << 10, (1 << 16) + 1, 1 << 20, (1 << 26) - 1):
        for e in (-20, -1, 0, 1, 3, 10, 20):
            big = np.float32(np.nextafter(np.float32(2.0 ** e), np.float32(0)))
            x = np.broadcast_to(big, (n,))
            s = shift(x)
            if s < 0:
                continue
            unit = int(np.rint(np.ldexp(np.float64(big), s)))
            assert n * unit < 2 ** 63, (n, e, s)
            # the same accumulation in int64 equals the exact integer sum
            part = np.full(min(n, 1 << 12), unit, np.int64)
            assert int(part.sum(dtype=np.int64)) == part.size * unit


def test_fixed_point_shift_keeps_worst_case_sums_exact():
    check_worst_case_sums_fit_int64(L.fixed_point_shift)
    # magnitudes whose worst-case sum cannot be held at any shift are refused
    assert L.fixed_point_shift(np.array([2.0 ** 70], np.float32)) == -1


def test_fixed_point_shift_resolves_unit_normal_data():
    """The shift resolves the bench-sized fit (2^24 unit-normal samples) to
    well below binary32 precision: means within 1e-10 of exact."""
    x = np.broadcast_to(np.float32(5.9), (1 << 24,))
    s = L.fixed_point_shift(x)
    assert s >= 0 and 2.0 ** -(s + 1) < 1e-10


def mutated_lloyd(old, new):
    """A copy of oracle/lloyd.py with one planted mistake (CPU only)."""
    src = open(L.__file__).read()
    assert old in src
    spec = importlib.util.spec_from_loader("lloyd_mutant", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(src.replace(old, new), "lloyd_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("old,new,check", [
    ("np.rint(np.ldexp", "np.floor(np.ldexp", "means"),
    ("np.rint(np.ldexp", "np.trunc(np.ldexp", "means"),
    ("s = 62 -", "s = 65 -", "overflow"),
    ("int(x.size).bit_length() - e", "int(x.size).bit_length() // 2 - e", "overflow"),
])
def test_pins_catch_planted_mistakes(old, new, check):
    mut = mutated_lloyd(old, new)
    with pytest.raises(AssertionError):
        if check == "means":
            check_means_against_fractions(mut.fit_samples)
        else:
            check_worst_case_sums_fit_int64(mut.fixed_point_shift)
