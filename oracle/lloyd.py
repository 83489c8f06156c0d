"""Lloyd-Max table fitting -- TEST INFRASTRUCTURE (oracle).

The page "mlx-bun 0.0.9 -> 0.0.11", src/mlx/turboquant-tables.ts (header
of ``LLOYD_MAX``) says the value tables are an iterative Lloyd-Max fit to
unit-normal samples, 500 iterations. Two plain numpy (binary64) versions:

* ``fit_samples`` -- Lloyd's iteration on a sample set, step by step:
  boundaries are midpoints of adjacent centroids, each sample goes to the
  number of boundaries strictly below it (the codec's bin rule), each
  centroid becomes the mean of its samples (an empty level keeps its
  value). Sums are taken over the exact integers rint(x * 2^s) (s from the
  sample count and largest magnitude, so they cannot overflow int64), which
  makes the result independent of summation order.
* ``fit_gaussian`` -- the same iteration on the N(0,1) density itself:
  the mean of N(0,1) on [a, b] is (phi(a) - phi(b)) / (Phi(b) - Phi(a)).
  Its fixed point is the textbook Lloyd-Max quantiser of a Gaussian.

Only ``tests/`` and ``bench.py``'s CPU baseline use this module.
"""
from __future__ import annotations

import math

import numpy as np


def fixed_point_shift(samples: np.ndarray) -> int:
    """s = min(40, 62 - bitlen(n) - e), |x| < 2^e for every sample; -1 when
    a sample is not finite or the magnitudes are too large."""
    x = np.asarray(samples, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        return -1
    a = float(np.max(np.abs(x))) if x.size else 0.0
    e = math.frexp(a)[1] if a != 0.0 else 0
    s = 62 - int(x.size).bit_length() - e
    return min(40, s) if s >= 0 else -1


def fit_samples(samples, init, iterations: int):
    """Lloyd iterations on float32 samples from the ascending centroids
    `init`; returns (centroids, boundaries) in binary64."""
    x = np.ascontiguousarray(samples, dtype=np.float32).ravel()
    c = np.array(init, dtype=np.float64)
    L = c.size
    s = fixed_point_shift(x)
    if s < 0:
        raise ValueError("samples not finite or too large for exact integer sums")
    q = np.rint(np.ldexp(x.astype(np.float64), s)).astype(np.int64)
    xd = x.astype(np.float64)
    for _ in range(iterations):
        b = (c[:-1] + c[1:]) * 0.5
        k = np.searchsorted(b, xd, side="left")  # number of boundaries strictly below x
        sums = np.zeros(L, np.int64)
        np.add.at(sums, k, q)
        cnt = np.bincount(k, minlength=L)
        nz = cnt > 0
        c = c.copy()
        c[nz] = np.ldexp(sums[nz].astype(np.float64), -s) / cnt[nz].astype(np.float64)
    return c, (c[:-1] + c[1:]) * 0.5


def _phi(t):
    return math.exp(-0.5 * t * t) / math.sqrt(2.0 * math.pi) if math.isfinite(t) else 0.0


def _Phi(t):
    if t == math.inf:
        return 1.0
    if t == -math.inf:
        return 0.0
    return 0.5 * math.erfc(-t / math.sqrt(2.0))


def fit_gaussian(init, iterations: int):
    """Lloyd iterations on the N(0,1) density (cells extend to -inf and
    +inf at the ends); returns (centroids, boundaries)."""
    c = [float(v) for v in init]
    L = len(c)
    for _ in range(iterations):
        b = [(c[j] + c[j + 1]) * 0.5 for j in range(L - 1)]
        edges = [-math.inf] + b + [math.inf]
        new = []
        for k in range(L):
            lo, hi = edges[k], edges[k + 1]
            mass = _Phi(hi) - _Phi(lo)
            new.append((_phi(lo) - _phi(hi)) / mass if mass > 0 else c[k])
        c = new
    c = np.array(c, dtype=np.float64)
    return c, (c[:-1] + c[1:]) * 0.5
