"""Writes lloyd_fit_2p24.txt: the fitting oracle's centroids and boundaries
after the tables page's 500 Lloyd iterations ("mlx-bun 0.0.9 -> 0.0.11",
turboquant-tables.ts, header of LLOYD_MAX: an iterative Lloyd-Max fit to
unit-normal samples, 500 iterations) on the fit workload's 2^24 seeded
unit-normal samples, started from the printed 4-bit table.

    python tests/golden/make_lloyd_fit.py

Calls only oracle/ (and the seeded sample generator, which holds no
arithmetic of the method). Takes several minutes on one core.
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle as O  # noqa: E402
from oracle import lloyd as OL  # noqa: E402
from kv_cache_quantization_tq_amd import workloads as W  # noqa: E402

OUT = os.path.join(HERE, "lloyd_fit_2p24.txt")


def main():
    cfg = W.LLOYD
    x = W.lloyd_samples()
    init = O.lloyd_max(4)[0].astype(np.float64)
    c, b = OL.fit_samples(x, init, cfg["iterations"])
    with open(OUT, "w") as f:
        f.write("# Fitting oracle (oracle/lloyd.py fit_samples) after 500 Lloyd iterations on the fit\n")
        f.write("# workload's samples: numpy default_rng(6).standard_normal(2**24, float32), 16 levels\n")
        f.write("# started from the printed 4-bit LLOYD_MAX table (\"mlx-bun 0.0.9 -> 0.0.11\",\n")
        f.write("# turboquant-tables.ts). Written by tests/golden/make_lloyd_fit.py; binary64 as hex.\n")
        f.write("centroids: " + " ".join(float(v).hex() for v in c) + "\n")
        f.write("boundaries: " + " ".join(float(v).hex() for v in b) + "\n")
    print(OUT)


if __name__ == "__main__":
    main()
