"""Comparison helpers for GPU-vs-oracle parity (test infrastructure).

The bar (per element):
* key codes, key scale/zero planes and value scales: bit-exact;
* value codes: bit-exact, except that at most 1e-4 of the codes may be off
  by one bin, and only where the oracle's normalised value lies within
  1e-5 of the boundary between the two bins;
* decoded outputs of identical packed input: within 1e-5 absolute of the
  oracle, NaN exactly where the oracle has NaN, infinities equal.
"""
from __future__ import annotations

import numpy as np

import oracle as O

INDEX_FLIP_FRACTION = 1e-4
INDEX_FLIP_DISTANCE = 1e-5
DECODE_ABS_TOL = 1e-5


def host_planes(planes: dict) -> dict:
    """GPU plane tensors -> numpy (fp16 planes as uint16 bits)."""
    out = {}
    for n, t in planes.items():
        a = t.detach().cpu().numpy()
        out[n] = a.view(np.uint16) if a.dtype == np.int16 else a
    return out


def device_planes(planes: dict, device) -> dict:
    import torch
    out = {}
    for n, a in planes.items():
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        out[n] = torch.from_numpy(a).to(device)
    return out


def decoded_to_f32(t) -> np.ndarray:
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy()


def oracle_decoded_f32(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a


def assert_decoded_close(got: np.ndarray, want: np.ndarray, what: str) -> float:
    got = np.asarray(got, np.float32).ravel()
    want = np.asarray(want, np.float32).ravel()
    assert got.shape == want.shape, what
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ ({int((gn != wn).sum())} elements)"
    m = ~wn
    g, w = got[m].astype(np.float64), want[m].astype(np.float64)
    same = g == w
    diff = np.where(same, 0.0, np.abs(g - w))
    bad = ~(diff <= DECODE_ABS_TOL)
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond {DECODE_ABS_TOL}; "
                           f"first at {int(np.flatnonzero(bad)[0])}: got {g[bad][0]!r} want {w[bad][0]!r}")
    return float(diff.max()) if diff.size else 0.0


def assert_key_planes_equal(got: dict, want: dict, what: str):
    for n in ("k_codes", "k_scale", "k_zero"):
        assert np.array_equal(got[n], want[n]), (
            f"{what}: {n} differs in {int((got[n] != want[n]).any(axis=-1).sum())} rows")


def assert_value_planes_match(got: dict, want: dict, v_rows_f32: np.ndarray, head_dim: int, bits: int,
                              what: str) -> np.ndarray:
    """v_scale bit-exact; v_codes within the off-by-one rule. `v_rows_f32`
    holds the value rows (binary32) the planes were encoded from, so the
    oracle can recompute the normalised values of any row with a flipped
    code. Returns the mask of rows whose codes differ."""
    assert np.array_equal(got["v_scale"], want["v_scale"]), (
        f"{what}: v_scale differs in {int((got['v_scale'] != want['v_scale']).any(axis=-1).sum())} rows")
    diff_rows = (got["v_codes"] != want["v_codes"]).any(axis=-1)
    if not diff_rows.any():
        return diff_rows
    _, bd = O.lloyd_max(bits)
    flips = 0
    for r in np.flatnonzero(diff_rows):
        gi = O.unpack_bits(got["v_codes"][r], head_dim, bits).astype(np.int32)
        oi = O.unpack_bits(want["v_codes"][r], head_dim, bits).astype(np.int32)
        _, _, z = O.value_encode_row(v_rows_f32[r], bits)
        for e in np.flatnonzero(gi != oi):
            assert abs(gi[e] - oi[e]) == 1, f"{what}: row {r} elem {e}: code {gi[e]} vs {oi[e]}"
            b = bd[min(gi[e], oi[e])]
            assert abs(float(z[e]) - float(b)) < INDEX_FLIP_DISTANCE, (
                f"{what}: row {r} elem {e}: flip at distance {abs(float(z[e]) - float(b))}")
            flips += 1
    total = got["v_codes"].shape[0] * head_dim
    assert flips <= INDEX_FLIP_FRACTION * total, f"{what}: {flips} flipped codes of {total}"
    return diff_rows


def rows_as_f32(x: np.ndarray) -> np.ndarray:
    """Oracle-form input rows (float32 or bf16 bits) as binary32 [rows, d]."""
    if x.dtype == np.uint16:
        x = (x.astype(np.uint32) << 16).view(np.float32)
    return x.reshape(-1, x.shape[-1])


# ---------------------------------------------------------------- full size

def oracle_threads() -> int:
    """Threads for the oracle over row ranges (its C calls release the GIL);
    at most 16, the host share of one GPU."""
    import os
    return max(1, min(16, os.cpu_count() or 1))


def _row_split(n: int, parts: int):
    cuts = [n * i // parts for i in range(parts + 1)]
    return [(cuts[i], cuts[i + 1]) for i in range(parts) if cuts[i + 1] > cuts[i]]


def oracle_encode_threaded(kn, vn, **cfg) -> dict:
    """O.encode_kv over row ranges in threads, planes concatenated in row order."""
    import concurrent.futures as cf
    parts = _row_split(kn.shape[0], oracle_threads())
    with cf.ThreadPoolExecutor(len(parts)) as ex:
        outs = list(ex.map(lambda ab: O.encode_kv(kn[ab[0]:ab[1]], vn[ab[0]:ab[1]], **cfg), parts))
    return {n: np.concatenate([o[n] for o in outs]) for n in outs[0]}


def oracle_decode_threaded(planes: dict, rows: int, **cfg):
    import concurrent.futures as cf
    parts = _row_split(rows, oracle_threads())
    with cf.ThreadPoolExecutor(len(parts)) as ex:
        outs = list(ex.map(lambda ab: O.decode_kv({n: p[ab[0]:ab[1]] for n, p in planes.items()},
                                                    rows=ab[1] - ab[0], **cfg), parts))
    return np.concatenate([o[0] for o in outs]), np.concatenate([o[1] for o in outs])
