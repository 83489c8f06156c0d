"""Token-axis batching of packed caches -- TEST INFRASTRUCTURE (oracle).

Plain numpy restatement of the page "mlx-bun 0.0.9 -> 0.0.11",
src/model/batched-quant.ts: ``leftPadTo``, ``mergeQuantRows``,
``extendQuantRows``, ``extractQuantRow``, ``filterQuantRows``. The page
works on [B, H, S, *] triples and pads / concatenates / slices / takes along
the token and batch axes; the codec's planes are token-major instead
([tokens(x batch), heads, row bytes]), so a sequence is a block of
consecutive tokens and a batch of b sequences of width W is b * W tokens.
The operations are the same index arithmetic on that layout, written out
with numpy slicing and concatenation. Only ``tests/`` use this module.

A cache is a dict of planes (numpy arrays [tokens * heads, row_bytes] or
[tokens * heads, G]) holding any subset of the five plane names.
"""
from __future__ import annotations

import numpy as np


def _tokens(plane: np.ndarray, heads: int) -> np.ndarray:
    """A plane viewed as [tokens, heads, row]."""
    return plane.reshape(plane.shape[0] // heads, heads, plane.shape[1])


def _flat(a: np.ndarray) -> np.ndarray:
    return a.reshape(a.shape[0] * a.shape[1], a.shape[2])


def left_pad_to(a: np.ndarray, pad: int) -> np.ndarray:
    """batched-quant.ts leftPadTo: `pad` zero tokens in front (axis 0 here,
    the token axis of one sequence [tokens, heads, row])."""
    z = np.zeros((pad,) + a.shape[1:], a.dtype)
    return np.concatenate([z, a], axis=0)


def n_tokens(cache: dict, heads: int) -> int:
    p = next(iter(cache.values()))
    return p.shape[0] // heads


def merge_rows(caches, heads: int, width: int | None = None):
    """mergeQuantRows: width = max length (or the given larger width), each
    cache left-padded to it, stacked along the batch axis. Returns
    (planes, left_pad, width)."""
    lens = [n_tokens(c, heads) for c in caches]
    w = max(lens) if width is None else width
    assert w >= max(lens)
    left_pad = [w - n for n in lens]
    out = {}
    for name in caches[0]:
        seqs = [left_pad_to(_tokens(c[name], heads), p) for c, p in zip(caches, left_pad)]
        out[name] = _flat(np.concatenate(seqs, axis=0))
    return out, left_pad, w


def _sequences(plane: np.ndarray, b: int, width: int, heads: int) -> np.ndarray:
    """A batch plane viewed as [b, width, heads, row]."""
    return plane.reshape(b, width, heads, plane.shape[1])


def extend_rows(batch, b: int, width: int, left_pad, row, heads: int, new_width: int | None = None):
    """extendQuantRows: width' = max(width, row length) (or the given larger
    width); the batch is padded by width' - width (existing pads grow), the
    row by width' - row length, and the row appended. Returns (planes,
    left_pad', width')."""
    lr = n_tokens(row, heads)
    w = max(width, lr) if new_width is None else new_width
    assert w >= width and w >= lr
    out = {}
    for name in row:
        parts = []
        if b > 0:
            seqs = _sequences(batch[name], b, width, heads)
            for s in range(b):
                parts.append(left_pad_to(seqs[s], w - width))
        parts.append(left_pad_to(_tokens(row[name], heads), w - lr))
        out[name] = _flat(np.concatenate(parts, axis=0))
    return out, [p + (w - width) for p in left_pad] + [w - lr], w


def extract_row(batch, b: int, width: int, left_pad: int, i: int, heads: int):
    """extractQuantRow: sequence i from its left pad to the end."""
    return {name: _flat(_sequences(p, b, width, heads)[i, left_pad:].copy()) for name, p in batch.items()}


def filter_rows(batch, b: int, width: int, keep, heads: int):
    """filterQuantRows: sequences keep[0], keep[1], ... along the batch axis."""
    keep = np.asarray(keep, dtype=np.int64)
    out = {}
    for name, p in batch.items():
        seqs = _sequences(p, b, width, heads)
        out[name] = _flat(seqs[keep].reshape(len(keep) * width, heads, p.shape[1]))
    return out
