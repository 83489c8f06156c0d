"""Pins of the batching oracle (oracle/batching.py) against what the page
"mlx-bun 0.0.9 -> 0.0.11", src/model/batched-quant.ts fixes: the left-pad
arithmetic of mergeQuantRows / extendQuantRows, extraction past the pad,
take semantics of filterQuantRows, and the property the page's header
states -- token-axis surgery never touches a quantisation group, so every
sequence's bytes (and hence its decoded values) come out unchanged and pad
tokens decode to zero. The decode checks use the codec oracle, a separate
code path."""
import numpy as np
import pytest

import oracle as O
from oracle import batching as B

HEADS = 2
D = 64
KB, VB = 3, 2   # 24-byte key rows: not a multiple of 16


def cache(tokens, seed):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((tokens * HEADS, D)).astype(np.float32)
    v = rng.standard_normal((tokens * HEADS, D)).astype(np.float32)
    return O.encode_kv(k, v, head_dim=D, k_bits=KB, v_bits=VB)


def decode(planes, tokens):
    return O.decode_kv(planes, rows=tokens * HEADS, head_dim=D, k_bits=KB, v_bits=VB, out_dtype="f32")


def test_merge_left_pad_arithmetic():
    cs = [cache(n, s) for s, n in enumerate((3, 5, 2))]
    out, pad, w = B.merge_rows(cs, HEADS)
    assert w == 5 and pad == [2, 0, 3]
    assert out["k_codes"].shape == (3 * 5 * HEADS, D * KB // 8)
    # a wider batch pads every sequence further
    out2, pad2, w2 = B.merge_rows(cs, HEADS, width=8)
    assert w2 == 8 and pad2 == [5, 3, 6]


def test_extend_pads_grow_and_never_shrink():
    cs = [cache(n, s) for s, n in enumerate((3, 5))]
    batch, pad, w = B.merge_rows(cs, HEADS)
    out, pad2, w2 = B.extend_rows(batch, 2, w, pad, cache(7, 9), HEADS)
    assert w2 == 7 and pad2 == [4, 2, 0]
    out3, pad3, w3 = B.extend_rows(out, 3, w2, pad2, cache(1, 10), HEADS)
    assert w3 == 7 and pad3 == [4, 2, 0, 6]
    # extending an empty batch is a single left-padded row
    out4, pad4, w4 = B.extend_rows(None, 0, 0, [], cache(4, 11), HEADS)
    assert w4 == 4 and pad4 == [0]


def test_merge_then_extract_returns_every_sequence_byte_exact():
    lens = (6, 1, 9, 4, 0)
    cs = [cache(n, 20 + s) for s, n in enumerate(lens)]
    batch, pad, w = B.merge_rows(cs, HEADS)
    for i, c in enumerate(cs):
        got = B.extract_row(batch, len(cs), w, pad[i], i, HEADS)
        for name in c:
            np.testing.assert_array_equal(got[name], c[name])


def test_pad_tokens_decode_to_zero_and_real_tokens_decode_unchanged():
    lens = (5, 2, 7)
    cs = [cache(n, 30 + s) for s, n in enumerate(lens)]
    batch, pad, w = B.merge_rows(cs, HEADS)
    kb, vb = decode(batch, len(cs) * w)
    kb = kb.reshape(len(cs), w, HEADS, D)
    vb = vb.reshape(len(cs), w, HEADS, D)
    for i, c in enumerate(cs):
        kc, vc = decode(c, lens[i])
        assert np.all(kb[i, :pad[i]] == 0) and np.all(vb[i, :pad[i]] == 0)
        np.testing.assert_array_equal(kb[i, pad[i]:], kc.reshape(lens[i], HEADS, D))
        np.testing.assert_array_equal(vb[i, pad[i]:], vc.reshape(lens[i], HEADS, D))


def test_filter_is_take_along_the_batch_axis():
    lens = (3, 3, 3, 3)
    cs = [cache(n, 40 + s) for s, n in enumerate(lens)]
    batch, pad, w = B.merge_rows(cs, HEADS)
    got = B.filter_rows(batch, 4, w, [3, 1], HEADS)
    want, _, _ = B.merge_rows([cs[3], cs[1]], HEADS)
    for name in batch:
        np.testing.assert_array_equal(got[name], want[name])
    ident = B.filter_rows(batch, 4, w, [0, 1, 2, 3], HEADS)
    for name in batch:
        np.testing.assert_array_equal(ident[name], batch[name])
    empty = B.filter_rows(batch, 4, w, [], HEADS)
    assert all(p.shape[0] == 0 for p in empty.values())


def test_extend_then_extract_new_row():
    batch, pad, w = B.merge_rows([cache(4, 50), cache(2, 51)], HEADS)
    row = cache(6, 52)
    out, pad2, w2 = B.extend_rows(batch, 2, w, pad, row, HEADS)
    got = B.extract_row(out, 3, w2, pad2[2], 2, HEADS)
    for name in row:
        np.testing.assert_array_equal(got[name], row[name])
    # the old sequences survive the shift
    old0 = B.extract_row(out, 3, w2, pad2[0], 0, HEADS)
    ref0 = B.extract_row(batch, 2, w, pad[0], 0, HEADS)
    for name in row:
        np.testing.assert_array_equal(old0[name], ref0[name])


@pytest.mark.parametrize("planes", [("k_codes", "k_scale", "k_zero"), ("v_codes", "v_scale")])
def test_one_side_only(planes):
    cs = [{n: c[n] for n in planes} for c in (cache(2, 60), cache(3, 61))]
    out, pad, w = B.merge_rows(cs, HEADS)
    assert set(out) == set(planes) and pad == [1, 0]
