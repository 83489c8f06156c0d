"""Pins of the attention oracle (oracle/attention.py): the deferred
un-rotation identity of ops.ts decodeValuesRotated (attention on rotated
values, un-rotated once, equals attention on fully decoded values, up to
the bf16 rounding of the decoded rows), single-token and uniform-weight
closed forms, hard attention at large scores, left padding, and the
grouped-query head mapping."""
import numpy as np
import pytest

import oracle as O
from oracle import attention as A

D, KB, VB = 64, 4, 3
HKV, G = 2, 2


def cache(batch, width, seed):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((batch * width * HKV, D)).astype(np.float32)
    v = rng.standard_normal((batch * width * HKV, D)).astype(np.float32)
    planes = O.encode_kv(k, v, head_dim=D, k_bits=KB, v_bits=VB)
    kd, vr = A.decoded_cache(planes, batch * width * HKV, D, KB, VB)
    return planes, kd, vr


def query(batch, seed, mag=1.0):
    return np.random.default_rng(seed).standard_normal((batch, HKV * G, D)) * mag


def test_deferred_unrotation_matches_fully_decoded_values():
    planes, kd, vr = cache(2, 40, 1)
    q = query(2, 2)
    o = A.attention_decode(q, kd, vr, 2, 40, [0, 7], HKV, 1 / np.sqrt(D))
    # the eager path: decode V fully (binary32 mode: no bf16 rounding) and attend
    _, vfull = O.decode_kv(planes, rows=2 * 40 * HKV, head_dim=D, k_bits=KB, v_bits=VB, out_dtype="f32")
    vfull = vfull.astype(np.float64).reshape(2, 40, HKV, D)
    K = kd.reshape(2, 40, HKV, D)
    for b, t0 in ((0, 0), (1, 7)):
        for h in range(HKV * G):
            s = K[b, t0:, h // G] @ q[b, h] / np.sqrt(D)
            p = np.exp(s - s.max())
            p /= p.sum()
            want = p @ vfull[b, t0:, h // G]
            # rotated rows are bf16-rounded before the un-rotation: |err| <= 2^-8 |v|
            np.testing.assert_allclose(o[b, h], want, atol=2e-2 * np.abs(vfull).max())
            assert np.abs(o[b, h] - want).max() < np.abs(want).max() * 0.05


def test_single_valid_token_is_its_unrotated_value():
    planes, kd, vr = cache(1, 10, 3)
    q = query(1, 4)
    o = A.attention_decode(q, kd, vr, 1, 10, [9], HKV, 0.3)
    V = vr.reshape(1, 10, HKV, D)
    for h in range(HKV * G):
        np.testing.assert_allclose(o[0, h], A.unrotate_f64(V[0, 9, h // G][None], D)[0], rtol=0, atol=1e-12)


def test_zero_query_gives_the_mean_value():
    planes, kd, vr = cache(1, 25, 5)
    o = A.attention_decode(np.zeros((1, HKV * G, D)), kd, vr, 1, 25, [5], HKV, 1.0)
    V = vr.reshape(1, 25, HKV, D)
    for h in range(HKV * G):
        np.testing.assert_allclose(o[0, h], A.unrotate_f64(V[0, 5:, h // G].mean(0)[None], D)[0], atol=1e-12)


def test_large_scores_pick_the_best_key():
    planes, kd, vr = cache(1, 30, 6)
    q = query(1, 7)
    o = A.attention_decode(q, kd, vr, 1, 30, [0], HKV, 1e4)
    K = kd.reshape(1, 30, HKV, D)
    V = vr.reshape(1, 30, HKV, D)
    for h in range(HKV * G):
        t = int(np.argmax(K[0, :, h // G] @ q[0, h]))
        np.testing.assert_allclose(o[0, h], A.unrotate_f64(V[0, t, h // G][None], D)[0], atol=1e-9)


def test_left_padding_equals_the_unpadded_sequence_and_empty_gives_zero():
    planes, kd, vr = cache(1, 20, 8)
    q = query(1, 9)
    o = A.attention_decode(q, kd, vr, 1, 20, [0], HKV, 0.125)
    # the same sequence left-padded by 12 zero tokens (pad rows decode to zero
    # but must not take part)
    pad_k = np.zeros((12 * HKV, D))
    o2 = A.attention_decode(q, np.concatenate([pad_k, kd]), np.concatenate([pad_k, vr]), 1, 32, [12], HKV, 0.125)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    o3 = A.attention_decode(q, kd, vr, 1, 20, [20], HKV, 0.125)
    assert np.all(o3 == 0)


def test_grouped_query_heads_read_their_kv_head():
    planes, kd, vr = cache(1, 16, 10)
    q = query(1, 11)
    o = A.attention_decode(q, kd, vr, 1, 16, [0], HKV, 0.2)
    # each KV head alone, as a single-head cache
    K = kd.reshape(16, HKV, D)
    V = vr.reshape(16, HKV, D)
    for j in range(HKV):
        oj = A.attention_decode(q[:, j * G:(j + 1) * G], K[:, j].copy(), V[:, j].copy(), 1, 16, [0], 1, 0.2)
        np.testing.assert_allclose(o[:, j * G:(j + 1) * G], oj, atol=1e-12)
