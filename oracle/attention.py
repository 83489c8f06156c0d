"""Attention of one query token over a packed cache -- TEST INFRASTRUCTURE
(oracle).

The page "@mlx-bun/inference 0.0.0-stage -> 1.0.0", ops.ts
(``decodeValuesRotated`` and ``unrotateValues``) describes the read path
this follows: keys are decoded (``decodeKeys``, bf16), values are decoded
only to the rotated domain (centroid x scale, bf16), attention runs on
those, and because attention is linear in V the output is un-rotated once
per query row instead of un-rotating every cached token. Written out in
binary64 from the codec oracle's decoded rows:

    s_t   = scale * <q, K_t>            over the valid tokens t of a sequence
    p     = softmax(s)
    o_rot = sum_t p_t * Vrot_t
    o     = signs * (H o_rot) / sqrt(d) (the inverse rotation: natural-order
                                         Hadamard, then the sign vector)

A batch is b sequences of width W tokens, token-major as the codec's planes
(sequence s holds tokens [s*W, (s+1)*W)); sequence s is left-padded by
left_pad[s] tokens, which take no part. Query head h reads KV head
h // (q_heads / kv_heads). A sequence with no valid token gives zeros.
Only ``tests/`` and ``bench.py``'s CPU baseline use this module.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import hadamard

import oracle as O


def bf16_bits_to_f64(u):
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def decoded_cache(planes, rows: int, head_dim: int, k_bits: int, v_bits: int, k_signed: bool = False):
    """K (bf16, decodeKeys) and rotated V (bf16, decodeValuesRotated) as
    binary64 arrays [rows, head_dim]."""
    k, v = O.decode_kv(planes, rows=rows, head_dim=head_dim, k_bits=k_bits, v_bits=v_bits, k_signed=k_signed,
                       out_dtype="bf16", rotated_v=True)
    return bf16_bits_to_f64(k), bf16_bits_to_f64(v)


def unrotate_f64(x, head_dim: int):
    """Inverse rotation in binary64: natural-order Hadamard / sqrt(d), then
    the sign vector (decode direction of ops.ts fwht)."""
    H = hadamard(head_dim).astype(np.float64)
    s = O.signs(head_dim).astype(np.float64)
    return (np.asarray(x, np.float64) @ H.T) / np.sqrt(head_dim) * s


def attention_decode(q, k_dec, v_rot, batch: int, width: int, left_pad, kv_heads: int, scale: float):
    """q: [batch, q_heads, d]; k_dec, v_rot: [batch * width * kv_heads, d]
    (binary64 decoded rows). Returns o [batch, q_heads, d] in binary64."""
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    g = Hq // kv_heads
    K = k_dec.reshape(batch, width, kv_heads, d)
    V = v_rot.reshape(batch, width, kv_heads, d)
    o_rot = np.zeros((B, Hq, d))
    for b in range(B):
        t0 = int(left_pad[b]) if left_pad is not None else 0
        if t0 >= width:
            continue
        for h in range(Hq):
            j = h // g
            s = scale * (K[b, t0:, j, :] @ q[b, h])
            p = np.exp(s - s.max())
            p /= p.sum()
            o_rot[b, h] = p @ V[b, t0:, j, :]
    out = unrotate_f64(o_rot.reshape(-1, d), d).reshape(B, Hq, d)
    for b in range(B):
        if left_pad is not None and int(left_pad[b]) >= width:
            out[b] = 0.0
    return out
