"""Seeded synthetic K/V inputs for the codec's workloads.

Input generation only: this module draws random tensors and holds none of
the codec's arithmetic. Both the HIP path and the CPU oracle are fed from
it. The pages measure no dataset, so these distributions stand in for
model K/V caches:

* ``tiny``        1 KV head, head_dim 128, 256 tokens, fp32 N(0,1) (seed 0,
                  numpy PCG64, K drawn before V); token 7 of K is the
                  constant 0.5 (its fp16 zero point overflows to +inf);
                  values 3-bit, keys 8-bit signed affine.
* ``prefill``     batch 1, 8 KV heads, head_dim 128, 32768 tokens, N(0,1)
                  times per-(head, channel) scales drawn log-uniform in
                  [0.1, 10], rounded to bf16; values 4-bit, keys 4-bit.
* ``small_head``  batch 16 x 4096 tokens, 4 KV heads, head_dim 64,
                  Student-t (nu = 4, as Z / sqrt(chi2_4 / 4)) with 2 distinct
                  outlier channels per (tensor, head) scaled x20, bf16;
                  values 2-bit, keys 8-bit signed.
* ``long_decode`` batch 1, 8 KV heads, head_dim 256, 131072 cached tokens
                  from fp32 N(0,1); each step appends one token per head
                  (fp32 N(0,1)) and decodes the whole cache to bf16; values
                  5-bit, keys 4-bit.
* ``long_k8v3``   batch 1, 8 KV heads, head_dim 256, 32768 tokens from fp32
                  N(0,1); values 3-bit, keys 8-bit signed: the ops page's
                  specialised long-sequence decode configuration
                  (tryDecodePackedKv: head_dim 256, 8-bit keys, 3-bit values,
                  at least 8192 tokens).
* ``joint_large`` batch 4 x 65536 tokens, 8 KV heads, head_dim 512, bf16
                  N(0,1) with 1% of the (token, head) rows zeroed (the same
                  rows in K and V); values 8-bit (one byte per code), keys
                  4-bit; one pass decodes K and V together.

* ``batch_merge`` 32 packed caches of 8 KV heads, head_dim 128, values
                  4-bit / keys 4-bit, with lengths drawn uniformly in
                  [4096, 32768] tokens (seed 5), merged into one left-padded
                  batch (the token-axis batching operations move bytes, so
                  the plane contents are seeded random bytes).

Batches fold into the token axis: tensors are [batch * tokens, heads, d].
Small tensors are drawn on the host with numpy; large ones on the target
device with a seeded torch generator, in token chunks.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    tokens: int
    heads: int
    head_dim: int
    dtype: str          # "f32" or "bf16": the dtype of the K/V handed to the encoder
    v_bits: int
    k_bits: int
    k_signed: bool
    seed: int
    kind: str           # distribution recipe

    @property
    def rows(self) -> int:
        return self.batch * self.tokens * self.heads

    @property
    def kv_tokens(self) -> int:
        return self.batch * self.tokens


WORKLOADS = {
    "tiny": Workload("tiny", 1, 256, 1, 128, "f32", 3, 8, True, 0, "gauss_const_row"),
    "prefill": Workload("prefill", 1, 32768, 8, 128, "bf16", 4, 4, False, 1, "gauss_channel_scaled"),
    "small_head": Workload("small_head", 16, 4096, 4, 64, "bf16", 2, 8, True, 2, "student_t_outliers"),
    "long_decode": Workload("long_decode", 1, 131072, 8, 256, "f32", 5, 4, False, 3, "gauss"),
    "joint_large": Workload("joint_large", 4, 65536, 8, 512, "bf16", 8, 4, False, 4, "gauss_zero_rows"),
    "long_k8v3": Workload("long_k8v3", 1, 32768, 8, 256, "f32", 3, 8, True, 8, "gauss"),
}


def scaled(w: Workload, tokens: int, batch: Optional[int] = None) -> Workload:
    """The same recipe with fewer tokens (and optionally a smaller batch)."""
    return Workload(w.name, w.batch if batch is None else batch, tokens, w.heads, w.head_dim, w.dtype,
                    w.v_bits, w.k_bits, w.k_signed, w.seed, w.kind)


def _torch():
    import torch
    return torch


def _gen(device, seed):
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def make_kv(w: Workload, device="cpu", chunk_tokens: int = 16384) -> Tuple["object", "object"]:
    """K and V of workload `w` as torch tensors [batch*tokens, heads, d] on `device`."""
    torch = _torch()
    T, H, D = w.kv_tokens, w.heads, w.head_dim
    out_dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    if w.kind == "gauss_const_row":
        rng = np.random.default_rng(w.seed)
        k = rng.standard_normal((T, H, D), dtype=np.float32)
        v = rng.standard_normal((T, H, D), dtype=np.float32)
        if T > 7:
            k[7, 0, :] = 0.5
        return (torch.from_numpy(k).to(device=device, dtype=out_dt),
                torch.from_numpy(v).to(device=device, dtype=out_dt))
    g = _gen(device, w.seed)
    k = torch.empty((T, H, D), dtype=out_dt, device=device)
    v = torch.empty((T, H, D), dtype=out_dt, device=device)
    if w.kind == "gauss_channel_scaled":
        lo, hi = np.log(0.1), np.log(10.0)
        sk = torch.exp(lo + (hi - lo) * torch.rand((H, D), generator=g, device=device))
        sv = torch.exp(lo + (hi - lo) * torch.rand((H, D), generator=g, device=device))
    elif w.kind == "student_t_outliers":
        sk = torch.ones((H, D), device=device)
        sv = torch.ones((H, D), device=device)
        for s in (sk, sv):
            for h in range(H):
                ch = torch.randperm(D, generator=g, device=device)[:2]
                s[h, ch] = 20.0
    else:
        sk = sv = None
    for t0 in range(0, T, chunk_tokens):
        t1 = min(T, t0 + chunk_tokens)
        for dst, sc in ((k, sk), (v, sv)):
            if w.kind == "student_t_outliers":
                z = torch.randn((t1 - t0, H, D), generator=g, device=device)
                chi = (torch.randn((4, t1 - t0, H, D), generator=g, device=device) ** 2).sum(0)
                x = z / torch.sqrt(chi / 4.0)
            else:
                x = torch.randn((t1 - t0, H, D), generator=g, device=device)
            if sc is not None:
                x = x * sc
            dst[t0:t1] = x.to(out_dt)
    if w.kind == "gauss_zero_rows":
        R = T * H
        nz = int(round(0.01 * R))
        idx = torch.randperm(R, generator=g, device=device)[:nz]
        k.view(R, D)[idx] = 0
        v.view(R, D)[idx] = 0
    return k, v


def append_token(w: Workload, step: int, device="cpu"):
    """The K, V rows [1, heads, d] appended at decode step `step` (fp32 N(0,1))."""
    torch = _torch()
    g = _gen(device, 1000003 * (w.seed + 1) + step)
    k = torch.randn((1, w.heads, w.head_dim), generator=g, device=device)
    v = torch.randn((1, w.heads, w.head_dim), generator=g, device=device)
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    return k.to(dt), v.to(dt)


def random_rows(rows: int, head_dim: int, dtype: str, seed: int, scale: float = 1.0, device="cpu"):
    """Generic [rows, 1, head_dim] N(0, scale^2) K and V for small tests."""
    torch = _torch()
    rng = np.random.default_rng(seed)
    k = (rng.standard_normal((rows, 1, head_dim)) * scale).astype(np.float32)
    v = (rng.standard_normal((rows, 1, head_dim)) * scale).astype(np.float32)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    return torch.from_numpy(k).to(device=device, dtype=dt), torch.from_numpy(v).to(device=device, dtype=dt)


def to_oracle(t) -> np.ndarray:
    """Host numpy view the oracle takes: float32 stays float32, bf16 becomes its uint16 bits."""
    torch = _torch()
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


# ---------------------------------------------------------------- fitting

LLOYD = dict(samples=1 << 24, levels=16, iterations=500, seed=6)


def lloyd_samples(n: int = LLOYD["samples"], seed: int = LLOYD["seed"]) -> np.ndarray:
    """The Lloyd-Max fit workload's samples: n unit-normal float32 draws from
    numpy's PCG64 with `seed` (the tables page fits its tables to unit-normal
    samples), drawn on the host so that any consumer can reproduce them."""
    return np.random.default_rng(seed).standard_normal(n, dtype=np.float32)


# ---------------------------------------------------------------- batching

MERGE = dict(sequences=32, heads=8, head_dim=128, k_bits=4, v_bits=4, min_len=4096, max_len=32768, seed=5)


def merge_lengths(sequences=MERGE["sequences"], lo=MERGE["min_len"], hi=MERGE["max_len"], seed=MERGE["seed"]):
    """Token counts of the caches merged by the batching workload."""
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.integers(lo, hi + 1, sequences)]


def random_planes(tokens: int, heads: int, head_dim: int, k_bits: int, v_bits: int, seed: int, device="cpu"):
    """A plane dict (k_codes, k_scale, k_zero, v_codes, v_scale) of seeded
    random bytes for `tokens` tokens; fp16 planes are int16 tensors."""
    torch = _torch()
    g = _gen(device, seed)
    G = head_dim // 32
    shapes = {"k_codes": (head_dim * k_bits // 8, torch.uint8), "k_scale": (G, torch.int16),
              "k_zero": (G, torch.int16), "v_codes": (head_dim * v_bits // 8, torch.uint8),
              "v_scale": (G, torch.int16)}
    out = {}
    for name, (width, dt) in shapes.items():
        lo, hi = (0, 256) if dt == torch.uint8 else (-32768, 32768)
        out[name] = torch.randint(lo, hi, (tokens * heads, width), generator=g, device=device, dtype=dt)
    return out
