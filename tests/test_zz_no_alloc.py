"""The allocation-free attention entry point, tq_attention_decode_static,
against tq_attention_decode with a caller-owned workspace. Both run the same
kernels with the same split count, so their outputs must be identical bit for
bit. Two calls in a row on the static buffer, the second smaller than the
first, each checked against its workspace twin."""
from __future__ import annotations

import pytest
import torch

import kv_cache_quantization_tq_amd as tq

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def randn(shape, dtype, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=DEV, dtype=torch.float32).to(dtype)


def one_case(batch, width, kv_heads, q_heads, d, kb, vb, ks, q_dtype, out_dtype, pads, seed):
    k = randn((batch * width, kv_heads, d), torch.bfloat16, seed)
    v = randn((batch * width, kv_heads, d), torch.bfloat16, seed + 1)
    cache = tq.encode_kv(k, v, v_bits=vb, k_bits=kb, k_signed=ks)
    q = randn((batch, q_heads, d), q_dtype, seed + 2)
    left_pad = torch.tensor(pads, dtype=torch.int32, device=DEV) if pads is not None else None
    args = dict(batch=batch, width=width, kv_heads=kv_heads, head_dim=d, k_bits=kb, v_bits=vb, k_signed=ks,
                left_pad=left_pad)
    nbytes = int(tq.lib().tq_attention_workspace_bytes(batch, kv_heads, q_heads, d, width))
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV)
    ref = tq.attention_decode(q, cache, out_dtype=out_dtype, workspace=ws, **args)
    out = torch.full_like(ref, float("nan"))
    tq.attention_decode_static(q, cache, out=out, **args)
    torch.cuda.synchronize()
    view = torch.int16 if out.element_size() == 2 else torch.int32
    assert torch.equal(out.view(view), ref.view(view)), \
        f"static-scratch attention differs from the workspace entry point (batch={batch}, width={width})"


def test_static_scratch_attention_equals_workspace_entry_point():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tq.lib()
    print("[no-alloc] call 1: batch 2, width 9000, 8 KV heads, 32 query heads, d=256, V5/K4, f32 out", flush=True)
    one_case(2, 9000, 8, 32, 256, 4, 5, False, torch.bfloat16, torch.float32, [0, 1234], seed=101)
    print("[no-alloc] call 2: batch 1, width 700, 2 KV heads, 8 query heads, d=128, V3/K8s, bf16 out", flush=True)
    one_case(1, 700, 2, 8, 128, 8, 3, True, torch.float32, torch.bfloat16, None, seed=202)


def test_static_attention_replays_in_a_hip_graph():
    """The use it exists for: the allocation-free call captured in a HIP
    graph (stream capture on a stream of its own) and replayed three times,
    with eager calls of the same entry point on another query in between
    (they overwrite the shared static buffer); every replay must reproduce
    the workspace entry point's output bit for bit. One eager call comes
    first: the first call on a device looks up the buffer's address."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_quantization_tq_amd.hiprt import HipGraph

    tq.lib()
    T, H, hq, d, kb, vb = 5000, 4, 16, 256, 4, 5
    print(f"[no-alloc] graph: width {T}, {H} KV heads, {hq} query heads, d={d}, V{vb}/K{kb}", flush=True)
    k = randn((T, H, d), torch.bfloat16, 301)
    v = randn((T, H, d), torch.bfloat16, 302)
    cache = tq.encode_kv(k, v, v_bits=vb, k_bits=kb)
    q, q2 = randn((1, hq, d), torch.bfloat16, 303), randn((1, hq, d), torch.bfloat16, 304)
    args = dict(batch=1, width=T, kv_heads=H, head_dim=d, k_bits=kb, v_bits=vb)
    ws = torch.empty(int(tq.lib().tq_attention_workspace_bytes(1, H, hq, d, T)), dtype=torch.uint8, device=DEV)
    ref = tq.attention_decode(q, cache, workspace=ws, **args)
    ref2 = tq.attention_decode(q2, cache, workspace=ws, **args)
    out, out2 = torch.empty_like(ref), torch.empty_like(ref)
    tq.attention_decode_static(q, cache, out=out, **args)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
    graph = HipGraph(torch, lambda: tq.attention_decode_static(q, cache, out=out, **args))
    try:
        for r in range(3):
            out.zero_()
            out2.zero_()
            tq.attention_decode_static(q2, cache, out=out2, **args)
            torch.cuda.synchronize()
            assert torch.equal(out2.view(torch.int32), ref2.view(torch.int32)), f"eager call before replay {r}"
            graph.launch()
            graph.synchronize()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), f"replay {r}"
    finally:
        graph.close()
