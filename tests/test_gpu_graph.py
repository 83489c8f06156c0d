"""Graph capture of the codec, attention and batching launches.

bench.py times its steps as one replay of a captured graph, so the launches
the library makes must replay exactly: every test below captures calls
through the C ABI into a graph (by torch's graph capture, and by the HIP
runtime's stream capture that bench.py uses), then replays it three times. Before
each replay the graph's outputs are cleared and unrelated eager work of the
same kernels runs, with synchronisations in between; after each replay every
output must equal the eager result bit for bit.
"""
from __future__ import annotations

import gc

import pytest
import torch

import kv_cache_quantization_tq_amd as tq
from kv_cache_quantization_tq_amd import workloads as W
from kv_cache_quantization_tq_amd.hiprt import HipGraph

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tq.lib()


def bits(t):
    """A tensor's raw bits, for exact comparison (NaN payloads included)."""
    return t.view(torch.int16) if t.element_size() == 2 else (t.view(torch.int32) if t.element_size() == 4 else t)


class Captured:
    """The launches of `record` captured either by torch's graph capture or
    by the HIP runtime's stream capture on a stream of its own (what
    bench.py times)."""

    def __init__(self, how, record):
        self.how = how
        if how == "torch":
            # no garbage collection during the capture (a destructor calling
            # the HIP runtime there would abort the process)
            gc.collect()
            gc.disable()
            try:
                self.g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(self.g):
                    record()
            finally:
                gc.enable()
        else:
            self.g = HipGraph(torch, record)
        torch.cuda.synchronize()

    def replay(self):
        if self.how == "torch":
            self.g.replay()
        else:
            self.g.launch()
            self.g.synchronize()
        torch.cuda.synchronize()

    def close(self):
        if self.how != "torch":
            self.g.close()


def check_replays(graph, outs, refs, between):
    try:
        for r in range(3):
            for t in outs:
                t.zero_()
            between(r)
            torch.cuda.synchronize()
            graph.replay()
            for name, got, want in zip(refs.keys(), outs, refs.values()):
                assert torch.equal(bits(got), bits(want)), \
                    f"{graph.how} graph, replay {r}: {name} differs from the eager result"
    finally:
        graph.close()


def randn(shape, dtype, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=DEV, dtype=torch.float32).to(dtype)


HOW = ["torch", "hip"]


@pytest.mark.parametrize("how", HOW)
@pytest.mark.parametrize("tokens,heads,d,vb,kb,ks,dtype", [
    (4096, 8, 128, 4, 4, False, torch.bfloat16),     # the prefill step's configuration, smaller
    (1001, 2, 256, 5, 4, False, torch.float32),      # ragged row count, long-context widths
    (777, 4, 64, 2, 8, True, torch.bfloat16),        # small-head widths, signed 8-bit keys
])
def test_encode_decode_graph_replays(tokens, heads, d, vb, kb, ks, dtype, how):
    k, v = randn((tokens, heads, d), dtype, 11), randn((tokens, heads, d), dtype, 12)
    rows = tokens * heads
    pe = tq.encode_kv(k, v, v_bits=vb, k_bits=kb, k_signed=ks)
    ke, ve = tq.decode_kv(pe, tokens=tokens, heads=heads, head_dim=d, v_bits=vb, k_bits=kb, k_signed=ks)
    torch.cuda.synchronize()
    refs = {**{f"plane {n}": p for n, p in pe.items()}, "decoded K": ke, "decoded V": ve}

    pg = tq.empty_planes(rows, d, kb, vb, DEV)
    kg, vg = torch.empty_like(ke), torch.empty_like(ve)

    def record():
        tq.encode_kv(k, v, v_bits=vb, k_bits=kb, k_signed=ks, out=pg)
        tq.decode_kv(pg, tokens=tokens, heads=heads, head_dim=d, v_bits=vb, k_bits=kb, k_signed=ks,
                     k_out=kg, v_out=vg)

    graph = Captured(how, record)

    ko, vo = randn((tokens, heads, d), dtype, 13), randn((tokens, heads, d), dtype, 14)

    def between(r):  # the same kernels on other data, eagerly
        po = tq.encode_kv(ko, vo, v_bits=vb, k_bits=kb, k_signed=ks)
        tq.decode_kv(po, tokens=tokens, heads=heads, head_dim=d, v_bits=vb, k_bits=kb, k_signed=ks)

    check_replays(graph, [pg[n] for n in pe] + [kg, vg], refs, between)


@pytest.mark.parametrize("how", HOW)
def test_attention_graph_replays(how):
    T, H, hq, d, kb, vb = 3000, 2, 8, 128, 4, 4
    k, v = randn((T, H, d), torch.bfloat16, 21), randn((T, H, d), torch.bfloat16, 22)
    cache = tq.encode_kv(k, v, v_bits=vb, k_bits=kb)
    q = randn((1, hq, d), torch.bfloat16, 23)
    ws = torch.empty(int(tq.lib().tq_attention_workspace_bytes(1, H, hq, d, T)), dtype=torch.uint8, device=DEV)
    ref = tq.attention_decode(q, cache, batch=1, width=T, kv_heads=H, head_dim=d, k_bits=kb, v_bits=vb,
                              workspace=ws)
    torch.cuda.synchronize()
    out = torch.empty_like(ref)
    graph = Captured(how, lambda: tq.attention_decode(q, cache, batch=1, width=T, kv_heads=H, head_dim=d,
                                                      k_bits=kb, v_bits=vb, out=out, workspace=ws))
    q2 = randn((1, hq, d), torch.bfloat16, 24)

    def between(r):  # another query through the same workspace, eagerly
        tq.attention_decode(q2, cache, batch=1, width=T, kv_heads=H, head_dim=d, k_bits=kb, v_bits=vb,
                            workspace=ws)

    check_replays(graph, [out], {"attention output": ref}, between)


@pytest.mark.parametrize("how", HOW)
def test_merge_graph_replays(how):
    H, d, kb, vb = 2, 128, 4, 4
    lens = [300, 0, 517, 129]
    caches = [W.random_planes(n, H, d, kb, vb, seed=31 + i, device=DEV) for i, n in enumerate(lens)]
    width = max(lens)
    ref, _, _ = tq.merge_rows(caches, lens, heads=H, head_dim=d, k_bits=kb, v_bits=vb)
    torch.cuda.synchronize()
    dst = tq.empty_planes(len(lens) * width * H, d, kb, vb, DEV)
    graph = Captured(how, lambda: tq.merge_rows(caches, lens, heads=H, head_dim=d, k_bits=kb, v_bits=vb,
                                                 out=dst))
    other = [W.random_planes(n, H, d, kb, vb, seed=41 + i, device=DEV) for i, n in enumerate(lens)]

    def between(r):  # a merge of other caches, eagerly
        tq.merge_rows(other, lens, heads=H, head_dim=d, k_bits=kb, v_bits=vb)

    check_replays(graph, [dst[n] for n in ref], {f"merged {n}": p for n, p in ref.items()}, between)


def many_caches(n, H, d, kb, vb, seed):
    lens = [37 + 11 * i for i in range(n)]
    return lens, [W.random_planes(m, H, d, kb, vb, seed=seed + i, device=DEV) for i, m in enumerate(lens)]


@pytest.mark.parametrize("how", HOW)
def test_multi_launch_merge_refuses_capture(how):
    """A merge needing more than one launch (30 caches: 300 plane segments,
    120 per launch) returns TQ_E_CAPTURE while its stream captures, having
    launched nothing; launched directly it still works."""
    H, d, kb, vb = 2, 64, 4, 4
    lens, caches = many_caches(30, H, d, kb, vb, seed=61)
    dst = tq.empty_planes(len(lens) * max(lens) * H, d, kb, vb, DEV)
    for p in dst.values():
        p.fill_(0x5A if p.dtype == torch.uint8 else 0x5A5A)
    torch.cuda.synchronize()
    before = {n: p.clone() for n, p in dst.items()}
    with pytest.raises(tq.TQError) as err:
        Captured(how, lambda: tq.merge_rows(caches, lens, heads=H, head_dim=d, k_bits=kb, v_bits=vb, out=dst))
    assert err.value.status == tq.TQ_E_CAPTURE
    torch.cuda.synchronize()
    for n in dst:
        assert torch.equal(dst[n], before[n]), f"plane {n} written by a refused call"
    ref, _, _ = tq.merge_rows(caches, lens, heads=H, head_dim=d, k_bits=kb, v_bits=vb)
    torch.cuda.synchronize()
    assert all(p.numel() > 0 for p in ref.values())


@pytest.mark.skip(reason="a graph replay of 20 captured 32-cache merges (three launches each, 2.9 KB segment "
                         "lists as kernel arguments) faulted the GPU once and no cause has been shown in this "
                         "library's code; such calls now refuse capture (TQ_E_CAPTURE) and this case stays "
                         "off the GPU")
def test_multi_launch_merge_graph_replays():
    H, d, kb, vb = 8, 128, 4, 4
    lens, caches = many_caches(32, H, d, kb, vb, seed=71)
    dst = tq.empty_planes(len(lens) * max(lens) * H, d, kb, vb, DEV)
    graph = Captured("hip", lambda: [tq.merge_rows(caches, lens, heads=H, head_dim=d, k_bits=kb, v_bits=vb,
                                                   out=dst) for _ in range(20)])
    graph.replay()
    graph.close()
