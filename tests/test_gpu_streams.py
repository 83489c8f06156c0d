"""Library calls on two streams at once: independent calls (disjoint
buffers, an attention workspace each) launched alternately on two streams,
so that their kernels overlap, give the same bytes as the same calls made
one after another on one stream. The library keeps no state between calls
beyond the timing events armed for the calling thread."""
from __future__ import annotations

import pytest
import torch

import kv_cache_quantization_tq_amd as tq

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tq.lib()


def randn(shape, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=DEV, dtype=torch.float32).to(torch.bfloat16)


def test_codec_calls_on_two_streams_equal_one_stream():
    T, H, d, kb, vb, nsets = 8192, 8, 128, 4, 4, 4
    print(f"[streams] encode + decode of {nsets} sets of {T} tokens x {H} heads, d={d}", flush=True)
    kw = dict(v_bits=vb, k_bits=kb)
    dk = dict(tokens=T, heads=H, head_dim=d, **kw)
    inputs = [(randn((T, H, d), 2 * s), randn((T, H, d), 2 * s + 1)) for s in range(nsets)]

    def outputs():
        planes = [tq.empty_planes(T * H, d, kb, vb, DEV) for _ in range(nsets)]
        dec = [(torch.empty((T, H, d), dtype=torch.bfloat16, device=DEV),
                torch.empty((T, H, d), dtype=torch.bfloat16, device=DEV)) for _ in range(nsets)]
        calls = [(tq.encode_kv(k, v, out=p, prepare=True, **kw),
                  tq.decode_kv(p, k_out=ko, v_out=vo, prepare=True, **dk))
                 for (k, v), p, (ko, vo) in zip(inputs, planes, dec)]
        return planes, dec, calls

    planes1, dec1, calls1 = outputs()
    for enc, de in calls1 * 3:
        enc()
        de()
    torch.cuda.synchronize()

    planes2, dec2, calls2 = outputs()
    main = torch.cuda.current_stream()
    side = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in side:
        s.wait_stream(main)
    for rep in range(3):
        for i, (enc, de) in enumerate(calls2):
            s = side[i % 2].cuda_stream  # set i always on stream i mod 2
            enc.on(s)()
            de.on(s)()
    for s in side:
        main.wait_stream(s)
    torch.cuda.synchronize()
    for a, b in zip(planes1, planes2):
        for n in a:
            assert torch.equal(a[n], b[n]), n
    for (k1, v1), (k2, v2) in zip(dec1, dec2):
        assert torch.equal(k1.view(torch.int16), k2.view(torch.int16))
        assert torch.equal(v1.view(torch.int16), v2.view(torch.int16))


def test_attention_on_two_streams_equals_one_stream():
    T, H, hq, d, kb, vb, n = 6000, 8, 32, 256, 4, 5, 4
    print(f"[streams] {n} attention calls over {T} tokens x {H} KV heads, d={d}, two streams", flush=True)
    cache = tq.encode_kv(randn((T, H, d), 101), randn((T, H, d), 102), v_bits=vb, k_bits=kb)
    qs = [randn((1, hq, d), 110 + i) for i in range(n)]
    args = dict(batch=1, width=T, kv_heads=H, head_dim=d, k_bits=kb, v_bits=vb)
    wsb = int(tq.lib().tq_attention_workspace_bytes(1, H, hq, d, T))

    def calls():
        outs = [torch.empty((1, hq, d), device=DEV) for _ in range(n)]
        wss = [torch.empty(wsb, dtype=torch.uint8, device=DEV) for _ in range(n)]
        return outs, [tq.attention_decode(q, cache, out=o, workspace=w, prepare=True, **args)
                      for q, o, w in zip(qs, outs, wss)]

    outs1, c1 = calls()
    for c in c1:
        c()
    torch.cuda.synchronize()
    outs2, c2 = calls()
    main = torch.cuda.current_stream()
    side = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in side:
        s.wait_stream(main)
    for i, c in enumerate(c2):
        c.on(side[i % 2].cuda_stream)()
    for s in side:
        main.wait_stream(s)
    torch.cuda.synchronize()
    for a, b in zip(outs1, outs2):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
