"""Kernel timing through the C ABI (tq_time_next_call): events bound to the
first and last dispatch of a call give its device time, which lies inside
events recorded around the call; a timed call's results equal an untimed
call's bit for bit; with timing armed, a capturing stream is refused before
anything launches, and the refused call disarms. Also the binding's prepared
calls (arguments marshalled once), through which the benchmark launches."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import kv_cache_quantization_tq_amd as tq
from kv_cache_quantization_tq_amd import workloads as W
from kv_cache_quantization_tq_amd.hiprt import HipEvent, HipGraph

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tq.lib()


def randn(shape, dtype, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=DEV, dtype=torch.float32).to(dtype)


def timed(call):
    """Run `call` with timing armed, between two events recorded around it;
    returns (bound interval, outer interval) in milliseconds."""
    s = torch.cuda.current_stream().cuda_stream
    outer0, outer1, a, b = (HipEvent(s) for _ in range(4))
    torch.cuda.synchronize()
    outer0.record()
    tq.time_next_call(a, b)
    call()
    outer1.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b), outer0.elapsed_time(outer1)


def test_timed_encode_and_decode_at_the_prefill_size():
    w = W.WORKLOADS["prefill"]
    print(f"[timing] encode + decode, {w.rows} rows, d={w.head_dim}", flush=True)
    k, v = W.make_kv(w, DEV)
    kw = dict(v_bits=w.v_bits, k_bits=w.k_bits, k_signed=w.k_signed)
    ref = tq.encode_kv(k, v, **kw)
    out = tq.empty_planes(w.rows, w.head_dim, w.k_bits, w.v_bits, DEV)
    inner, outer = timed(lambda: tq.encode_kv(k, v, out=out, **kw))
    assert 0 < inner <= outer
    for n in ref:
        assert torch.equal(ref[n], out[n]), n
    dk = dict(tokens=w.kv_tokens, heads=w.heads, head_dim=w.head_dim, **kw)
    ko0, vo0 = tq.decode_kv(ref, **dk)
    ko, vo = torch.empty_like(ko0), torch.empty_like(vo0)
    inner, outer = timed(lambda: tq.decode_kv(ref, k_out=ko, v_out=vo, **dk))
    assert 0 < inner <= outer
    assert torch.equal(ko.view(torch.int16), ko0.view(torch.int16))
    assert torch.equal(vo.view(torch.int16), vo0.view(torch.int16))


def test_stop_event_alone_ends_at_the_last_kernel():
    """A stop event alone: the interval from an event recorded before the
    call to it covers the call (no shorter than the start-bound interval of
    the same call made again) and ends before an event recorded after it."""
    T, H, d = 20000, 8, 128
    print(f"[timing] stop event only, encode of {T} tokens x {H} heads", flush=True)
    k, v = randn((T, H, d), torch.bfloat16, 41), randn((T, H, d), torch.bfloat16, 42)
    out = tq.empty_planes(T * H, d, 4, 4, DEV)
    call = tq.encode_kv(k, v, v_bits=4, k_bits=4, out=out, prepare=True)
    call()
    s = torch.cuda.current_stream().cuda_stream
    before, stop, after = HipEvent(s), HipEvent(s), HipEvent(s)
    torch.cuda.synchronize()
    before.record()
    tq.time_next_call(None, stop)
    call()
    after.record()
    torch.cuda.synchronize()
    to_stop, total = before.elapsed_time(stop), before.elapsed_time(after)
    inner, _ = timed(call)
    assert 0 < to_stop <= total
    assert to_stop >= 0.5 * inner


def test_timed_attention_spans_both_launches():
    T, H, hq, d, kb, vb = 20000, 8, 32, 256, 4, 5
    print(f"[timing] attention, width {T}, {H} KV heads, {hq} query heads, d={d}", flush=True)
    cache = tq.encode_kv(randn((T, H, d), torch.bfloat16, 11), randn((T, H, d), torch.bfloat16, 12),
                         v_bits=vb, k_bits=kb)
    q = randn((1, hq, d), torch.bfloat16, 13)
    args = dict(batch=1, width=T, kv_heads=H, head_dim=d, k_bits=kb, v_bits=vb)
    ws = torch.empty(int(tq.lib().tq_attention_workspace_bytes(1, H, hq, d, T)), dtype=torch.uint8, device=DEV)
    ref = tq.attention_decode(q, cache, workspace=ws, **args)
    out = torch.empty_like(ref)
    inner, outer = timed(lambda: tq.attention_decode(q, cache, out=out, workspace=ws, **args))
    assert 0 < inner <= outer
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))


def test_timed_fit_spans_its_launch_sequence():
    n, levels, its = 1 << 16, 16, 20
    print(f"[timing] Lloyd-Max fit, {n} samples, {levels} levels, {its} iterations", flush=True)
    x = torch.from_numpy(W.lloyd_samples(n, seed=5)).to(DEV)
    init = tq.lloyd_max_table(4)[0].astype(np.float64)
    ref = tq.lloyd_max_fit(x, levels, init, its)
    got = {}
    inner, outer = timed(lambda: got.update(r=tq.lloyd_max_fit(x, levels, init, its)))
    assert 0 < inner <= outer
    np.testing.assert_array_equal(np.asarray(got["r"][0]), np.asarray(ref[0]))


def test_armed_timing_refuses_a_capturing_stream():
    T, H, d = 64, 2, 128
    print("[timing] armed call under stream capture", flush=True)
    k, v = randn((T, H, d), torch.bfloat16, 21), randn((T, H, d), torch.bfloat16, 22)
    ref = tq.encode_kv(k, v, v_bits=4, k_bits=4)
    out = tq.empty_planes(T * H, d, 4, 4, DEV)
    s = torch.cuda.current_stream().cuda_stream
    a, b = HipEvent(s), HipEvent(s)
    torch.cuda.synchronize()

    def record():
        tq.time_next_call(a, b)
        tq.encode_kv(k, v, v_bits=4, k_bits=4, out=out)

    with pytest.raises(tq.TQError) as e:
        HipGraph(torch, record)
    assert e.value.status == tq.TQ_E_CAPTURE
    # the refused call disarmed: the same call now captures and replays
    g = HipGraph(torch, lambda: tq.encode_kv(k, v, v_bits=4, k_bits=4, out=out))
    try:
        g.launch()
        g.synchronize()
    finally:
        g.close()
    torch.cuda.synchronize()
    for n in ref:
        assert torch.equal(ref[n], out[n]), n


def test_prepared_calls_equal_the_keyword_calls():
    """PreparedCall (arguments marshalled once, as the benchmark's launch
    loops use it) makes the same C call as the keyword functions: outputs
    equal bit for bit, eagerly and rebound to a capturing stream."""
    T, H, d, kb, vb = 3000, 4, 256, 4, 5
    print(f"[timing] prepared calls, {T} tokens x {H} heads, d={d}", flush=True)
    k, v = randn((T, H, d), torch.bfloat16, 31), randn((T, H, d), torch.bfloat16, 32)
    ref = tq.encode_kv(k, v, v_bits=vb, k_bits=kb)
    kd, vd = tq.decode_kv(ref, tokens=T, heads=H, head_dim=d, v_bits=vb, k_bits=kb, rotated_v=True)
    q = randn((1, 16, d), torch.bfloat16, 33)
    args = dict(batch=1, width=T, kv_heads=H, head_dim=d, k_bits=kb, v_bits=vb)
    ws = torch.empty(int(tq.lib().tq_attention_workspace_bytes(1, H, 16, d, T)), dtype=torch.uint8, device=DEV)
    att = tq.attention_decode(q, ref, workspace=ws, **args)
    un = tq.unrotate_values(att)

    planes = tq.empty_planes(T * H, d, kb, vb, DEV)
    ko, vo = torch.empty_like(kd), torch.empty_like(vd)
    att2, un2 = torch.empty_like(att), torch.empty_like(un)
    calls = [tq.encode_kv(k, v, v_bits=vb, k_bits=kb, out=planes, prepare=True),
             tq.decode_kv(planes, tokens=T, heads=H, head_dim=d, v_bits=vb, k_bits=kb, rotated_v=True, k_out=ko,
                          v_out=vo, prepare=True),
             tq.attention_decode(q, planes, out=att2, workspace=ws, prepare=True, **args),
             tq.unrotate_values(att2, out=un2, prepare=True)]
    assert all(isinstance(c, tq.PreparedCall) for c in calls)

    def check():
        torch.cuda.synchronize()
        for n in ref:
            assert torch.equal(ref[n], planes[n]), n
        assert torch.equal(ko.view(torch.int16), kd.view(torch.int16))
        assert torch.equal(vo.view(torch.int16), vd.view(torch.int16))
        assert torch.equal(att2.view(torch.int32), att.view(torch.int32))
        assert torch.equal(un2.view(torch.int32), un.view(torch.int32))

    def clear():
        for t in (*planes.values(), ko, vo, att2, un2):
            t.zero_()
        torch.cuda.synchronize()

    for c in calls:
        c()
    check()
    clear()
    g = HipGraph(torch, lambda: [c.on(torch.cuda.current_stream().cuda_stream)() for c in calls])
    try:
        for _ in range(2):
            g.launch()
            g.synchronize()
            check()
            clear()
    finally:
        g.close()


def test_stop_event_alone_refuses_capture_before_any_launch():
    """Armed with a stop event only, a two-launch call (attention) on a
    capturing stream returns TQ_E_CAPTURE before its first launch: the
    captured graph holds no node."""
    import ctypes
    import gc

    from kv_cache_quantization_tq_amd.hiprt import HIP_STREAM_CAPTURE_MODE_GLOBAL, HIP_STREAM_NON_BLOCKING, hip

    T, H, hq, d = 2000, 4, 16, 128
    print("[timing] stop event only, attention under stream capture", flush=True)
    cache = tq.encode_kv(randn((T, H, d), torch.bfloat16, 51), randn((T, H, d), torch.bfloat16, 52),
                         v_bits=4, k_bits=4)
    q = randn((1, hq, d), torch.bfloat16, 53)
    ws = torch.empty(int(tq.lib().tq_attention_workspace_bytes(1, H, hq, d, T)), dtype=torch.uint8, device=DEV)
    out = torch.empty((1, hq, d), device=DEV)
    call = tq.attention_decode(q, cache, batch=1, width=T, kv_heads=H, head_dim=d, k_bits=4, v_bits=4, out=out,
                               workspace=ws, prepare=True)
    L = hip()
    L.hipGraphGetNodes.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)]
    s = ctypes.c_void_p()
    assert L.hipStreamCreateWithFlags(ctypes.byref(s), HIP_STREAM_NON_BLOCKING) == 0
    stop = HipEvent(s.value)
    on_s = call.on(s.value)
    torch.cuda.synchronize()
    graph = ctypes.c_void_p()
    status = None
    gc.collect()
    gc.disable()  # no destructor may call the runtime during a global-mode capture
    try:
        assert L.hipStreamBeginCapture(s, HIP_STREAM_CAPTURE_MODE_GLOBAL) == 0
        try:
            tq.time_next_call(None, stop)
            on_s()
        except tq.TQError as e:
            status = e.status
        finally:
            end = L.hipStreamEndCapture(s, ctypes.byref(graph))
    finally:
        gc.enable()
    try:
        assert end == 0
        assert status == tq.TQ_E_CAPTURE
        n = ctypes.c_size_t(99)
        assert L.hipGraphGetNodes(graph, None, ctypes.byref(n)) == 0
        assert n.value == 0
    finally:
        if graph:
            L.hipGraphDestroy(graph)
        L.hipStreamDestroy(s)
