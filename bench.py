#!/usr/bin/env python3
"""Throughput of the TurboQuant KV-cache codec on one MI355X.

    python bench.py [--workload NAME] [--steps K] [--warmup W]

The default workload is the headline one, prefill: batch 1, 8 KV heads,
head_dim 128, 32768 tokens, bf16 K/V with per-channel scales; values 4-bit
Lloyd-Max, keys 4-bit affine. What one step is:

* prefill, small_head  encode K and V of every token into the packed planes,
                       then decode every token back to bf16 K and V; steps
                       rotate over enough independent buffer sets that a
                       step's data cannot stay in the 256 MB last-level cache;
* prefill_encode,      the prefill encode alone, or the prefill decode alone
  prefill_decode       (planes encoded beforehand), over rotating sets;
* long_decode          append one token per head to a 131072-token cache
                       (encode 8 rows at the cache's end), then decode the
                       whole cache to bf16;
* joint_large          one joint decode of packed K and V (262144 tokens x 8
                       heads, head_dim 512) to bf16;
* long_k8v3            one joint decode of the ops page's long-sequence
                       configuration (head_dim 256, K8 signed, V3, 32768
                       tokens x 8 heads);
* deferred_v           the long_decode cache decoded with values left in the
                       rotated domain, then one 32-head attention output
                       un-rotated (the eager decode timed alongside);
* batch_merge          merge 32 packed caches of 4096..32768 tokens into one
                       left-padded batch (the token-axis batching
                       operation; KV tokens = tokens merged);
* lloyd_fit            one 500-iteration Lloyd-Max fit of 16 levels to 2^24
                       samples (value = sample-iterations per second);
* attn_decode          one query token per head attending over the
                       long_decode cache, decoding inside the kernel (KV
                       tokens = cached tokens attended).

Inputs are resident in HBM before timing starts. The timed region is
exactly K steps launched one by one after W warm-up steps, bracketed by
synchronisations and two HIP events on the launch stream (the step time).
Inside it every kernel call carries a HIP event that the library binds to
the end of its last dispatch (tq_time_next_call), which adds nothing to the
launch: a kernel's time is the interval from the previous call's end to its
own, i.e. its device time plus the dispatch gap ahead of it (the Lloyd fit,
which waits for the host, from its first dispatch's start). Steps launch
library calls prepared once (tq.PreparedCall), so that the host keeps ahead
of the GPU.
Prints one JSON line: value = KV tokens per second (one KV token = one
position with K and V of all its heads; for the decode workloads, tokens
decoded), the roofline of the dominant kernel (algorithmic bytes per
launch / its average event-timed duration; beside it the committed
rocprofv3 trace of the workload under profiles/ when that trace was taken
on the current sources), HBM traffic from the committed counter runs under
the same condition, the CPU oracle timed on the host as a baseline, and
`graph_replay`: the same K steps captured in one HIP graph and replayed
once after the timed region (one submission for all kernels; not for the Lloyd fit or
the merge; --no-graph skips it), and `pipelined`: for the workloads that
rotate over an even number of buffer sets, the same K steps with step i
launched on stream i mod 2 (--no-pipeline skips it). Diagnostics go to
stderr.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from kv_cache_quantization_tq_amd.hiprt import HipEvent, HipGraph  # noqa: E402

HEADLINE_METRIC = "KV tokens/sec encode+decode (d=128, 4-bit) and achieved HBM GB/s vs peak"
PEAK_HBM_GBPS = 8000.0

DESCRIPTION = {
    "prefill": "prefill: batch 1, 8 KV heads, head_dim 128, 32768 tokens, bf16 K/V (N(0,1) x per-channel "
               "log-uniform [0.1,10] scales); values 4-bit Lloyd-Max, keys 4-bit affine; encode all + decode "
               "all to bf16",
    "small_head": "small_head: batch 16 x 4096 tokens, 4 KV heads, head_dim 64, bf16 K/V Student-t(4) with 2 "
                  "outlier channels per head x20; values 2-bit, keys 8-bit signed affine; encode all + decode "
                  "all to bf16",
    "long_decode": "long_decode: batch 1, 8 KV heads, head_dim 256, 131072 cached tokens (fp32 N(0,1)) at "
                   "5-bit values / 4-bit keys; per step append 1 token per head, then decode the whole "
                   "cache to bf16",
    "joint_large": "joint_large: batch 4 x 65536 tokens, 8 KV heads, head_dim 512, bf16 N(0,1) with 1% of "
                   "rows zeroed; values 8-bit (unpacked bytes), keys 4-bit; one joint K/V decode to bf16",
    "prefill_encode": "prefill_encode: the prefill inputs (batch 1, 8 KV heads, head_dim 128, 32768 tokens, bf16 "
                      "K/V) encoded alone (values 4-bit, keys 4-bit), rotating over buffer sets so that the inputs "
                      "are read from HBM",
    "prefill_decode": "prefill_decode: the prefill cache (batch 1, 8 KV heads, head_dim 128, 32768 tokens, values "
                      "4-bit, keys 4-bit) decoded to bf16 K and V alone, rotating over buffer sets so that the "
                      "packed planes are read from HBM",
    "long_k8v3": "long_k8v3: the ops page's specialised long-sequence decode configuration (tryDecodePackedKv: "
                 "head_dim 256, 8-bit signed keys, 3-bit values, >= 8192 tokens): 32768 tokens x 8 KV heads from "
                 "fp32 N(0,1), one joint K/V decode to bf16",
    "deferred_v": "deferred_v: the long_decode cache (131072 tokens x 8 KV heads, head_dim 256, V5/K4) decoded "
                  "with values left in the rotated domain (decodeValuesRotated), then one attention output of 32 "
                  "query heads un-rotated (unrotateValues); the eager decode is timed alongside",
    "batch_merge": "batch_merge: 32 packed caches (8 KV heads, head_dim 128, V4/K4 planes of seeded random "
                   "bytes) of 4096..32768 tokens merged into one left-padded batch",
    "lloyd_fit": "lloyd_fit: 4-bit (16-level) Lloyd-Max table fitted to 2^24 N(0,1) float32 samples (numpy "
                 "PCG64 seed 6, drawn on the host), 500 iterations from the printed table",
    "attn_decode": "attn_decode: one query token (32 heads, bf16) attending over the long_decode cache (131072 "
                   "tokens x 8 KV heads, head_dim 256, V5/K4 packed), decoded inside the attention kernel",
}

METRIC = {
    "prefill": HEADLINE_METRIC,
    "small_head": "KV tokens/sec encode+decode (d=64, V2/K8s) and achieved HBM GB/s vs peak",
    "long_decode": "KV tokens/sec decoded per step (append 1 token + full decode, d=256, V5/K4) and "
                   "achieved HBM GB/s vs peak",
    "joint_large": "KV tokens/sec joint K/V decode (d=512, V8/K4) and achieved HBM GB/s vs peak",
    "prefill_encode": "KV tokens/sec encode alone (d=128, V4/K4, bf16 inputs from HBM) and achieved HBM GB/s vs peak",
    "prefill_decode": "KV tokens/sec decode alone (d=128, 4-bit, planes from HBM) and achieved HBM GB/s vs peak",
    "long_k8v3": "KV tokens/sec joint K/V decode (d=256, K8 signed, V3, 32768 tokens) and achieved HBM GB/s vs peak",
    "deferred_v": "KV tokens/sec decoded with deferred value un-rotation (d=256, V5/K4) and achieved HBM GB/s vs "
                  "peak",
    "batch_merge": "KV tokens/sec merged into a left-padded batch (d=128, V4/K4 planes) and achieved HBM GB/s "
                   "vs peak",
    "lloyd_fit": "Lloyd-Max fit sample-iterations/sec (16 levels, 2^24 samples) and achieved HBM GB/s vs peak",
    "attn_decode": "KV tokens/sec attended per decode step over the packed cache (d=256, V5/K4, 32 query heads) "
                   "and achieved HBM GB/s vs peak",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def row_bytes(w):
    """Algorithmic bytes per row (one token of one head) moved by encode and
    by decode: inputs read plus outputs written, tables excluded."""
    d, G = w.head_dim, w.head_dim // 32
    in_b = 4 if w.dtype == "f32" else 2
    planes = d * w.v_bits // 8 + 2 * G + d * w.k_bits // 8 + 4 * G
    return 2 * d * in_b + planes, planes + 2 * d * 2


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.json")


def kernel_kind_of(name):
    """The kind (profiling/build vocabulary) of a bench kernel name."""
    return {"append": "encode", "merge": "merge", "fit": "fit", "attention": "attention"}.get(name, name)


def measured_traffic(workload, kernel):
    """HBM bytes per launch from the committed counter runs, if they were
    taken on the current kernel source."""
    try:
        with open(traffic_file(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    from kv_cache_quantization_tq_amd.build import source_digest
    k = t.get("kernels", {}).get(kernel)
    if not k or k.get("source_sha256") != source_digest(kernel):
        return None
    return int(k["fetch_bytes"] + k["write_bytes"])


def committed_trace(workload, kernel):
    """The kernel-trace figures of `kernel` in profiles/<workload>_kernel_trace.json,
    if they were taken on the kernel's current sources."""
    try:
        with open(os.path.join(ROOT, "profiles", f"{workload}_kernel_trace.json")) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    from kv_cache_quantization_tq_amd.build import source_digest
    k = t.get(kernel)
    if not k or k.get("source_sha256") != source_digest(kernel):
        return None
    if "per_operation_us" in k:  # an operation of several launches: time per operation
        return {**k, "avg_us": k["per_operation_us"], "p10_us": None, "p90_us": None}
    return k


def device_copy_gbps(torch, dev, mib=256, nbuf=6, reps=20):
    """Read + write GB/s of torch's device-to-device copy over rotating
    buffers (context for the roofline: what a plain streaming kernel
    reaches on this GPU)."""
    n = mib * 2 ** 20 // 4
    bufs = [(torch.ones(n, device=dev), torch.empty(n, device=dev)) for _ in range(nbuf)]
    for i in range(nbuf):
        bufs[i][1].copy_(bufs[i][0])
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for i in range(reps):
        bufs[i % nbuf][1].copy_(bufs[i % nbuf][0])
    b.record()
    torch.cuda.synchronize()
    t = a.elapsed_time(b) * 1e-3 / reps
    del bufs
    return 2 * mib * 2 ** 20 / t / 1e9


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, single thread and on all host threads
# ---------------------------------------------------------------------------

def _oracle_threads():
    """Threads for the oracle: the host CPUs this process may run on, at most
    16 (the host share of one GPU on the machines this runs on)."""
    return max(1, min(16, host_cpus()["cpus_usable"]))


def host_cpus():
    """The host's CPU count and how many this process may run on."""
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return {"host_cpus": os.cpu_count() or 1, "cpus_usable": usable}


def _par(fn, rows, threads):
    """Run fn(r0, r1) over `threads` contiguous row ranges at once (the
    oracle's C calls release the GIL)."""
    if threads == 1:
        fn(0, rows)
        return
    cuts = [rows * i // threads for i in range(threads + 1)]
    with cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda i: fn(cuts[i], cuts[i + 1]), range(threads)))


def _passes(fn, min_s=1.0, max_passes=16):
    """Run fn() until it has taken min_s seconds in all (at most max_passes
    times); returns (seconds per pass, passes). On 16 threads one second of
    passes is about 16 s of CPU work."""
    total, n = 0.0, 0
    while n < max_passes and (n == 0 or total < min_s):
        total += fn()
        n += 1
    return total / n, n


def cpu_baseline(w, kn, vn, do_encode, do_decode, tokens_per_row):
    """Oracle throughput on host rows kn, vn ([rows, d] numpy, the workload's
    input dtype): time of encode and/or decode over those rows, single
    thread and on all threads, scaled to KV tokens/s."""
    import oracle as O

    d = w.head_dim
    rows = kn.reshape(-1, d).shape[0]
    kn, vn = kn.reshape(rows, d), vn.reshape(rows, d)
    args = dict(head_dim=d, k_bits=w.k_bits, v_bits=w.v_bits, k_signed=w.k_signed)
    planes = O.encode_kv(kn, vn, **args)  # decode input (untimed when only decode is measured)
    O.decode_kv({n: p[:64] for n, p in planes.items()}, rows=64, **args)  # warm-up, untimed

    def run(threads):
        def enc(r0, r1):
            O.encode_kv(kn[r0:r1], vn[r0:r1], **args)

        def dec(r0, r1):
            O.decode_kv({n: p[r0:r1] for n, p in planes.items()}, rows=r1 - r0, **args)

        t0 = time.perf_counter()
        if do_encode:
            _par(enc, rows, threads)
        if do_decode:
            _par(dec, rows, threads)
        return time.perf_counter() - t0

    t1 = run(1)
    nt = _oracle_threads()
    tn, passes = _passes(lambda: run(nt)) if nt > 1 else (t1, 1)
    kv_tok = rows * tokens_per_row
    what = " + ".join(s for s, on in (("encode", do_encode), ("decode", do_decode)) if on)
    log(f"cpu oracle ({what}, {rows} rows): 1 thread {t1:.2f} s, {nt} threads {tn:.2f} s per pass ({passes} passes)")
    return {"value": kv_tok / tn, "unit": "KV tokens/s", "cores": nt, "kind": "oracle",
            "value_1_thread": kv_tok / t1, **host_cpus(),
            "sample": f"{what} of {rows} rows ({rows // w.heads} tokens x {w.heads} heads) of this workload, "
                      f"rows split over {nt} threads, {passes} passes (single-thread figure alongside, one pass)"}


# ---------------------------------------------------------------------------
# Workload steps
# ---------------------------------------------------------------------------

class Timer:
    """Kernel timing inside the timed region. Every kernel call gets a HIP
    event that the library binds to the end of its last dispatch
    (tq_time_next_call with a stop event only, which adds nothing to the
    launch); a call's time is the interval from the end of the call before
    it (for the first call, the event that opens the region) to its own
    end: its device time plus the dispatch gap ahead of it, and the calls'
    times add up to the region's. Calls that wait for the host (the Lloyd
    fit) are timed from their first dispatch's start instead (`spans`): a
    start event makes the runtime enqueue a marker ahead of the kernel,
    which a host-synchronous call does not notice."""

    def __init__(self, torch, steps, names, spans=()):
        stream = ctypes_stream(torch)
        self.start, self.end = HipEvent(stream), HipEvent(stream)
        self.names = list(names)
        self.spans = set(spans)
        self.ev = [{n: (HipEvent(stream) if n in self.spans else None, HipEvent(stream)) for n in self.names}
                   for _ in range(steps)]

    def per_kernel_ms(self, name):
        out, prev = [], self.start
        for row in self.ev:
            for n in self.names:
                a, b = row[n]
                if n == name:
                    out.append((a if a is not None else prev).elapsed_time(b))
                prev = b
        return out


def arm(tq, ev, name):
    """Bind the step's events for `name` to the next library call (no-op
    outside the timed region)."""
    if ev is not None:
        tq.time_next_call(*ev[name])


def run(call, stream):
    """Issue a prepared library call, on `stream` when one is given (the
    graph capture's stream) or else on the stream it was prepared on. The
    steps prepare their calls once: the binding's per-call marshalling plus
    the HIP runtime's cost of a launch with timing events (~8 us) would
    otherwise pace the launches of the smaller workloads from the host."""
    return call() if stream is None else call.on(stream)()


def ctypes_stream(torch):
    """The current torch stream as the hipStream_t the codec is launched on."""
    return torch.cuda.current_stream().cuda_stream


def setup_encode_decode(torch, tq, W, w, dev, sets_hint):
    """Rotating buffer sets for an encode-all + decode-all step."""
    k0, v0 = W.make_kv(w, dev)
    enc_b, _ = row_bytes(w)
    per_set = w.rows * (enc_b + 2 * w.head_dim * 2 * 2)
    nsets = sets_hint or max(2, math.ceil(1.5 * 2 ** 30 / per_set))
    sets = []
    for s in range(nsets):
        k = k0 if s == 0 else k0.clone()
        v = v0 if s == 0 else v0.clone()
        planes = tq.empty_planes(w.rows, w.head_dim, w.k_bits, w.v_bits, dev)
        ko, vo = torch.empty_like(k, dtype=torch.bfloat16), torch.empty_like(v, dtype=torch.bfloat16)
        sets.append((tq.encode_kv(k, v, v_bits=w.v_bits, k_bits=w.k_bits, k_signed=w.k_signed, out=planes,
                                  prepare=True),
                     tq.decode_kv(planes, tokens=w.kv_tokens, heads=w.heads, head_dim=w.head_dim, v_bits=w.v_bits,
                                  k_bits=w.k_bits, k_signed=w.k_signed, k_out=ko, v_out=vo, prepare=True)))
    log(f"workload {w.name}: {w.rows} rows, {nsets} buffer sets of {per_set / 2**20:.0f} MiB")

    def step(i, ev=None, stream=None):
        enc, dec = sets[i % nsets]
        arm(tq, ev, "encode")
        run(enc, stream)
        arm(tq, ev, "decode")
        run(dec, stream)

    step.sets = nsets  # steps i and j share buffers only when i = j mod nsets

    enc_b, dec_b = row_bytes(w)
    kernels = {"encode": w.rows * enc_b, "decode": w.rows * dec_b}
    tokens = lambda i: w.kv_tokens
    cpu = lambda: cpu_baseline(w, W.to_oracle(k0), W.to_oracle(v0), True, True, 1.0 / w.heads)
    return step, kernels, tokens, cpu, {**codec_config(w), "buffer_sets": nsets}


def setup_long_decode(torch, tq, W, w, dev, max_steps):
    """A cache of w.tokens tokens with room for max_steps appends."""
    T, H, d = w.tokens, w.heads, w.head_dim
    k, v = W.make_kv(w, dev)
    planes = tq.empty_planes((T + max_steps) * H, d, w.k_bits, w.v_bits, dev)
    head = {n: p[: T * H] for n, p in planes.items()}
    tq.encode_kv(k, v, v_bits=w.v_bits, k_bits=w.k_bits, out=head)
    torch.cuda.synchronize()
    sample = (W.to_oracle(k[:32768]), W.to_oracle(v[:32768]))
    del k, v
    appends = [W.append_token(w, s, dev) for s in range(max_steps)]
    ko = torch.empty(((T + max_steps), H, d), dtype=torch.bfloat16, device=dev)
    vo = torch.empty_like(ko)
    row_b = {n: p.shape[1] * p.element_size() for n, p in planes.items()}
    log(f"workload {w.name}: {T} cached tokens x {H} heads, room for {max_steps} appends")
    calls = []
    for i in range(max_steps):
        n = T + i  # tokens already cached
        view = {nm: p[n * H:(n + 1) * H] for nm, p in planes.items()}
        nk, nv = appends[i]
        calls.append((tq.encode_kv(nk, nv, v_bits=w.v_bits, k_bits=w.k_bits, out=view, prepare=True),
                      tq.decode_kv(planes, tokens=n + 1, heads=H, head_dim=d, v_bits=w.v_bits, k_bits=w.k_bits,
                                   k_out=ko[: n + 1], v_out=vo[: n + 1], prepare=True)))

    def step(i, ev=None, stream=None):
        append, dec = calls[i]
        arm(tq, ev, "append")
        run(append, stream)
        arm(tq, ev, "decode")
        run(dec, stream)

    enc_b, dec_b = row_bytes(w)
    # decode bytes of the first timed step's cache length (the cache grows by
    # one token per step: under 0.1% over a run)
    kernels = {"append": H * enc_b, "decode": (T + 1) * H * dec_b}
    tokens = lambda i: T + i + 1
    cpu = lambda: cpu_baseline(w, sample[0], sample[1], False, True, 1.0 / w.heads)
    return step, kernels, tokens, cpu, {**codec_config(w), "cached_tokens": T, "appended_per_step": 1}


def setup_joint(torch, tq, W, w, dev):
    k, v = W.make_kv(w, dev)
    planes = tq.encode_kv(k, v, v_bits=w.v_bits, k_bits=w.k_bits, k_signed=w.k_signed)
    torch.cuda.synchronize()
    ns = 16384 * w.heads  # rows of the oracle sample: the first 16384 tokens
    sample = (W.to_oracle(k.view(-1, w.head_dim)[:ns]), W.to_oracle(v.view(-1, w.head_dim)[:ns]))
    del k, v
    ko = torch.empty((w.kv_tokens, w.heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    vo = torch.empty_like(ko)
    log(f"workload {w.name}: {w.rows} rows")
    dec = tq.decode_kv(planes, tokens=w.kv_tokens, heads=w.heads, head_dim=w.head_dim, v_bits=w.v_bits,
                       k_bits=w.k_bits, k_signed=w.k_signed, k_out=ko, v_out=vo, prepare=True)

    def step(i, ev=None, stream=None):
        arm(tq, ev, "decode")
        run(dec, stream)

    _, dec_b = row_bytes(w)
    cpu = lambda: cpu_baseline(w, sample[0], sample[1], False, True, 1.0 / w.heads)
    return step, {"decode": w.rows * dec_b}, (lambda i: w.kv_tokens), cpu, codec_config(w)


def codec_config(w):
    return {"workload": DESCRIPTION[w.name], "tokens": w.kv_tokens, "heads": w.heads, "head_dim": w.head_dim,
            "v_bits": w.v_bits, "k_bits": w.k_bits, "k_signed": w.k_signed, "input_dtype": w.dtype}


def setup_decode_only(torch, tq, W, w, dev, sets_hint):
    """Decode alone, rotating over buffer sets of planes encoded beforehand
    (untimed), so that each step reads its planes from HBM."""
    k0, v0 = W.make_kv(w, dev)
    _, dec_b = row_bytes(w)
    per_set = w.rows * dec_b
    nsets = sets_hint or max(2, math.ceil(1.5 * 2 ** 30 / per_set))
    sets = []
    for s in range(nsets):
        planes = tq.encode_kv(k0, v0, v_bits=w.v_bits, k_bits=w.k_bits, k_signed=w.k_signed)
        ko, vo = torch.empty_like(k0, dtype=torch.bfloat16), torch.empty_like(v0, dtype=torch.bfloat16)
        sets.append(tq.decode_kv(planes, tokens=w.kv_tokens, heads=w.heads, head_dim=w.head_dim, v_bits=w.v_bits,
                                 k_bits=w.k_bits, k_signed=w.k_signed, k_out=ko, v_out=vo, prepare=True))
    torch.cuda.synchronize()
    ns = min(w.rows, 65536)
    sample = (W.to_oracle(k0.view(-1, w.head_dim)[:ns]), W.to_oracle(v0.view(-1, w.head_dim)[:ns]))
    del k0, v0
    log(f"workload {w.name}: {w.rows} rows, {nsets} plane sets of {per_set / 2**20:.0f} MiB (planes + outputs)")

    def step(i, ev=None, stream=None):
        arm(tq, ev, "decode")
        run(sets[i % nsets], stream)

    step.sets = nsets  # steps i and j share buffers only when i = j mod nsets

    cpu = lambda: cpu_baseline(w, sample[0], sample[1], False, True, 1.0 / w.heads)
    return step, {"decode": w.rows * dec_b}, (lambda i: w.kv_tokens), cpu, \
        {**codec_config(w), "workload": DESCRIPTION[w.name], "buffer_sets": nsets}


def setup_encode_only(torch, tq, W, w, dev, sets_hint):
    """Encode alone, rotating over buffer sets of K/V inputs and planes, so
    that each step reads its inputs from HBM and no decode's output is being
    written back meanwhile."""
    k0, v0 = W.make_kv(w, dev)
    enc_b, _ = row_bytes(w)
    per_set = w.rows * enc_b
    nsets = sets_hint or max(2, math.ceil(1.5 * 2 ** 30 / per_set))
    sets = []
    for s in range(nsets):
        k = k0 if s == 0 else k0.clone()
        v = v0 if s == 0 else v0.clone()
        sets.append(tq.encode_kv(k, v, v_bits=w.v_bits, k_bits=w.k_bits, k_signed=w.k_signed,
                                 out=tq.empty_planes(w.rows, w.head_dim, w.k_bits, w.v_bits, dev), prepare=True))
    torch.cuda.synchronize()
    log(f"workload {w.name}: {w.rows} rows, {nsets} buffer sets of {per_set / 2**20:.0f} MiB (inputs + planes)")

    def step(i, ev=None, stream=None):
        arm(tq, ev, "encode")
        run(sets[i % nsets], stream)

    step.sets = nsets  # steps i and j share buffers only when i = j mod nsets

    cpu = lambda: cpu_baseline(w, W.to_oracle(k0), W.to_oracle(v0), True, False, 1.0 / w.heads)
    return step, {"encode": w.rows * enc_b}, (lambda i: w.kv_tokens), cpu, \
        {**codec_config(w), "workload": DESCRIPTION[w.name], "buffer_sets": nsets}


def setup_deferred_v(torch, tq, W, dev):
    """Rotated-domain value decode plus one un-rotation of an attention
    output per step; the eager decode (inverse transform for every token) of
    the same cache is timed after the timed region for comparison."""
    w = W.WORKLOADS["long_decode"]
    T, H, d, hq = w.tokens, w.heads, w.head_dim, 32
    k, v = W.make_kv(w, dev)
    planes = tq.encode_kv(k, v, v_bits=w.v_bits, k_bits=w.k_bits)
    torch.cuda.synchronize()
    ns = 32768
    sample = (W.to_oracle(k[:ns]), W.to_oracle(v[:ns]))
    del k, v
    ko = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev)
    vo = torch.empty_like(ko)
    g = torch.Generator(device=dev)
    g.manual_seed(9)
    att = torch.randn((1, hq, d), generator=g, device=dev)  # stands for an attention output over rotated values
    att_out = torch.empty_like(att)
    log(f"workload deferred_v: {T} tokens x {H} heads, rotated decode + un-rotation of {hq} rows")
    dec = tq.decode_kv(planes, tokens=T, heads=H, head_dim=d, v_bits=w.v_bits, k_bits=w.k_bits, k_out=ko, v_out=vo,
                       rotated_v=True, prepare=True)
    unrot = tq.unrotate_values(att, out=att_out, prepare=True)
    eager = tq.decode_kv(planes, tokens=T, heads=H, head_dim=d, v_bits=w.v_bits, k_bits=w.k_bits, k_out=ko,
                         v_out=vo, prepare=True)

    def step(i, ev=None, stream=None):
        arm(tq, ev, "decode")
        run(dec, stream)
        arm(tq, ev, "unrotate")
        run(unrot, stream)

    def eager_us(reps=20):
        """Average device time of the eager decode (values fully decoded),
        timed like the kernels of the timed loop."""
        t0 = HipEvent(ctypes_stream(torch))
        ev = [HipEvent(ctypes_stream(torch)) for _ in range(reps)]
        for _ in range(3):
            eager()
        torch.cuda.synchronize()
        t0.record()
        for b in ev:
            tq.time_next_call(None, b)
            eager()
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in zip([t0] + ev[:-1], ev)) / reps * 1e3

    def cpu():
        import oracle as O
        kn, vn = sample
        rows = ns * H
        planes_h = O.encode_kv(kn.reshape(rows, d), vn.reshape(rows, d), head_dim=d, k_bits=w.k_bits,
                               v_bits=w.v_bits)
        O.decode_kv({n: p[:64] for n, p in planes_h.items()}, rows=64, head_dim=d, k_bits=w.k_bits,
                    v_bits=w.v_bits, rotated_v=True)
        att_h = att.cpu().numpy().reshape(-1, d)

        def run(threads):
            def dec(r0, r1):
                O.decode_kv({n: p[r0:r1] for n, p in planes_h.items()}, rows=r1 - r0, head_dim=d,
                            k_bits=w.k_bits, v_bits=w.v_bits, rotated_v=True)
            t0 = time.perf_counter()
            _par(dec, rows, threads)
            O.unrotate(att_h, d)
            return time.perf_counter() - t0

        t1 = run(1)
        nt = _oracle_threads()
        tn, passes = _passes(lambda: run(nt)) if nt > 1 else (t1, 1)
        log(f"cpu oracle (rotated decode of {rows} rows + un-rotation): 1 thread {t1:.2f} s, {nt} threads "
            f"{tn:.2f} s per pass ({passes} passes)")
        return {"value": ns / tn, "unit": "KV tokens/s", "cores": nt, "kind": "oracle", "value_1_thread": ns / t1,
                **host_cpus(),
                "sample": f"rotated decode of the first {ns} tokens x {H} heads plus one un-rotation, rows split "
                          f"over {nt} threads, {passes} passes (single-thread figure alongside, one pass)"}

    _, dec_b = row_bytes(w)
    kernels = {"decode": T * H * dec_b, "unrotate": 2 * hq * d * 4}
    config = {**codec_config(w), "workload": DESCRIPTION["deferred_v"], "q_heads": hq, "rotated_v": True}
    return step, kernels, (lambda i: T), cpu, config, eager_us


def setup_batch_merge(torch, tq, W, dev):
    """Merge 32 caches into one left-padded batch per step."""
    m = W.MERGE
    lens = W.merge_lengths()
    H, d, kb, vb = m["heads"], m["head_dim"], m["k_bits"], m["v_bits"]
    caches = [W.random_planes(n, H, d, kb, vb, seed=m["seed"] * 1000 + i, device=dev) for i, n in enumerate(lens)]
    width = max(lens)
    dst = tq.empty_planes(len(lens) * width * H, d, kb, vb, dev)
    tok_b = H * (d * (kb + vb) // 8 + 6 * (d // 32))  # plane bytes per token
    nbytes = sum(lens) * tok_b + len(lens) * width * tok_b  # read the caches, write the batch
    log(f"workload batch_merge: {len(lens)} caches, {sum(lens)} tokens, width {width}")
    from kv_cache_quantization_tq_amd import _packed, TQConfig, TQPackedKV
    import ctypes
    import numpy as np
    srcs = (TQPackedKV * len(lens))(*[_packed(c) for c in caches])
    lens_a = np.asarray(lens, dtype=np.int64)
    cfg = TQConfig(d, kb, vb, 0)
    pk = _packed(dst)

    stream0 = ctypes_stream(torch)

    def step(i, ev=None, stream=None):
        arm(tq, ev, "merge")
        st = tq.lib().tq_merge_rows(srcs, lens_a.ctypes.data, len(lens), width, H, ctypes.byref(cfg),
                                    ctypes.byref(pk), None, stream0 if stream is None else stream)
        if st:
            raise tq.TQError(st, "tq_merge_rows")

    def cpu():
        import oracle.batching as OB
        host = [{n: (p.cpu().numpy().view(np.uint16) if p.dtype == torch.int16 else p.cpu().numpy())
                 for n, p in c.items()} for c in caches]
        def once():
            t0 = time.perf_counter()
            OB.merge_rows(host, H)
            return time.perf_counter() - t0

        t, passes = _passes(once)
        ntok = sum(lens)
        log(f"cpu oracle (merge of all {len(lens)} caches, {ntok} tokens): {t:.2f} s per pass ({passes} passes)")
        return {"value": ntok / t, "unit": "KV tokens/s", "cores": 1, "kind": "oracle", **host_cpus(),
                "sample": f"the whole merge of the {len(lens)} caches ({ntok} tokens), one thread (numpy), "
                          f"{passes} passes"}

    config = {"workload": DESCRIPTION["batch_merge"], "sequences": len(lens), "tokens": sum(lens), "width": width,
              "heads": H, "head_dim": d, "v_bits": vb, "k_bits": kb}
    return step, {"merge": nbytes}, (lambda i: sum(lens)), cpu, config


def setup_lloyd_fit(torch, tq, W, dev, iterations=500):
    """One full fit per step: the samples are sorted once, then every
    iteration searches the sorted keys."""
    n, levels = W.LLOYD["samples"], W.LLOYD["levels"]
    xh = W.lloyd_samples()
    x = torch.from_numpy(xh).to(dev)
    init = tq.lloyd_max_table(4)[0].astype("float64")
    ws = torch.empty(int(tq.lib().tq_lloyd_max_workspace_bytes(n)), dtype=torch.uint8, device=dev)
    log(f"workload lloyd_fit: {n} samples, {levels} levels, {iterations} iterations per step")

    def step(i, ev=None, stream=None):
        arm(tq, ev, "fit")
        tq.lloyd_max_fit(x, levels, init, iterations, workspace=ws, stream=stream)

    def cpu():
        import numpy as np
        from oracle import lloyd as OL
        ns, it = 1 << 22, 25
        xs = xh[:ns]
        t0 = time.perf_counter()
        OL.fit_samples(xs, init, it)
        t = time.perf_counter() - t0
        log(f"cpu oracle (fit of {ns} samples, {it} iterations): {t:.2f} s")
        return {"value": ns * it / t, "unit": "sample-iterations/s", "cores": 1, "kind": "oracle", **host_cpus(),
                "sample": f"{it} iterations on the first {ns} samples, one thread (numpy)"}

    config = {"workload": DESCRIPTION["lloyd_fit"], "samples": n, "levels": levels, "iterations": iterations}
    # Bytes the sorted method moves per fit: the samples read once for their
    # largest magnitude (4n), four radix passes each reading and writing the
    # 4-byte keys (32n), and the prefix pass reading the keys and writing the
    # int64 prefix sums (12n). The iterations read a few windows of keys and
    # sums per boundary each and are bound by their dependent latency, not by
    # bandwidth.
    return step, {"fit": 48 * n}, (lambda i: n * iterations), cpu, config


def setup_attn_decode(torch, tq, W, dev):
    """The long_decode cache, attended by one bf16 query token of 32 heads."""
    w = W.WORKLOADS["long_decode"]
    T, H, d, hq = w.tokens, w.heads, w.head_dim, 32
    k, v = W.make_kv(w, dev)
    planes = tq.encode_kv(k, v, v_bits=w.v_bits, k_bits=w.k_bits)
    torch.cuda.synchronize()
    ns = 32768  # tokens of the oracle sample
    sample = (W.to_oracle(k[:ns]), W.to_oracle(v[:ns]))
    del k, v
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    q = torch.randn((1, hq, d), generator=g, device=dev).to(torch.bfloat16)
    out = torch.empty((1, hq, d), dtype=torch.float32, device=dev)
    ws = torch.empty(int(tq.lib().tq_attention_workspace_bytes(1, H, hq, d, T)), dtype=torch.uint8, device=dev)
    row_b = d * (w.k_bits + w.v_bits) // 8 + 6 * (d // 32)
    nbytes = T * H * row_b + q.numel() * 2 + out.numel() * 4
    log(f"workload attn_decode: {T} tokens x {H} KV heads, {hq} query heads, {T * H * row_b / 1e6:.1f} MB of cache")

    attn = tq.attention_decode(q, planes, batch=1, width=T, kv_heads=H, head_dim=d, k_bits=w.k_bits,
                               v_bits=w.v_bits, out=out, workspace=ws, prepare=True)

    def step(i, ev=None, stream=None):
        arm(tq, ev, "attention")
        run(attn, stream)

    def cpu():
        import numpy as np
        import oracle as O
        from oracle import attention as OA
        kn, vn = sample
        rows = ns * H
        planes_h = O.encode_kv(kn.reshape(rows, d), vn.reshape(rows, d), head_dim=d, k_bits=w.k_bits,
                               v_bits=w.v_bits)
        qh = q.float().cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        kd, vr = OA.decoded_cache(planes_h, rows, d, w.k_bits, w.v_bits)
        OA.attention_decode(qh, kd, vr, 1, ns, None, H, 1.0 / np.sqrt(d))
        t = time.perf_counter() - t0
        log(f"cpu oracle (decode + attention over {ns} tokens): {t:.2f} s")
        return {"value": ns / t, "unit": "KV tokens/s", "cores": 1, "kind": "oracle", **host_cpus(),
                "sample": f"decode + attention over the first {ns} tokens of the cache, one thread"}

    config = {"workload": DESCRIPTION["attn_decode"], "tokens": T, "kv_heads": H, "q_heads": hq, "head_dim": d,
              "v_bits": w.v_bits, "k_bits": w.k_bits, "q_dtype": "bf16"}
    return step, {"attention": nbytes}, (lambda i: T), cpu, config


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0, help="timed steps (0: 50, or 20 for the decode workloads)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill", choices=sorted(DESCRIPTION))
    ap.add_argument("--sets", type=int, default=0, help="buffer sets to rotate (0: enough for >= 1.5 GiB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph replay of the timed steps reported alongside")
    ap.add_argument("--no-pipeline", action="store_true",
                    help="skip the two-stream run of the timed steps reported alongside")
    ap.add_argument("--no-eager", action="store_true",
                    help="deferred_v: skip timing the eager decode alongside (keeps a kernel trace to the timed steps)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this codec is benchmarked on one GPU only (rows are independent, so a multi-GPU "
              "deployment shards rows with no communication); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import kv_cache_quantization_tq_amd as tq
    from kv_cache_quantization_tq_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    tq.lib()
    dev = torch.device("cuda:0")
    w = W.WORKLOADS.get(args.workload)
    steps = args.steps or {"long_decode": 20, "joint_large": 20, "batch_merge": 20, "lloyd_fit": 3,
                           "attn_decode": 50, "deferred_v": 20, "long_k8v3": 50,
                           "prefill_decode": 50, "prefill_encode": 50}.get(args.workload, 50)

    extra = None
    if args.workload in ("prefill", "small_head"):
        step, kernels, tokens, cpu_fn, config = setup_encode_decode(torch, tq, W, w, dev, args.sets)
    elif args.workload == "prefill_encode":
        w = W.WORKLOADS["prefill"]
        w = W.Workload("prefill_encode", w.batch, w.tokens, w.heads, w.head_dim, w.dtype, w.v_bits, w.k_bits,
                       w.k_signed, w.seed, w.kind)
        step, kernels, tokens, cpu_fn, config = setup_encode_only(torch, tq, W, w, dev, args.sets)
    elif args.workload == "prefill_decode":
        w = W.WORKLOADS["prefill"]
        w = W.Workload("prefill_decode", w.batch, w.tokens, w.heads, w.head_dim, w.dtype, w.v_bits, w.k_bits,
                       w.k_signed, w.seed, w.kind)
        step, kernels, tokens, cpu_fn, config = setup_decode_only(torch, tq, W, w, dev, args.sets)
    elif args.workload == "long_k8v3":
        step, kernels, tokens, cpu_fn, config = setup_joint(torch, tq, W, w, dev)
        config["workload"] = DESCRIPTION["long_k8v3"]
    elif args.workload == "deferred_v":
        step, kernels, tokens, cpu_fn, config, extra = setup_deferred_v(torch, tq, W, dev)
    elif args.workload == "long_decode":
        step, kernels, tokens, cpu_fn, config = setup_long_decode(torch, tq, W, w, dev,
                                                                         args.warmup + steps)
    elif args.workload == "joint_large":
        step, kernels, tokens, cpu_fn, config = setup_joint(torch, tq, W, w, dev)
    elif args.workload == "batch_merge":
        step, kernels, tokens, cpu_fn, config = setup_batch_merge(torch, tq, W, dev)
    elif args.workload == "lloyd_fit":
        step, kernels, tokens, cpu_fn, config = setup_lloyd_fit(torch, tq, W, dev)
    else:
        step, kernels, tokens, cpu_fn, config = setup_attn_decode(torch, tq, W, dev)
    torch.cuda.synchronize()

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * 2 ** 20 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {args.copy_calibration_mib} MiB read + {args.copy_calibration_mib} MiB written")
        del src, dst

    # warm-up steps, timed like the timed region (the first launches with
    # bound events pay a one-time cost)
    spans = ("fit",)
    warm = Timer(torch, args.warmup, kernels, spans)
    for i in range(args.warmup):
        step(i, warm.ev[i])
    torch.cuda.synchronize()

    # the timed region: exactly `steps` steps launched one by one between
    # two events on the launch stream, every kernel call timed by a stop
    # event bound to its last dispatch
    tm = Timer(torch, steps, kernels, spans)
    torch.cuda.synchronize()
    tm.start.record()
    for i in range(steps):
        step(args.warmup + i, tm.ev[i])
    tm.end.record()
    torch.cuda.synchronize()
    ms_per_step = tm.start.elapsed_time(tm.end) / steps
    kv_tokens = sum(tokens(args.warmup + i) for i in range(steps))

    # reported alongside: the same `steps` steps captured in one graph and
    # replayed once (one submission for all their kernels),
    # after an untimed replay that uploads the graph. Not for the Lloyd fit,
    # which reads its result back to the host every step, nor the merge,
    # whose graph replay faulted (its launches carry 2.9 KB segment lists as
    # kernel arguments; the cause is not established)
    graph_ms_per_step = None
    if args.workload not in ("lloyd_fit", "batch_merge") and not args.no_graph:
        graph = HipGraph(torch, lambda: [step(args.warmup + i, None, ctypes_stream(torch)) for i in range(steps)])
        graph.launch()
        graph.synchronize()
        t0, t1 = HipEvent(graph.stream), HipEvent(graph.stream)
        torch.cuda.synchronize()
        t0.record()
        graph.launch()
        t1.record()
        graph.synchronize()
        torch.cuda.synchronize()
        graph_ms_per_step = t0.elapsed_time(t1) / steps
        graph.close()
        log(f"graph replay of the same {steps} steps: {graph_ms_per_step * 1e3:.1f} us per step "
            f"(timed region, launched one by one: {ms_per_step * 1e3:.1f} us)")

    # reported alongside: the same `steps` steps with consecutive steps on
    # two streams (step i on stream i mod 2), for the workloads whose steps
    # rotate over an even number of buffer sets (a set then stays on one
    # stream, so no two steps in flight share a buffer): one kernel's ramp
    # and drain overlap the other stream's, which launching one by one leaves
    # idle. Timed after three untimed passes: on new streams the first two
    # passes overlap less (prefill 67.0, 61.5, 57.9, 57.3 us per step in four
    # consecutive passes on one box)
    pipe_ms_per_step = None
    if getattr(step, "sets", 0) % 2 == 0 and getattr(step, "sets", 0) >= 2 and not args.no_pipeline:
        main_s = torch.cuda.current_stream()
        side = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]

        def pipelined():
            for st in side:
                st.wait_stream(main_s)
            for i in range(steps):
                step(args.warmup + i, None, side[i % 2].cuda_stream)
            for st in side:
                main_s.wait_stream(st)

        for _ in range(3):
            pipelined()
        torch.cuda.synchronize()
        t0, t1 = HipEvent(main_s.cuda_stream), HipEvent(main_s.cuda_stream)
        t0.record()
        pipelined()
        t1.record()
        torch.cuda.synchronize()
        pipe_ms_per_step = t0.elapsed_time(t1) / steps
        log(f"the same {steps} steps on two streams: {pipe_ms_per_step * 1e3:.1f} us per step "
            f"(timed region, one stream: {ms_per_step * 1e3:.1f} us)")

    stats = {}
    for name, nbytes in kernels.items():
        ms = sorted(tm.per_kernel_ms(name))
        avg = sum(ms) / len(ms)
        gbps = nbytes / (avg * 1e-3) / 1e9
        stats[name] = {"avg_us": avg * 1e3, "median_us": ms[len(ms) // 2] * 1e3, "GBps": gbps,
                       "bytes": nbytes, "frac": gbps / PEAK_HBM_GBPS}
        log(f"{name}: avg {avg * 1e3:.1f} us  median {ms[len(ms) // 2] * 1e3:.1f} us  "
            f"{gbps:.0f} GB/s ({gbps / PEAK_HBM_GBPS:.1%} of 8 TB/s)")
    step_bytes = sum(kernels.values())
    step_gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    copy_gbps = device_copy_gbps(torch, dev)
    log(f"step: {ms_per_step * 1e3:.1f} us, {step_gbps:.0f} GB/s ({step_gbps / PEAK_HBM_GBPS:.1%} of 8 TB/s); "
        f"device copy reference {copy_gbps:.0f} GB/s")

    dom = max(stats, key=lambda n: stats[n]["avg_us"])
    extra_fields = {}
    if extra is not None and not args.no_eager:
        eager = extra()
        extra_fields["eager_decode"] = {"avg_us": eager, "rotated_decode_plus_unrotate_us":
                                        stats["decode"]["avg_us"] + stats["unrotate"]["avg_us"]}
        log(f"eager decode (inverse transform of every token): {eager:.1f} us; rotated decode "
            f"{stats['decode']['avg_us']:.1f} us + un-rotation {stats['unrotate']['avg_us']:.1f} us")
    cpu = None if args.no_cpu_baseline else cpu_fn()
    # the committed kernel trace of this workload on the same sources, beside
    # the live event figures
    tr = committed_trace(args.workload, kernel_kind_of(dom))
    trace_fields = None if tr is None else {
        "source": f"profiles/{args.workload}_kernel_trace.json", "avg_us": tr["avg_us"],
        "frac": stats[dom]["bytes"] / (tr["avg_us"] * 1e-6) / 1e9 / PEAK_HBM_GBPS,
        "p10_frac": None if tr["p90_us"] is None else stats[dom]["bytes"] / (tr["p90_us"] * 1e-6) / 1e9 / PEAK_HBM_GBPS,
        "p90_frac": None if tr["p10_us"] is None else stats[dom]["bytes"] / (tr["p10_us"] * 1e-6) / 1e9 / PEAK_HBM_GBPS}

    out = {
        "metric": METRIC[args.workload],
        "value": kv_tokens / (steps * ms_per_step * 1e-3),
        "unit": "sample-iterations/s" if args.workload == "lloyd_fit" else "KV tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"batch_merge": "u8", "lloyd_fit": "f64"}.get(args.workload, "f32"),
        "data": "synthetic",
        "config": config,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": stats[dom]["GBps"], "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": stats[dom]["GBps"] / PEAK_HBM_GBPS,
                     "traffic": measured_traffic(args.workload, kernel_kind_of(dom)),
                     "algorithmic_bytes": stats[dom]["bytes"], "avg_kernel_us": stats[dom]["avg_us"],
                     "committed_trace": trace_fields},
        "kernels": {**stats, "step": {"GBps": step_gbps, "frac": step_gbps / PEAK_HBM_GBPS},
                    "device_copy_reference_GBps": copy_gbps},
        "graph_replay": None if graph_ms_per_step is None else {
            "ms_per_step": graph_ms_per_step, "value": kv_tokens / (steps * graph_ms_per_step * 1e-3)},
        "pipelined": None if pipe_ms_per_step is None else {
            "streams": 2, "ms_per_step": pipe_ms_per_step, "value": kv_tokens / (steps * pipe_ms_per_step * 1e-3)},
        "cpu_baseline": cpu,
        **extra_fields,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
