#!/usr/bin/env python3
"""Throughput of the TurboQuant KV-cache codec on one MI355X.

A step is one pass of the whole hot path over the prefill workload (batch 1,
8 KV heads, head_dim 128, 32768 tokens, bf16 K/V with per-channel scales;
values 4-bit Lloyd-Max, keys 4-bit affine): encode K and V of every token
into the packed planes, then decode every token back to bf16 K and V. The
inputs are resident in HBM before timing starts. Steps rotate over several
independent buffer sets so that the working set exceeds the 256 MB
last-level cache and every step streams from HBM.

Prints one JSON line: value = KV tokens per second for encode + decode
(one KV token = one position with K and V of all its heads), plus the
roofline of the dominant kernel (algorithmic bytes / average kernel
duration from HIP events on the launch stream) and the CPU oracle timed on
the host as a baseline. Diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KV tokens/sec encode+decode (d=128, 4-bit) and achieved HBM GB/s vs peak"
PEAK_HBM_GBPS = 8000.0
TRAFFIC = os.path.join(ROOT, "profiles", "prefill_hbm_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(w):
    """Bytes the method itself must move per launch (tables excluded)."""
    d, R, G = w.head_dim, w.rows, w.head_dim // 32
    in_b = 4 if w.dtype == "f32" else 2
    planes = d * w.v_bits // 8 + 2 * G + d * w.k_bits // 8 + 4 * G
    enc = R * (2 * d * in_b + planes)
    dec = R * (planes + 2 * d * 2)
    return enc, dec


def source_digest():
    from kv_cache_quantization_tq_amd.build import source_digest as digest
    return digest()


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed counter runs, if they were
    taken on the current kernel source."""
    try:
        with open(TRAFFIC) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_digest():
        return None
    k = t.get("kernels", {}).get(kernel)
    if not k:
        return None
    return int(k["fetch_bytes"] + k["write_bytes"])


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


def cpu_baseline(w, k, v):
    import oracle as O
    from kv_cache_quantization_tq_amd import workloads as W

    kn, vn = W.to_oracle(k), W.to_oracle(v)
    t0 = time.perf_counter()
    planes = O.encode_kv(kn, vn, head_dim=w.head_dim, k_bits=w.k_bits, v_bits=w.v_bits, k_signed=w.k_signed)
    t1 = time.perf_counter()
    O.decode_kv(planes, rows=w.rows, head_dim=w.head_dim, k_bits=w.k_bits, v_bits=w.v_bits, k_signed=w.k_signed)
    t2 = time.perf_counter()
    log(f"cpu oracle: encode {t1 - t0:.2f} s, decode {t2 - t1:.2f} s for {w.rows} rows")
    return {"value": w.kv_tokens / (t2 - t0), "unit": "KV tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"whole workload, one pass: encode + decode of {w.rows} rows "
                      f"({w.kv_tokens} tokens x {w.heads} heads), single thread"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sets", type=int, default=0, help="buffer sets to rotate (0: enough for >= 1.5 GiB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    w = W.WORKLOADS["prefill"]
    enc_bytes, dec_bytes = algorithmic_bytes(w)
    k0, v0 = W.make_kv(w, dev)
    per_set = 2 * k0.numel() * k0.element_size() * 2 + enc_bytes - 2 * k0.numel() * k0.element_size()
    nsets = args.sets or max(2, math.ceil(1.5 * 2 ** 30 / per_set))
    sets = []
    for s in range(nsets):
        k = k0 if s == 0 else k0.clone()
        v = v0 if s == 0 else v0.clone()
        planes = tq.empty_planes(w.rows, w.head_dim, w.k_bits, w.v_bits, dev)
        ko = torch.empty_like(k)
        vo = torch.empty_like(v)
        sets.append((k, v, planes, ko, vo))
    torch.cuda.synchronize()
    log(f"workload prefill: {w.rows} rows, {nsets} buffer sets of {per_set / 2**20:.0f} MiB")

    def step(i, ev=None):
        k, v, planes, ko, vo = sets[i % nsets]
        if ev is not None:
            ev[0].record()
        tq.encode_kv(k, v, v_bits=w.v_bits, k_bits=w.k_bits, k_signed=w.k_signed, out=planes)
        if ev is not None:
            ev[1].record()
        tq.decode_kv(planes, tokens=w.kv_tokens, heads=w.heads, head_dim=w.head_dim, v_bits=w.v_bits,
                     k_bits=w.k_bits, k_signed=w.k_signed, k_out=ko, v_out=vo)
        if ev is not None:
            ev[2].record()

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * 2 ** 20 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {args.copy_calibration_mib} MiB read + {args.copy_calibration_mib} MiB written")
        del src, dst

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # whole-step timing
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(i)
    t_end.record()
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps

    # per-kernel durations (events on the stream the kernels are launched on)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    enc_ms = sorted(e[0].elapsed_time(e[1]) for e in evs)
    dec_ms = sorted(e[1].elapsed_time(e[2]) for e in evs)
    enc_avg = sum(enc_ms) / len(enc_ms)
    dec_avg = sum(dec_ms) / len(dec_ms)
    enc_gbps = enc_bytes / (enc_avg * 1e-3) / 1e9
    dec_gbps = dec_bytes / (dec_avg * 1e-3) / 1e9
    log(f"encode: avg {enc_avg * 1e3:.1f} us  median {enc_ms[len(enc_ms) // 2] * 1e3:.1f} us  "
        f"{enc_gbps:.0f} GB/s ({enc_gbps / PEAK_HBM_GBPS:.1%} of 8 TB/s)")
    log(f"decode: avg {dec_avg * 1e3:.1f} us  median {dec_ms[len(dec_ms) // 2] * 1e3:.1f} us  "
        f"{dec_gbps:.0f} GB/s ({dec_gbps / PEAK_HBM_GBPS:.1%} of 8 TB/s)")
    log(f"step: {ms_per_step * 1e3:.1f} us")

    # context: a plain device-to-device copy of the same size class on this GPU
    copy_gbps = device_copy_gbps(torch, dev)
    step_gbps = (enc_bytes + dec_bytes) / (ms_per_step * 1e-3) / 1e9
    log(f"whole step: {step_gbps:.0f} GB/s ({step_gbps / PEAK_HBM_GBPS:.1%} of 8 TB/s); "
        f"device copy reference {copy_gbps:.0f} GB/s")

    if enc_avg >= dec_avg:
        kern, nbytes, avg, gbps = "encode", enc_bytes, enc_avg, enc_gbps
    else:
        kern, nbytes, avg, gbps = "decode", dec_bytes, dec_avg, dec_gbps

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, k0, v0)

    out = {
        "metric": METRIC,
        "value": w.kv_tokens / (ms_per_step * 1e-3),
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "prefill: batch 1, 8 KV heads, head_dim 128, 32768 tokens, bf16 K/V "
                               "(N(0,1) x per-channel log-uniform [0.1,10] scales); values 4-bit Lloyd-Max, "
                               "keys 4-bit affine; encode all + decode all to bf16",
                   "tokens": w.kv_tokens, "heads": w.heads, "head_dim": w.head_dim, "v_bits": w.v_bits,
                   "k_bits": w.k_bits, "input_dtype": w.dtype, "buffer_sets": nsets},
        "roofline": {"bound": "hbm", "kernel": kern, "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": gbps / PEAK_HBM_GBPS, "traffic": measured_traffic(kern),
                     "algorithmic_bytes": nbytes, "avg_kernel_us": avg * 1e3},
        "kernels": {"encode": {"avg_us": enc_avg * 1e3, "GBps": enc_gbps, "bytes": enc_bytes},
                    "decode": {"avg_us": dec_avg * 1e3, "GBps": dec_gbps, "bytes": dec_bytes},
                    "step": {"GBps": step_gbps, "frac": step_gbps / PEAK_HBM_GBPS},
                    "device_copy_reference_GBps": copy_gbps},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
