"""Summaries of rocprofv3 output for the codec kernels.

    python -m kv_cache_quantization_tq_amd.profiling trace <kernel_trace.csv> [--stats <kernel_stats.csv>]
    python -m kv_cache_quantization_tq_amd.profiling traffic <fetch.csv> <write.csv> \
        --copy-mib 512 [--json out.json] [--ops merge=N]

``trace`` prints per-kernel dispatch counts and average / median / 10th
and 90th percentile / min durations from a ``--kernel-trace`` CSV, and with ``--stats`` the codec
kernels' rows of rocprofv3's own ``--stats`` table; ``--json`` also writes the per-kind figures
with the SHA-256 of each kind's sources (bench.py reports them beside its own timing when the
sources still match). ``counters`` summarises one ``--pmc`` pass of the SQ counters
(instructions, busy cycles, wave cycles) per kernel kind with the derived
clock, VALU busy fraction and occupancy. ``traffic`` turns the FETCH_SIZE and
WRITE_SIZE counters (KiB per dispatch) of two ``--pmc`` runs of
``bench.py --copy-calibration-mib N`` into HBM bytes per launch: each
counter is scaled by the factor that maps the same counter, read on the
plain device copy of N MiB in the same run, to its known N MiB. Each
kernel's entry records the SHA-256 of the sources it is built from, so a
reader can tell whether the figures still describe the current kernel.
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import re
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


KINDS = ("encode", "decode", "unrotate", "merge", "fit", "attention")


def kernel_kind(name: str) -> str:
    if "encode_kernel" in name:
        return "encode"
    if "decode_kernel" in name:
        return "decode"
    if "unrotate_kernel" in name:
        return "unrotate"
    if "segment_copy_kernel" in name:
        return "merge"
    if "fit_" in name and "_kernel" in name:
        return "fit"
    if "attn_" in name and "_kernel" in name:
        return "attention"
    if "copyBuffer" in name:
        return "copy"
    return "other"


def short_name(name: str) -> str:
    m = re.search(r"(\w+_kernel(<[^>]*>)?)", name)
    return m.group(1) if m else name[:80]


def read_trace(path: str):
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
            out.setdefault(short_name(name), []).append(dur)
    return out


def percentile(d, q: float) -> float:
    """Nearest-rank q-th percentile (0 < q <= 100) of a non-empty sample."""
    s = sorted(d)
    k = -(-q * len(s) // 100)  # ceil(q n / 100)
    return s[min(len(s), max(1, int(k))) - 1]


def trace_summary(path: str, ops: dict | None = None) -> str:
    rows = []
    tr = read_trace(path)
    for name, d in tr.items():
        if kernel_kind(name) in KINDS:
            rows.append((name, len(d), sum(d) / len(d), statistics.median(d), percentile(d, 10), percentile(d, 90),
                         min(d)))
    lines = [f"{'kernel':70s} {'calls':>5s} {'avg_us':>8s} {'med_us':>8s} {'p10_us':>8s} {'p90_us':>8s} "
             f"{'min_us':>8s}"]
    for name, n, avg, med, p10, p90, mn in sorted(rows):
        lines.append(f"{name[:70]:70s} {n:5d} {avg:8.2f} {med:8.2f} {p10:8.2f} {p90:8.2f} {mn:8.2f}")
    for kind, n in (ops or {}).items():
        tot = sum(sum(d) for name, d in tr.items() if kernel_kind(name) == kind)
        lines.append(f"{kind}: {n} operations, {tot / n:.2f} us of kernel time per operation")
    return "\n".join(lines)


def trace_kinds(path: str, ops: dict | None = None) -> dict:
    """Per kernel kind: dispatches and average / median / 10th and 90th
    percentile duration (us) over the trace, with the SHA-256 of that kind's
    sources; with ops[kind] = N, also the kernel time per operation (one
    operation being several launches)."""
    from kv_cache_quantization_tq_amd.build import source_digest
    tr = read_trace(path)
    res = {}
    for kind in KINDS:
        d = [v for name, vs in tr.items() if kernel_kind(name) == kind for v in vs]
        if not d:
            continue
        res[kind] = {"dispatches": len(d), "avg_us": sum(d) / len(d), "median_us": statistics.median(d),
                     "p10_us": percentile(d, 10), "p90_us": percentile(d, 90), "min_us": min(d),
                     "source_sha256": source_digest(kind)}
        if ops and kind in ops:
            res[kind]["operations"] = ops[kind]
            res[kind]["per_operation_us"] = sum(d) / ops[kind]
    return res


def stats_summary(path: str) -> str:
    lines = [f"{'kernel (rocprofv3 --stats)':70s} {'calls':>5s} {'avg_us':>8s} {'min_us':>8s} {'max_us':>8s}"]
    with open(path) as f:
        for r in csv.DictReader(f):
            name = short_name(r["Name"])
            if kernel_kind(name) in KINDS:
                lines.append(f"{name[:70]:70s} {int(r['Calls']):5d} {float(r['AverageNs']) * 1e-3:8.2f} "
                             f"{float(r['MinNs']) * 1e-3:8.2f} {float(r['MaxNs']) * 1e-3:8.2f}")
    return "\n".join(lines)


def read_counter(path: str, counter: str):
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def traffic(fetch_csv: str, write_csv: str, copy_mib: int, ops: dict | None = None) -> dict:
    fetch = read_counter(fetch_csv, "FETCH_SIZE")
    write = read_counter(write_csv, "WRITE_SIZE")
    copy_kib = copy_mib * 1024.0

    def copy_reading(d):
        vals = [v for name, vs in d.items() if "copyBuffer" in name for v in vs]
        # the calibration copy is the largest blit of the run
        return max(vals)

    f_scale = copy_kib / copy_reading(fetch)
    w_scale = copy_kib / copy_reading(write)
    from kv_cache_quantization_tq_amd.build import source_digest
    res = {"copy_mib": copy_mib, "fetch_scale": f_scale, "write_scale": w_scale, "kernels": {}}
    for kind in ("encode", "decode", "merge", "fit", "attention"):
        fv = [v for n, vs in fetch.items() if kernel_kind(n) == kind for v in vs]
        wv = [v for n, vs in write.items() if kernel_kind(n) == kind for v in vs]
        if fv and wv and ops and kind in ops:
            # one operation is several launches: total over the run / operations
            n = ops[kind]
            res["kernels"][kind] = {
                "source_sha256": source_digest(kind), "operations": n, "dispatches": len(fv),
                "fetch_kib_raw": sum(fv) / n, "write_kib_raw": sum(wv) / n,
                "fetch_bytes": int(sum(fv) / n * f_scale * 1024),
                "write_bytes": int(sum(wv) / n * w_scale * 1024),
            }
        elif fv and wv:
            res["kernels"][kind] = {
                "source_sha256": source_digest(kind),
                "fetch_kib_raw": statistics.median(fv), "write_kib_raw": statistics.median(wv),
                "fetch_bytes": int(statistics.median(fv) * f_scale * 1024),
                "write_bytes": int(statistics.median(wv) * w_scale * 1024),
            }
    return res


SQ_COUNTERS = ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES",
               "SQ_INSTS_LDS", "SQ_INSTS_MFMA", "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE")

# MI355X: 256 compute units of 4 SIMDs in 32 shader engines; SQ cycle
# counters are summed over the shader engines, instruction counters over all
# wavefronts, and SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES count 4-cycle units.
N_SIMD, N_SE = 1024, 32


def counter_summary(path: str) -> dict:
    """Per kernel, the median per dispatch of each SQ counter in a
    --pmc CSV, and derived figures: shader clock = SQ_BUSY_CYCLES / 32 /
    duration; VALU busy = 4 * SQ_ACTIVE_INST_VALU / (1024 SIMDs * busy
    cycles per engine); mean wavefronts per SIMD = 4 * SQ_WAVE_CYCLES /
    (1024 * busy cycles per engine); VALU instructions per wavefront."""
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            kind = kernel_kind(r["Kernel_Name"])
            if kind not in KINDS:
                continue
            key = (short_name(r["Kernel_Name"]), r["Dispatch_Id"])
            d = per.setdefault(key, {"dur_ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"]), "kind": kind})
            d[r["Counter_Name"]] = float(r["Counter_Value"])
    from kv_cache_quantization_tq_amd.build import source_digest
    out = {}
    for name in sorted({k for k, _ in per}):
        ds = [d for (k, _), d in per.items() if k == name]
        kind = ds[0]["kind"]
        med = {c: statistics.median([d[c] for d in ds if c in d]) for c in ds[0] if c != "kind"}
        res = {"kind": kind, "dispatches": len(ds), "source_sha256": source_digest(kind), "median": med}
        if {"SQ_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES", "SQ_INSTS_VALU", "SQ_WAVES"} <= set(med):
            cyc = med["SQ_BUSY_CYCLES"] / N_SE
            res["derived"] = {
                "duration_us": med["dur_ns"] * 1e-3,
                "shader_clock_GHz": cyc / med["dur_ns"],
                "valu_busy": 4 * med["SQ_ACTIVE_INST_VALU"] / (N_SIMD * cyc),
                "mean_waves_per_simd": 4 * med["SQ_WAVE_CYCLES"] / (N_SIMD * cyc),
                "valu_insts_per_wave": med["SQ_INSTS_VALU"] / med["SQ_WAVES"],
            }
        out[name] = res
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("csv")
    t.add_argument("--stats")
    t.add_argument("--ops", action="append", default=[], help="KIND=N: also report kernel time per operation")
    t.add_argument("--json", help="also write per-kind figures (with source digests) to this file")
    q = sub.add_parser("counters")
    q.add_argument("csv")
    q.add_argument("--json")
    c = sub.add_parser("traffic")
    c.add_argument("fetch_csv")
    c.add_argument("write_csv")
    c.add_argument("--copy-mib", type=int, required=True)
    c.add_argument("--json")
    c.add_argument("--ops", action="append", default=[],
                   help="KIND=N: that kind's launches form N operations; report bytes per operation")
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        ops = {k: int(v) for k, v in (o.split("=") for o in a.ops)}
        print(trace_summary(a.csv, ops))
        if a.json:
            with open(a.json, "w") as f:
                f.write(json.dumps(trace_kinds(a.csv, ops), indent=1) + "\n")
        if a.stats:
            print()
            print(stats_summary(a.stats))
    elif a.cmd == "counters":
        res = counter_summary(a.csv)
        txt = json.dumps(res, indent=1)
        if a.json:
            with open(a.json, "w") as f:
                f.write(txt + "\n")
        print(txt)
    else:
        ops = {k: int(v) for k, v in (o.split("=") for o in a.ops)}
        res = traffic(a.fetch_csv, a.write_csv, a.copy_mib, ops)
        txt = json.dumps(res, indent=1)
        if a.json:
            with open(a.json, "w") as f:
                f.write(txt + "\n")
        print(txt)


if __name__ == "__main__":
    sys.exit(main())
