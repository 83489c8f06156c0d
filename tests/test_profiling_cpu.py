"""The rocprofv3 summary helpers (host code): percentiles and the
per-kernel trace table, on a small synthetic kernel-trace CSV."""
import csv

from kv_cache_quantization_tq_amd import profiling as P


def test_nearest_rank_percentile():
    assert P.percentile([7.0], 10) == 7.0 and P.percentile([7.0], 90) == 7.0
    d = [float(v) for v in range(1, 11)]
    assert (P.percentile(d, 10), P.percentile(d, 50), P.percentile(d, 90), P.percentile(d, 100)) == (1, 5, 9, 10)
    assert P.percentile(list(reversed(d)), 90) == 9  # order of the sample does not matter


def test_trace_summary_columns(tmp_path):
    path = tmp_path / "trace_kernel_trace.csv"
    durations_us = [10, 20, 30, 40, 50, 60, 70, 80, 90, 100]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 1000
        for us in durations_us:
            w.writerow({"Kernel_Name": "void (anonymous namespace)::decode_kernel<128, 4, true>(args)",
                        "Start_Timestamp": t, "End_Timestamp": t + us * 1000})
            t += 200000
        w.writerow({"Kernel_Name": "some_other_kernel()", "Start_Timestamp": 0, "End_Timestamp": 5000})
    out = P.trace_summary(str(path), {"decode": 5}).splitlines()
    assert out[0].split() == ["kernel", "calls", "avg_us", "med_us", "p10_us", "p90_us", "min_us"]
    row = [ln for ln in out if ln.startswith("decode_kernel")]
    assert len(row) == 1
    assert row[0].split()[-6:] == ["10", "55.00", "55.00", "10.00", "90.00", "10.00"]
    assert not any("some_other_kernel" in ln for ln in out)
    assert out[-1] == "decode: 5 operations, 110.00 us of kernel time per operation"
