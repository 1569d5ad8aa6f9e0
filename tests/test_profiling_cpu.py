"""Host logic of the rocprofv3 summaries: counter scaling by the copy
calibration and the kernel-time table, on small hand-made CSV files."""

import csv
import json

from dense_pretraining_amd import profiling

COLS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write_counters(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=COLS)
        w.writeheader()
        for i, (name, counter, value) in enumerate(rows, 1):
            w.writerow(dict(Correlation_Id=i, Dispatch_Id=i, Kernel_Name=name, Counter_Name=counter,
                            Counter_Value=value))


def test_traffic_scaled_by_copy(tmp_path):
    k = "void nc::gemm_dma_kernel<1, 1, nc::EpiF32>(nc::GemmShape, nc::EpiF32)"
    # the copy of 1 MiB reads as 512 KiB fetched (factor 2) and 1024 KiB written (factor 1)
    _write_counters(tmp_path / "f.csv", [(k, "FETCH_SIZE", 100.0), ("__amd_rocclr_copyBuffer", "FETCH_SIZE", 2.0),
                                         (k, "FETCH_SIZE", 300.0), ("__amd_rocclr_copyBuffer", "FETCH_SIZE", 512.0)])
    _write_counters(tmp_path / "w.csv", [(k, "WRITE_SIZE", 10.0), ("__amd_rocclr_copyBuffer", "WRITE_SIZE", 1024.0),
                                         (k, "WRITE_SIZE", 30.0)])
    out = tmp_path / "t.json"
    profiling.main(["traffic", "--fetch", str(tmp_path / "f.csv"), "--write", str(tmp_path / "w.csv"),
                    "--kernel", r"gemm_dma_kernel<1, 1, nc::EpiF32>", "--scope", "gemm_dw_bf16", "--copy-mib", "1",
                    "--out", str(out)])
    rec = json.loads(out.read_text())
    assert rec["fetch"]["factor"] == 2.0 and rec["write"]["factor"] == 1.0
    # mean fetch 200 KiB x 2 + mean write 20 KiB x 1
    assert rec["traffic_bytes_per_launch"] == (200 * 2 + 20) * 1024
    # the record is tied to the GEMM's own source files, not to the rest of the library
    assert rec["sources"] == ["gemm.h", "gemm.hip", "common.h"]
    assert rec["source_sha256"] == profiling.source_hash(rec["sources"])
    assert rec["source_sha256"] != profiling.source_hash(["gemm.h", "gemm.hip", "common.h", "attn.hip"])


def test_stats_table(tmp_path):
    p = tmp_path / "s.csv"
    with open(p, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Name", "Calls", "TotalDurationNs"])
        w.writeheader()
        w.writerow(dict(Name="a_kernel", Calls=4, TotalDurationNs=4_000_000))
        w.writerow(dict(Name="b_kernel", Calls=2, TotalDurationNs=1_000_000))
    t = profiling.stats_table(str(p), steps=2, kernel="a_k", bench_ms=1.02)
    assert "| `a_kernel` | 4 | 4.00 | 1000.0 | 80.00 |" in t
    assert "2.5 ms/step" in t
    assert "average 1.0000 ms" in t and "+2.0 %" in t
