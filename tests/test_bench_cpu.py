"""Host logic of bench.py (no GPU): the kernel table, the roofline figure of
the dominant kernel, the traffic lookup, and the refusal of several GPUs."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _summary():
    # two steps of a made-up profile: a GEMM class and a memory-bound class
    return {
        "gemm_dw_bf16": {"launches": 4, "ms": 2.0, "flops": 4.0e12, "bytes": 2.0e9},
        "rmsnorm_bwd_bf16": {"launches": 8, "ms": 0.4, "flops": 0.0, "bytes": 2.4e9},
        "gemm_fwd_fp8": {"launches": 2, "ms": 0.1, "flops": 4.0e11, "bytes": 1.0e8},
    }


def test_kernel_table_per_step_and_sorted():
    t = bench.kernel_table(_summary(), steps=2)
    assert list(t) == ["gemm_dw_bf16", "rmsnorm_bwd_bf16", "gemm_fwd_fp8"]  # by time per step
    r = t["gemm_dw_bf16"]
    assert r["ms_per_step"] == pytest.approx(1.0) and r["launches_per_step"] == pytest.approx(2.0)
    assert r["tflops"] == pytest.approx(4.0e12 / 2.0e-3 / 1e12)
    assert r["flops_per_launch"] == pytest.approx(1.0e12)
    assert t["rmsnorm_bwd_bf16"]["gbps"] == pytest.approx(2.4e9 / 0.4e-3 / 1e9)


def test_roofline_of_a_contraction_uses_its_own_peak():
    name, rl = bench.roofline(bench.kernel_table(_summary(), 2))
    assert name == "gemm_dw_bf16" and rl["bound"] == "mfma" and rl["unit"] == "TFLOP/s"
    assert rl["peak"] == pytest.approx(bench.PEAK_BF16 / 1e12, rel=1e-3)
    assert rl["frac"] == pytest.approx(rl["achieved"] / rl["peak"], rel=1e-3)
    assert rl["avg_launch_ms"] == pytest.approx(0.5)
    fp8 = {"gemm_fwd_fp8": _summary()["gemm_fwd_fp8"]}
    _, rl8 = bench.roofline(bench.kernel_table(fp8, 1))
    assert rl8["peak"] == pytest.approx(bench.PEAK_FP8 / 1e12, rel=1e-3)


def test_roofline_of_a_memory_bound_kernel():
    only = {"rmsnorm_bwd_bf16": _summary()["rmsnorm_bwd_bf16"]}
    _, rl = bench.roofline(bench.kernel_table(only, 2))
    assert rl["bound"] == "hbm" and rl["unit"] == "GB/s"
    assert rl["achieved"] == pytest.approx(6000.0) and rl["frac"] == pytest.approx(6000.0 / 8000.0, rel=1e-3)


def test_traffic_is_none_for_an_unmeasured_kernel():
    assert bench.measured_traffic("no_such_kernel") is None


def test_committed_traffic_record_is_consistent():
    path = os.path.join(ROOT, "profiles", "gemm_dw_bf16_traffic.json")
    rec = json.load(open(path))
    total = rec["fetch"]["bytes_per_launch"] + rec["write"]["bytes_per_launch"]
    assert rec["traffic_bytes_per_launch"] == pytest.approx(total)
    # each counter scaled by what it reads for a plain copy of known size
    for k in ("fetch", "write"):
        assert rec[k]["bytes_per_launch"] == pytest.approx(rec[k]["kib_per_launch"] * 1024 * rec[k]["factor"])


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})])
def test_several_gpus_refused_before_any_gpu_work(args, env):
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       env={**os.environ, **env}, timeout=120)
    assert p.returncode == 2
    assert "one GPU only" in p.stderr and p.stdout == ""
