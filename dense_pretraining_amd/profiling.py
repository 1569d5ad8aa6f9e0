"""Summaries of rocprofv3 output for the kernels of the training step.

Two jobs, both reading the CSV files rocprofv3 writes with
``--output-format csv``:

* ``stats``: the ``*_kernel_stats.csv`` of a ``--kernel-trace --stats`` run
  as a markdown table (calls, total and average time per kernel), with the
  average launch time of one kernel checked against what bench.py measured
  with HIP events in the same run.
* ``classes``: per kernel class of the step (the weight-gradient GEMM, the
  attention backward passes, the norms, ...), the launch time from a
  ``--kernel-trace`` run and the mean of every counter of one or more
  ``--pmc`` runs of the same command, with the figures derived from them:
  matrix-core busy share, shader clock, L2 hit rate, HBM bytes per launch
  (copy-calibrated as below) and the HBM rate they imply.
* ``traffic``: HBM bytes per launch of one kernel from two ``--pmc`` runs
  (``FETCH_SIZE``, then ``WRITE_SIZE``, both in KiB per dispatch). Each
  counter is first scaled by what it reads for a plain device copy of known
  size in the same process (bench.py ``--copy-mib``), so that the figure is in
  the copy's bytes. The result goes to a JSON file that records a hash of the
  files the kernel is built from; bench.py reports the figure only while that
  hash matches.

Usage (paths are those rocprofv3 wrote):

    python -m dense_pretraining_amd.profiling stats STATS_CSV --steps N \
        --bench-log LOG --kernel REGEX --title TEXT --command TEXT > summary.md
    python -m dense_pretraining_amd.profiling traffic --fetch CSV --write CSV \
        --kernel REGEX --scope NAME --copy-mib MIB --command TEXT --out profiles/x.json
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys

PKG = os.path.dirname(os.path.abspath(__file__))


def source_hash(names=None) -> str:
    """sha256 over the named files of csrc/ (default: every HIP source and
    header of the library), in name order."""
    h = hashlib.sha256()
    if names:
        files = sorted(os.path.join(PKG, "csrc", n) for n in names)
    else:
        files = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")) + glob.glob(os.path.join(PKG, "csrc", "*.h")))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _rows(path):
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def _col(row, *names):
    for n in names:
        if n in row:
            return row[n]
    raise KeyError(f"none of {names} in {sorted(row)}")


def stats_table(path, steps, kernel=None, bench_ms=None, top=25):
    rows = _rows(path)
    out = []
    total = 0.0
    recs = []
    for r in rows:
        name = _col(r, "Name", "KernelName", "Kernel_Name")
        calls = int(float(_col(r, "Calls")))
        tot_ns = float(_col(r, "TotalDurationNs", "Total_Duration_Ns"))
        recs.append((name, calls, tot_ns))
        total += tot_ns
    recs.sort(key=lambda t: -t[2])
    out.append("| kernel | calls | total ms | avg us | % |")
    out.append("|---|---:|---:|---:|---:|")
    for name, calls, tot in recs[:top]:
        shown = name if len(name) <= 160 else name[:157] + "..."
        out.append(f"| `{shown}` | {calls} | {tot / 1e6:.2f} | {tot / calls / 1e3:.1f} | {100 * tot / total:.2f} |")
    out.append("")
    out.append(f"Sum of all kernels: {total / 1e6:.1f} ms over {steps} steps = {total / 1e6 / steps:.1f} ms/step.")
    if kernel:
        rx = re.compile(kernel)
        hit = [(n, c, t) for n, c, t in recs if rx.search(n)]
        if hit:
            calls = sum(c for _, c, _ in hit)
            tot = sum(t for _, _, t in hit)
            line = (f"Dominant kernel (`{kernel}`): {calls} launches, average {tot / calls / 1e6:.4f} ms "
                    f"per launch under rocprofv3")
            if bench_ms is not None:
                line += (f"; HIP events in bench.py, same run: {bench_ms:.4f} ms "
                         f"({100 * (bench_ms / (tot / calls / 1e6) - 1):+.1f} %)")
            out.append("")
            out.append(line + ".")
    return "\n".join(out)


def counter_per_dispatch(path, counter):
    """{dispatch id: (kernel name, value)} for one counter."""
    res = {}
    for r in _rows(path):
        if _col(r, "Counter_Name", "CounterName") != counter:
            continue
        did = int(float(_col(r, "Dispatch_Id", "DispatchId")))
        name = _col(r, "Kernel_Name", "KernelName")
        val = float(_col(r, "Counter_Value", "CounterValue"))
        prev = res.get(did)
        res[did] = (name, val + (prev[1] if prev else 0.0))
    return res


def scaled_counter(path, counter, kernel_rx, copy_bytes):
    """Mean per-launch value of `counter` (KiB) for kernels matching
    kernel_rx, in bytes, scaled by copy_bytes / (counter of the copy)."""
    disp = counter_per_dispatch(path, counter)
    rx = re.compile(kernel_rx)
    vals = [v for n, v in disp.values() if rx.search(n)]
    if not vals:
        raise SystemExit(f"no dispatch of {kernel_rx} with {counter} in {path}")
    # the copy of bench.py --copy-mib: by far the largest copy kernel the
    # process dispatches (the others move a few bytes)
    copies = [v for n, v in disp.values() if "copy" in n.lower() and "_ZN2nc" not in n and "nc::" not in n]
    if not copies:
        raise SystemExit(f"no copy kernel dispatch in {path} (run bench.py with --copy-mib)")
    copy_kib = max(copies)
    factor = (copy_bytes / 1024.0) / copy_kib
    return dict(kib_per_launch=sum(vals) / len(vals), launches=len(vals), copy_kib=copy_kib, factor=factor,
                bytes_per_launch=sum(vals) / len(vals) * 1024.0 * factor)


# Kernel classes of the step, matched against the symbol rocprofv3 reports
# (mangled, or demangled with some template arguments lost); first match wins.
CLASSES = [
    ("gemm_dw (weight grads, split K)", r"EpiF32"),
    ("gemm_dx_drelusq (W2 input grad + dReLU^2)", r"EpiDReluSq"),
    ("gemm_lmhead_softcap", r"EpiSoftcap"),
    ("gemm_lmhead_dx (unembedding input grad, row factors)", r"EpiRowScale"),
    ("gemm_dx (input grads)", r"ILi0ELi1ENS_8EpiStore|<0, 1, nc::EpiStore"),
    ("gemm_fwd +residual (O, W2)", r"ILi0ELi0ENS_8EpiStoreIDF16bLb0ELb0ELb1E"),
    ("gemm_fwd (QKV)", r"ILi0ELi0ENS_8EpiStoreIDF16bLb0ELb0ELb0E"),
    ("gemm_fwd_relusq (W1 + ReLU^2)", r"ILi0ELi0ENS_8EpiStoreIDF16bLb1E|<0, 0, nc::EpiStore<bool _Accum, bool, E, false"),
    ("attn_bwd_dkdv", r"attn_bwd_dkdv_kernel"),
    ("attn_bwd_dq", r"attn_bwd_dq_kernel"),
    ("attn_fwd", r"attn_fwd_kernel"),
    ("rmsnorm_bwd", r"rmsnorm_bwd_kernel"),
    ("embed_gather_rmsnorm", r"rmsnorm_fwd_kernelIDF16bLb1E|rmsnorm_fwd_kernel<[^>]*true"),
    ("rmsnorm_fwd", r"rmsnorm_fwd_kernel"),
    ("qknorm_rope_bwd", r"qknorm_rope_bwd_kernel"),
    ("qknorm_rope_fwd", r"qknorm_rope_fwd_kernel"),
    ("xent_grad_prep", r"xent_grad_prep_kernel"),
    ("xent_loss", r"xent_rows_kernel|xent_final_kernel"),
    ("splitk_reduce", r"splitk_reduce_kernel"),
    ("embed_bwd (sort, window sums with the norm backward, fixup)", r"eb_\w+_kernel"),
    ("fills", r"fill_u32_kernel|fill_f32_kernel"),
]
NUM_CUS, SIMDS_PER_CU, XCDS = 256, 4, 8


def classify(name):
    for cls, rx in CLASSES:
        if re.search(rx, name):
            return cls
    return None


def trace_durations(path):
    """{class: [durations in ns]} from a --kernel-trace CSV."""
    out = {}
    for r in _rows(path):
        cls = classify(_col(r, "Kernel_Name", "KernelName"))
        if cls is None:
            continue
        dur = float(_col(r, "End_Timestamp", "EndTimestamp")) - float(_col(r, "Start_Timestamp", "StartTimestamp"))
        out.setdefault(cls, []).append(dur)
    return out


def pmc_means(paths):
    """{class: {counter: mean value per dispatch}} over the --pmc CSVs."""
    acc = {}
    for path in paths:
        per = {}
        for r in _rows(path):
            cls = classify(_col(r, "Kernel_Name", "KernelName"))
            if cls is None:
                continue
            did = int(float(_col(r, "Dispatch_Id", "DispatchId")))
            ctr = _col(r, "Counter_Name", "CounterName")
            per.setdefault((cls, ctr), {}).setdefault(did, 0.0)
            per[(cls, ctr)][did] += float(_col(r, "Counter_Value", "CounterValue"))
        for (cls, ctr), d in per.items():
            acc.setdefault(cls, {})[ctr] = sum(d.values()) / len(d)
    return acc


def copy_factor(paths, counter, copy_bytes):
    """copy_bytes / (KiB the counter reads for the largest plain copy kernel) * 1024."""
    for path in paths:
        disp = counter_per_dispatch(path, counter)
        copies = [v for n, v in disp.values() if "copy" in n.lower() and "_ZN2nc" not in n and "nc::" not in n]
        if copies:
            return copy_bytes / (max(copies) * 1024.0)
    return None


def classes_table(trace, pmcs, steps, copy_bytes):
    dur = trace_durations(trace)
    cnt = pmc_means(pmcs)
    ff = copy_factor(pmcs, "FETCH_SIZE", copy_bytes) if copy_bytes else None
    fw = copy_factor(pmcs, "WRITE_SIZE", copy_bytes) if copy_bytes else None
    rows = ["| kernel class | launches/step | ms/launch | ms/step | MFMA busy | clock GHz | L2 hit | "
            "HBM MB/launch (read + write) | HBM TB/s | waves waiting |",
            "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    order = sorted(dur, key=lambda c: -sum(dur[c]))
    for cls in order:
        d = dur[cls]
        ms = sum(d) / len(d) / 1e6
        c = cnt.get(cls, {})
        gui = c.get("GRBM_GUI_ACTIVE")
        clock = mfma = hit = hbm = rate = wait = None
        if gui:
            clock = gui / XCDS / (ms * 1e6)  # cycles per ns
            if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                mfma = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui / XCDS * NUM_CUS * SIMDS_PER_CU)
        if c.get("TCC_HIT_sum") is not None and c.get("TCC_MISS_sum") is not None:
            tot = c["TCC_HIT_sum"] + c["TCC_MISS_sum"]
            hit = c["TCC_HIT_sum"] / tot if tot else None
        if ff and fw and "FETCH_SIZE" in c and "WRITE_SIZE" in c:
            rd, wr = c["FETCH_SIZE"] * 1024 * ff, c["WRITE_SIZE"] * 1024 * fw
            hbm = (rd / 1e6, wr / 1e6)
            rate = (rd + wr) / (ms * 1e-3) / 1e12
        if c.get("SQ_WAVE_CYCLES") and c.get("SQ_WAIT_ANY") is not None:
            wait = c["SQ_WAIT_ANY"] / c["SQ_WAVE_CYCLES"]
        f = lambda v, fmt: "" if v is None else fmt.format(v)
        rows.append(f"| {cls} | {len(d) / steps:.0f} | {ms:.4f} | {sum(d) / 1e6 / steps:.2f} | {f(mfma, '{:.1%}')} | "
                    f"{f(clock, '{:.2f}')} | {f(hit, '{:.1%}')} | "
                    f"{'' if hbm is None else f'{hbm[0]:.0f} + {hbm[1]:.0f}'} | {f(rate, '{:.2f}')} | {f(wait, '{:.1%}')} |")
    return "\n".join(rows)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--steps", type=int, required=True)
    s.add_argument("--kernel")
    s.add_argument("--bench-log")
    s.add_argument("--title", default="Kernel time")
    s.add_argument("--command", default="")
    c = sub.add_parser("classes")
    c.add_argument("--trace", required=True, help="kernel trace CSV of the command")
    c.add_argument("--pmc", nargs="+", required=True, help="counter collection CSVs of the same command")
    c.add_argument("--steps", type=int, required=True, help="training steps the command ran")
    c.add_argument("--copy-mib", type=float, default=0.0)
    c.add_argument("--title", default="Counters per kernel class")
    c.add_argument("--command", default="")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True, help="regex of the kernel symbol")
    t.add_argument("--scope", required=True, help="bench.py kernel name the figure belongs to")
    t.add_argument("--copy-mib", type=float, required=True)
    t.add_argument("--sources", default="gemm.h,gemm.hip,common.h",
                   help="comma-separated csrc/ files the kernel is built from; the figure is stale once they change")
    t.add_argument("--command", default="")
    t.add_argument("--out", required=True)
    a = ap.parse_args(argv)

    if a.cmd == "stats":
        bench_ms = None
        if a.bench_log:
            for line in open(a.bench_log):
                if line.startswith("{"):
                    rl = json.loads(line).get("roofline") or {}
                    bench_ms = rl.get("avg_launch_ms")
        print(f"# {a.title}\n")
        if a.command:
            print("Command (from /tmp on the MI355X, repository at $GRAFT_REPO_ROOT):\n\n```\n" + a.command + "\n```\n")
        print(stats_table(a.csv, a.steps, a.kernel, bench_ms))
        return 0

    if a.cmd == "classes":
        print(f"# {a.title}\n")
        if a.command:
            print("Commands (from /tmp on the MI355X, repository at $GRAFT_REPO_ROOT):\n\n```\n" + a.command + "\n```\n")
        print(classes_table(a.trace, a.pmc, a.steps, a.copy_mib * 1024 * 1024))
        return 0

    copy_bytes = a.copy_mib * 1024 * 1024
    f = scaled_counter(a.fetch, "FETCH_SIZE", a.kernel, copy_bytes)
    w = scaled_counter(a.write, "WRITE_SIZE", a.kernel, copy_bytes)
    res = dict(scope=a.scope, kernel_regex=a.kernel, traffic_bytes_per_launch=f["bytes_per_launch"] + w["bytes_per_launch"],
               fetch=f, write=w, copy_bytes=copy_bytes, sources=a.sources.split(","),
               source_sha256=source_hash(a.sources.split(",")), command=a.command)
    with open(a.out, "w") as fh:
        json.dump(res, fh, indent=1)
    print(json.dumps(res, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
