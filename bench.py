#!/usr/bin/env python3
"""Training-step benchmark on one MI355X.

One step = nc_model_loss_and_grad: embedding + norm, all blocks, final norm,
unembedding with logit softcap, cross-entropy, and the full backward pass,
over one batch of seeded synthetic tokens resident in HBM.

Default workload: the depth-20 model (d_model 1280, 10 query heads of 128,
one KV head, MLP 5120, vocab 65536) at 32 rows x 2048 tokens, bf16 storage
with fp32 accumulation -- one GPU's share of the pretraining step the
imeisheng.com page ("预训练") describes.

Prints one JSON line: tokens/s, MFU, the dominant kernel's roofline (its
launches timed with HIP events inside the timed region, the only events
there), the per-kernel table (from untimed steps with every launch timed)
and the fp64 CPU oracle's throughput on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from dense_pretraining_amd import config as C  # noqa: E402
from dense_pretraining_amd import synth  # noqa: E402

METRIC = "train tokens/sec (fwd+bwd) + MFU, depth-20 B=32 T=2048 bf16, 1 MI355X"
INFER = dict(cfg=C.DEPTH20.with_(batch=64, seq_len=1024 + 256), prompt=1024, steps=256,
             desc="depth-20 decoder, 64 sequences: 1024-token prefill then 256 greedy decode steps, bf16, "
                  "one-head K/V cache")
WORKLOADS = {
    "depth20": (C.DEPTH20, "depth-20 decoder (d 1280, 10x128 heads, 1 KV head, MLP 5120, vocab 65536), "
                           "32 x 2048 tokens, bf16, forward+backward"),
    "depth30": (C.DEPTH30, "depth-30 decoder (d 1920, 15x128 heads, 1 KV head, MLP 7680, vocab 65536), "
                           "16 x 2048 tokens, bf16, forward+backward"),
    "depth20_fp8": (C.DEPTH20.with_(dtype="bf16_fp8"),
                    "depth-20 decoder as above, 32 x 2048 tokens, bf16 storage with the four forward block "
                    "products in FP8 E4M3 (per-tensor scales), forward+backward"),
}
PEAK_BF16 = C.MI355X_BF16_DENSE_PEAK
PEAK_FP8 = C.MI355X_FP8_DENSE_PEAK
PEAK_HBM = C.MI355X_HBM_PEAK


def flat_params(p):
    parts = [p["wte"].reshape(-1)]
    for w in p["layers"]:
        parts += [np.concatenate([w["wq"], w["wk"], w["wv"]]).reshape(-1), w["wo"].reshape(-1),
                  w["w1"].reshape(-1), w["w2"].reshape(-1)]
    parts.append(p["wlm"].reshape(-1))
    return np.concatenate(parts)


def kernel_table(prof, steps):
    rows = {}
    for name, r in prof.items():
        ms = r["ms"]
        rows[name] = dict(ms_per_step=ms / steps, launches_per_step=r["launches"] / steps,
                          tflops=(r["flops"] / (ms * 1e-3) / 1e12) if ms > 0 else 0.0,
                          gbps=(r["bytes"] / (ms * 1e-3) / 1e9) if ms > 0 else 0.0,
                          flops_per_launch=r["flops"] / max(r["launches"], 1),
                          bytes_per_launch=r["bytes"] / max(r["launches"], 1))
    return dict(sorted(rows.items(), key=lambda kv: -kv[1]["ms_per_step"]))


def roofline(table):
    name, r = next(iter(table.items()))
    if r["flops_per_launch"] > 0:
        ach = r["tflops"]
        peak = (PEAK_FP8 if name.endswith("_fp8") else PEAK_BF16) / 1e12  # a contraction against its own dtype
        return name, dict(bound="mfma", achieved=round(ach, 2), peak=round(peak, 1), unit="TFLOP/s",
                          frac=round(ach / peak, 4), traffic=None,
                          kernel=name, flops_per_launch=r["flops_per_launch"],
                          avg_launch_ms=round(r["ms_per_step"] / r["launches_per_step"], 4))
    ach = r["gbps"]
    return name, dict(bound="hbm", achieved=round(ach, 1), peak=PEAK_HBM / 1e9, unit="GB/s",
                      frac=round(ach / (PEAK_HBM / 1e9), 4), traffic=None, kernel=name,
                      bytes_per_launch=r["bytes_per_launch"],
                      avg_launch_ms=round(r["ms_per_step"] / r["launches_per_step"], 4))


def measured_traffic(scope):
    """HBM bytes per launch of `scope` from the committed counter summary
    (profiles/*_traffic.json), or None if there is none for it or the kernel
    sources changed since the counters were taken."""
    import glob
    from dense_pretraining_amd.profiling import source_hash

    for f in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.json"))):
        with open(f) as fh:
            rec = json.load(fh)
        if rec.get("scope") != scope:
            continue
        if rec.get("source_sha256") == source_hash(rec.get("sources")):
            return rec["traffic_bytes_per_launch"]
    return None


def host_info():
    """The host's CPU model (lscpu), its usable cores and the BLAS library
    NumPy calls, for the cpu_baseline record."""
    import subprocess
    from threadpoolctl import threadpool_info

    model = None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for line in out.splitlines():
            if line.lower().startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    if model is None:
        try:
            with open("/proc/cpuinfo") as fh:
                for line in fh:
                    if line.startswith("model name"):
                        model = line.split(":", 1)[1].strip()
                        break
        except OSError:
            model = "unknown"
    blas = [f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer', '?')})"
            for i in threadpool_info() if i.get("user_api") == "blas"]
    return dict(cpu=model, nproc=len(os.sched_getaffinity(0)), blas=", ".join(blas) or "unknown")


def _oracle_time(cfg, p, idx, tg, T, threads=None):
    """Wall time of the oracle's forward+backward over row 0's first T tokens."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits

    oc = oracle.Cfg(depth=cfg.depth, d_model=cfg.d_model, n_head=cfg.n_head, head_dim=cfg.head_dim,
                    n_kv_head=cfg.n_kv_head, d_ff=cfg.d_ff, vocab=cfg.vocab, batch=1, seq_len=T,
                    softcap=cfg.softcap, rope_base=cfg.rope_base, norm_eps=cfg.norm_eps)
    with threadpool_limits(limits=threads):
        used = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        t0 = time.perf_counter()
        oracle.model_loss_and_grad(oc, p, idx[:1, :T], tg[:1, :T])
        dt = time.perf_counter() - t0
    return dt, int(used)


def cpu_baseline(cfg, p, idx, tg, tokens, tokens_1t):
    """The fp64 oracle, untuned, on a bounded sample of the same workload: one
    of the batch's rows (T tokens, all blocks, the full vocabulary) on every
    host core the BLAS library uses, and a shorter row on one thread. Every
    cost of the oracle is linear in the number of rows at a fixed T, so the
    full batch takes `batch` times the first sample's time."""
    info = host_info()
    T = min(tokens, cfg.seq_len)
    dt, used = _oracle_time(cfg, p, idx, tg, T)
    rec = dict(value=round(T / dt, 2), unit="tokens/s", cores=used, kind="oracle",
               sample=f"fp64 NumPy oracle, forward+backward of the same {cfg.depth}-layer model over one of the "
                      f"batch's {cfg.batch} rows ({T} tokens, full vocabulary): {dt:.1f} s wall on {used} BLAS "
                      f"threads",
               full_batch_s_extrapolated=round(dt * cfg.batch * cfg.seq_len / T, 1) if T == cfg.seq_len else None,
               **info)
    if tokens_1t > 0:
        T1 = min(tokens_1t, cfg.seq_len)
        dt1, _ = _oracle_time(cfg, p, idx, tg, T1, threads=1)
        rec["single_thread"] = dict(value=round(T1 / dt1, 2), unit="tokens/s", cores=1,
                                    sample=f"one row of {T1} tokens on 1 thread: {dt1:.1f} s wall")
    return rec


def decode_bytes(cfg, n):
    """HBM bytes one decode step must move at cache length n: every matrix
    once, the embedding rows, the K/V cache read and the new K/V written."""
    es = 2 if cfg.dtype == "bf16" else 4
    gd = cfg.n_kv_head * cfg.head_dim
    return (es * (C.matmul_params(cfg) + cfg.batch * cfg.d_model)
            + es * cfg.depth * cfg.batch * gd * 2 * (n + 1))


def bench_infer(a, torch, lib):
    """Greedy generation: prefill of 64 x 1024 tokens, then decode steps timed
    as a group (HIP events on the library's stream). The timed generation runs
    without per-kernel events; a second one, with them, gives the kernel table."""
    cfg, n_prompt, n_steps = INFER["cfg"], INFER["prompt"], INFER["steps"]
    torch.cuda.set_device(0)
    lib.load()
    p = synth.init_params(cfg.depth, cfg.d_model, cfg.n_head, cfg.head_dim, cfg.n_kv_head, cfg.d_ff, cfg.vocab,
                          std=0.02, seed=0, dtype=cfg.dtype, out=np.float32)
    prompt, _ = synth.zipf_tokens(cfg.vocab, cfg.batch, n_prompt)
    params = torch.from_numpy(flat_params(p)).to("cuda", lib.torch_dtype(cfg))
    idx = torch.from_numpy(prompt.reshape(-1).astype(np.int32)).cuda()
    sz = lib.infer_query_sizes(cfg)
    cache = lib.alloc_bytes(sz.cache)
    ws = lib.alloc_bytes(sz.workspace)
    lib.clear_status(ws)
    nxt = torch.zeros(cfg.batch, dtype=torch.int32, device="cuda")
    toks = torch.zeros(cfg.batch, dtype=torch.int32, device="cuda")

    def generate(steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        lib.prefill(cfg, params, idx, n_prompt, cache, nxt, ws)
        e[1].record()
        for s in range(steps):
            toks.copy_(nxt)
            lib.decode_step(cfg, params, toks, n_prompt + s, cache, nxt, ws)
        e[2].record()
        torch.cuda.synchronize()
        return e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2])

    for i in range(max(a.warmup, 1)):
        generate(8)
        print(f"# warmup {i + 1}", file=sys.stderr, flush=True)
    t_pre, t_dec = generate(n_steps)
    timing = not a.no_kernel_timing
    if timing:
        lib.profile_enable(True)
        generate(n_steps)
        lib.profile_enable(False)
    st = lib.read_status(ws)
    ms_step = t_dec / n_steps
    bytes_step = sum(decode_bytes(cfg, n_prompt + s) for s in range(n_steps)) / n_steps
    out = {
        "metric": "decode tokens/s (greedy, KV cache), depth-20, 64 sequences, 1 MI355X",
        "value": round(cfg.batch * n_steps / (t_dec * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": n_steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic: seeded Zipf(1.1) prompts, N(0, 0.02) weights",
        "config": {"workload": INFER["desc"], "global_batch": cfg.batch, "seq_len": cfg.seq_len,
                   "parallelism": "none"},
        "prefill_tokens_per_s": round(cfg.batch * n_prompt / (t_pre * 1e-3), 1),
        "prefill_ms": round(t_pre, 3),
        "roofline": {"bound": "hbm", "achieved": round(bytes_step / (ms_step * 1e-3) / 1e9, 1),
                     "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                     "frac": round(bytes_step / (ms_step * 1e-3) / PEAK_HBM, 4), "traffic": None,
                     "kernel": "decode step (all kernels)", "bytes_per_step": round(bytes_step)},
        "status": st,
    }
    if timing:
        table = kernel_table(lib.profile_summary(), n_steps)
        out["kernels"] = {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()
                              if kk in ("ms_per_step", "launches_per_step", "tflops", "gbps")}
                          for k, v in table.items()}
    if a.cpu_tokens > 0:
        print("# timing the CPU oracle sample ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_infer(cfg, p, prompt, 64)
    print(json.dumps(out), flush=True)


def cpu_baseline_infer(cfg, p, prompt, n_prompt, n_steps=8):
    """The fp64 oracle's cached decode for one sequence after a short prefill
    (untimed): decode tokens per second. The per-token cost is the weight
    traffic of the whole model; the context length changes it little."""
    import oracle
    from oracle import infer
    from threadpoolctl import threadpool_info

    oc = oracle.Cfg(depth=cfg.depth, d_model=cfg.d_model, n_head=cfg.n_head, head_dim=cfg.head_dim,
                    n_kv_head=cfg.n_kv_head, d_ff=cfg.d_ff, vocab=cfg.vocab, batch=1, seq_len=cfg.seq_len,
                    softcap=cfg.softcap, rope_base=cfg.rope_base, norm_eps=cfg.norm_eps)
    cache, z = infer.prefill(oc, p, prompt[:1, :n_prompt])
    tok = infer.argmax_lowest(z)
    t0 = time.perf_counter()
    for s in range(n_steps):
        cache, z = infer.decode_step(oc, p, cache, tok, n_prompt + s)
        tok = infer.argmax_lowest(z)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return dict(value=round(n_steps / dt, 3), unit="tokens/s", cores=int(threads), kind="oracle",
                sample=f"fp64 NumPy oracle, {n_steps} cached decode steps of one sequence after a {n_prompt}-token "
                       f"prefill, {dt:.1f} s wall on {threads} BLAS threads")


# Hyperparameters of the optimizer benchmark. The pages fix none of them (only
# the 1/sqrt(dim) scaling and the end-of-run decay); the time of a step does
# not depend on their values.
OPT_HP = dict(lr_matrix=0.02, lr_embed=0.2, lr_unembed=0.004, momentum=0.95, nesterov=True, beta1=0.8, beta2=0.95,
              eps=1e-10, wd_matrix=0.0, wd_adam=0.0)


def opt_flops(cfg):
    """Newton-Schulz FLOPs of one optimizer step: per block matrix in its tall
    orientation (R >= C), five steps of A = X^T X (2RC^2), B = bA + cA^2
    (2C^3) and X B (2RC^2)."""
    d, F = cfg.d_model, cfg.d_ff
    HD, GD = cfg.n_head * cfg.head_dim, cfg.n_kv_head * cfg.head_dim
    tot = 0
    for R, Cc in ((HD, d), (GD, d), (GD, d), (d, HD), (F, d), (d, F)):
        R, Cc = max(R, Cc), min(R, Cc)
        tot += 5 * (4 * R * Cc * Cc + 2 * Cc ** 3)
    return cfg.depth * tot


def bench_opt(a, torch, lib):
    """nc_opt_step at depth 20 on seeded gradients, timed with HIP events."""
    cfg = C.DEPTH20
    torch.cuda.set_device(0)
    lib.load()
    p = synth.init_params(cfg.depth, cfg.d_model, cfg.n_head, cfg.head_dim, cfg.n_kv_head, cfg.d_ff, cfg.vocab,
                          std=0.02, seed=0, dtype=cfg.dtype, out=np.float32)
    params = torch.from_numpy(flat_params(p)).to("cuda", lib.torch_dtype(cfg))
    _, n = lib.param_layout(cfg)
    gen = torch.Generator(device="cuda").manual_seed(5)
    grads = torch.randn(n, generator=gen, device="cuda", dtype=torch.float32) * 1e-3
    sz = lib.opt_query_sizes(cfg)
    state = lib.alloc_bytes(sz.state)
    ws = lib.alloc_bytes(sz.workspace)
    lib.opt_init(cfg, params, state)
    step = [0]

    def one():
        step[0] += 1
        lib.opt_step(cfg, lib.opt_hparams(step=step[0], **OPT_HP), params, grads, state, ws)

    for i in range(a.warmup):
        one()
        torch.cuda.synchronize()
        print(f"# warmup {i + 1}/{a.warmup}", file=sys.stderr, flush=True)
    # kernel table from untimed steps, then the timed steps with events around the dominant kernel only
    timing = not a.no_kernel_timing
    if timing:
        lib.profile_only(None)
        lib.profile_enable(True)
        for _ in range(a.table_steps):
            one()
        torch.cuda.synchronize()
        lib.profile_enable(False)
        table = kernel_table(lib.profile_summary(), a.table_steps)
        lib.profile_only(next(iter(table)))
        lib.profile_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(a.steps):
        one()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps
    if timing:
        lib.profile_enable(False)
        live = kernel_table(lib.profile_summary(), a.steps)
        lib.profile_only(None)
    out = {
        "metric": "optimizer step time (Muon for the block matrices, AdamW for Wte and Wlm), depth-20, 1 MI355X",
        "value": round(ms, 3),
        "unit": "ms",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic: N(0, 0.02) weights, N(0, 1e-3) seeded gradients",
        "config": {"workload": "optimizer step of the depth-20 decoder (502M parameters; 120 Muon matrices, "
                               "Newton-Schulz products in bf16; AdamW over 2 x 65536 x 1280)",
                   "parallelism": "none"},
        "newton_schulz_tflops": round(opt_flops(cfg) / (ms * 1e-3) / 1e12, 1),
    }
    if timing:
        name, rl = roofline(live)
        out["roofline"] = rl
        out["kernels"] = {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()
                              if kk in ("ms_per_step", "launches_per_step", "tflops", "gbps")}
                          for k, v in table.items()}
    if a.cpu_tokens > 0:
        print("# timing the CPU oracle sample ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_opt(cfg, p)
    print(json.dumps(out), flush=True)


def cpu_baseline_opt(cfg, p, layers=4):
    """The fp64 oracle on layers/depth of the step (the six Muon matrices of
    the first ``layers`` layers and as large a share of the rows of Wte and
    Wlm through AdamW), scaled to the whole step."""
    from oracle import optim
    from threadpoolctl import threadpool_info

    rng = np.random.default_rng(5)
    rows = cfg.vocab * layers // cfg.depth
    t0 = time.perf_counter()
    for l in range(layers):
        for k in ("wq", "wk", "wv", "wo", "w1", "w2"):
            W = np.asarray(p["layers"][l][k], dtype=np.float64)
            optim.muon_update(W, rng.standard_normal(W.shape) * 1e-3, np.zeros_like(W), OPT_HP["lr_matrix"],
                              OPT_HP["momentum"])
    for k in ("wte", "wlm"):
        W = np.asarray(p[k][:rows], dtype=np.float64)
        optim.adamw_update(W, rng.standard_normal(W.shape) * 1e-3, 0 * W, 0 * W, 1, 0.2, 0.8, 0.95, 1e-10)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    scale = cfg.depth / layers
    return dict(value=round(dt * scale * 1e3, 1), unit="ms", cores=int(threads), kind="oracle",
                sample=f"fp64 NumPy oracle on the Muon matrices of {layers} of {cfg.depth} layers and {rows} rows "
                       f"of Wte and Wlm (AdamW), {dt:.1f} s wall on {threads} BLAS threads, scaled x{scale:g}")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", choices=sorted(WORKLOADS) + ["infer", "opt"], default="depth20",
                    help="training step (depth20, depth30, depth20_fp8), KV-cache generation (infer) or the optimizer step (opt)")
    ap.add_argument("--cpu-tokens", type=int, default=2048,
                    help="sequence length of the oracle sample for cpu_baseline, one row on every core (0 skips "
                         "the CPU baseline)")
    ap.add_argument("--cpu-tokens-1t", type=int, default=256,
                    help="sequence length of the single-thread oracle sample (0 skips it)")
    ap.add_argument("--no-kernel-timing", action="store_true",
                    help="no per-kernel HIP events: no kernel table, no roofline")
    ap.add_argument("--table-steps", type=int, default=2,
                    help="untimed steps after the warmup whose every launch is timed by HIP events (the kernel "
                         "table); the timed steps then time the dominant kernel only")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the timed steps, copy this many MiB device to device once (a plain copy kernel "
                         "of known size that calibrates the HBM byte counters of a profiling run)")
    a = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}, WORLD_SIZE {world}): the library's "
              "data-parallel step on several GPUs (one process per GPU, one gradient all-reduce) is not "
              "implemented.", file=sys.stderr)
        sys.exit(2)

    import torch
    from dense_pretraining_amd import lib

    if a.workload == "infer":
        return bench_infer(a, torch, lib)
    if a.workload == "opt":
        return bench_opt(a, torch, lib)
    cfg, desc = WORKLOADS[a.workload]
    torch.cuda.set_device(0)
    lib.load()
    t_gen = time.perf_counter()
    p = synth.init_params(cfg.depth, cfg.d_model, cfg.n_head, cfg.head_dim, cfg.n_kv_head, cfg.d_ff, cfg.vocab,
                          std=0.02, seed=0, dtype="f32" if cfg.dtype == "f32" else "bf16", out=np.float32)
    idx, tg = synth.zipf_tokens(cfg.vocab, cfg.batch, cfg.seq_len)
    params = torch.from_numpy(flat_params(p)).to("cuda", lib.torch_dtype(cfg))
    idx_d = torch.from_numpy(idx.reshape(-1)).cuda()
    tg_d = torch.from_numpy(tg.reshape(-1)).cuda()
    sz = lib.query_sizes(cfg)
    ws = lib.alloc_bytes(sz.model_workspace)
    lib.clear_status(ws)
    grads = torch.zeros(sz.n_params, dtype=torch.float32, device="cuda")
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    print(f"# inputs ready in {time.perf_counter() - t_gen:.1f} s; workspace {sz.model_workspace / 1e9:.1f} GB",
          file=sys.stderr, flush=True)

    def step():
        lib.model_loss_and_grad(cfg, params, idx_d, tg_d, loss, grads, ws)

    for i in range(a.warmup):
        step()
        torch.cuda.synchronize()
        print(f"# warmup {i + 1}/{a.warmup}", file=sys.stderr, flush=True)
    st = lib.read_status(ws)
    if st:
        print(f"# device status bits set: {st:#x}", file=sys.stderr)

    # Per-kernel table from a few untimed steps with every launch bracketed by
    # events; the timed steps then carry events around the dominant kernel
    # only (its roofline figure is measured live), since two event records
    # per launch of all ~500 launches would add about 1 % to the step.
    timing = not a.no_kernel_timing
    table = dominant = None
    if timing:
        lib.profile_only(None)
        lib.profile_enable(True)
        for _ in range(a.table_steps):
            step()
        torch.cuda.synchronize()
        lib.profile_enable(False)
        table = kernel_table(lib.profile_summary(), a.table_steps)
        dominant = next(iter(table))
        lib.profile_only(dominant)
    torch.cuda.synchronize()
    if timing:
        lib.profile_enable(True)
    # one event at every step boundary (on the stream the library launches on):
    # the per-step median, minimum and maximum beside the timed region's mean
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(a.steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    e0, e1 = ev[0], ev[-1]
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(a.steps))
    if timing:
        lib.profile_enable(False)
        live = kernel_table(lib.profile_summary(), a.steps)
        lib.profile_only(None)
    ms = e0.elapsed_time(e1) / a.steps
    print(f"# timed {a.steps} steps: {ms:.2f} ms/step (wall {wall / a.steps * 1e3:.2f})", file=sys.stderr,
          flush=True)

    if a.copy_mib > 0:
        src = torch.ones(a.copy_mib * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    tokens = cfg.batch * cfg.seq_len
    tps = tokens / (ms * 1e-3)
    f_causal = C.flops_per_token(cfg, "causal")
    f_palm = C.flops_per_token(cfg, "palm")
    out = {
        "metric": METRIC if a.workload == "depth20" else f"train tokens/sec (fwd+bwd), {a.workload}",
        "value": round(tps, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic: seeded Zipf(1.1) token ids, N(0, 0.02) weights",
        "config": {"workload": desc, "global_batch": cfg.batch, "seq_len": cfg.seq_len, "parallelism": "none"},
        # MFU against the bf16 peak in every mode (FP8 mode: the forward block products run at up to twice it)
        "mfu": round(tps * f_causal / PEAK_BF16, 4),
        "mfu_palm": round(tps * f_palm / PEAK_BF16, 4),
        "loss": round(float(loss.item()), 6),
        "step_ms": {"median": round(float(np.median(per_step)), 3), "min": round(per_step[0], 3),
                    "max": round(per_step[-1], 3)},
    }
    if timing:
        name, rl = roofline(live)
        tb = measured_traffic(name)
        rl["traffic"] = None if tb is None else round(tb)
        out["roofline"] = rl
        out["kernels"] = {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()
                              if kk in ("ms_per_step", "launches_per_step", "tflops", "gbps")}
                          for k, v in table.items()}
        out["kernel_ms_sum"] = round(sum(v["ms_per_step"] for v in table.values()), 3)
    if a.cpu_tokens > 0:
        print("# timing the CPU oracle sample ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, p, idx, tg, a.cpu_tokens, a.cpu_tokens_1t)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
