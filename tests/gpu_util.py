"""Helpers shared by the GPU parity tests: host <-> device conversion, running
the C-ABI entry points on seeded inputs, and error metrics."""

import numpy as np
import torch

import oracle
from dense_pretraining_amd import lib, synth
from dense_pretraining_amd.config import Config

TOL = {"bf16": dict(loss=1e-2, grad=3e-2, act=3e-2), "f32": dict(loss=1e-4, grad=1e-4, act=1e-4)}


def ocfg(cfg: Config) -> oracle.Cfg:
    return oracle.Cfg(depth=cfg.depth, d_model=cfg.d_model, n_head=cfg.n_head, head_dim=cfg.head_dim,
                      n_kv_head=cfg.n_kv_head, d_ff=cfg.d_ff, vocab=cfg.vocab, batch=cfg.batch,
                      seq_len=cfg.seq_len, softcap=cfg.softcap, rope_base=cfg.rope_base, norm_eps=cfg.norm_eps)


def dev(a, cfg, dtype=None):
    """float64 array holding storage-rounded values -> device tensor (exact)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device="cuda", dtype=dtype or lib.torch_dtype(cfg))


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_fro(g, ref):
    den = np.linalg.norm(ref)
    return np.linalg.norm(g - ref) / (den if den > 0 else 1.0)


def assert_close(g, ref, tol, name):
    """Per-tensor relative Frobenius error <= tol, and every element within
    tol of the tensor's largest magnitude."""
    g = np.asarray(g, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, (name, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), name
    e = rel_fro(g, ref)
    scale = np.max(np.abs(ref)) if ref.size else 0.0
    emax = np.max(np.abs(g - ref)) if ref.size else 0.0
    assert e <= tol, f"{name}: relative Frobenius error {e:.3e} > {tol:.1e}"
    assert emax <= tol * max(scale, 1e-30), f"{name}: max element error {emax:.3e} > {tol:.1e} * {scale:.3e}"
    return e


def params(cfg, seed=0, std=0.02, fan_in=False):
    return synth.init_params(cfg.depth, cfg.d_model, cfg.n_head, cfg.head_dim, cfg.n_kv_head, cfg.d_ff,
                             cfg.vocab, std=std, seed=seed, dtype=cfg.dtype, fan_in_std=fan_in)


def pack_block(w):
    return dict(wqkv=np.concatenate([w["wq"], w["wk"], w["wv"]], axis=0), wo=w["wo"], w1=w["w1"], w2=w["w2"])


def unpack_qkv(g, cfg):
    H, G, D = cfg.n_head, cfg.n_kv_head, cfg.head_dim
    return g[: H * D], g[H * D:(H + G) * D], g[(H + G) * D:]


def flat_params(cfg, p):
    """Flat parameter vector in the library's layout."""
    parts = [p["wte"].reshape(-1)]
    for w in p["layers"]:
        b = pack_block(w)
        parts += [b["wqkv"].reshape(-1), b["wo"].reshape(-1), b["w1"].reshape(-1), b["w2"].reshape(-1)]
    parts.append(p["wlm"].reshape(-1))
    return np.concatenate(parts)


def split_grads(cfg, flat):
    offs, n = lib.param_layout(cfg)
    d, V, F = cfg.d_model, cfg.vocab, cfg.d_ff
    HD = cfg.n_head * cfg.head_dim
    out = dict(wte=flat[offs[0]:offs[0] + V * d].reshape(V, d), layers=[],
               wlm=flat[offs[-1]:offs[-1] + V * d].reshape(V, d))
    for l in range(cfg.depth):
        o = offs[1 + 4 * l: 5 + 4 * l]
        wqkv = flat[o[0]:o[0] + cfg.qkv_dim * d].reshape(cfg.qkv_dim, d)
        wq, wk, wv = unpack_qkv(wqkv, cfg)
        out["layers"].append(dict(wq=wq, wk=wk, wv=wv, wo=flat[o[1]:o[1] + d * HD].reshape(d, HD),
                                  w1=flat[o[2]:o[2] + F * d].reshape(F, d), w2=flat[o[3]:o[3] + d * F].reshape(d, F)))
    return out


class ModelRun:
    """Device buffers for nc_model_loss_and_grad on one configuration."""

    def __init__(self, cfg, p, idx, targets):
        self.cfg = cfg
        self.params = dev(flat_params(cfg, p), cfg)
        self.idx = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32).reshape(-1)).cuda()
        self.tg = torch.from_numpy(np.ascontiguousarray(targets, dtype=np.int32).reshape(-1)).cuda()
        sz = lib.query_sizes(cfg)
        self.ws = lib.alloc_bytes(sz.model_workspace)
        lib.clear_status(self.ws)
        self.grads = torch.zeros(sz.n_params, dtype=torch.float32, device="cuda")
        self.loss = torch.zeros(1, dtype=torch.float32, device="cuda")

    def run(self, dloss=1.0, accumulate=False):
        lib.model_loss_and_grad(self.cfg, self.params, self.idx, self.tg, self.loss, self.grads, self.ws,
                                dloss=dloss, accumulate=accumulate)
        torch.cuda.synchronize()
        return float(self.loss.item())

    def status(self):
        return lib.read_status(self.ws)
