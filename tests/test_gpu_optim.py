"""The optimizer step (nc_opt_init, nc_opt_step) on the GPU against the
optimizer oracle (oracle/optim.py).

Compared per tensor: the change of the float32 master weights since the
first step (Muon's orthogonalised direction runs its Newton-Schulz products
in the storage type, so in bf16 its tolerance is the gradient one; AdamW and
the momentum arithmetic are float32 in both modes), the Muon momentum and
AdamW moments, and the stored parameters, which must be the master weights
rounded to the storage type."""

import numpy as np
import pytest
import torch

from oracle import optim
from dense_pretraining_amd import lib, synth
from dense_pretraining_amd.config import DEPTH20, Config
from gpu_util import TOL, assert_close, dev, flat_params, host

pytestmark = pytest.mark.gpu

HP = dict(lr_matrix=0.02, lr_embed=0.3, lr_unembed=0.004, momentum=0.95, nesterov=True, beta1=0.8, beta2=0.95,
          eps=1e-10, wd_matrix=0.0, wd_adam=0.0)
# three steps: the plain setting, then no look-ahead with weight decay, then another learning rate
HP_STEPS = [HP, dict(HP, nesterov=False, wd_matrix=0.1, wd_adam=0.01, lr_matrix=0.01), dict(HP, lr_embed=0.1)]
MATS = ("wq", "wk", "wv", "wo", "w1", "w2")


def _cfg(**kw):
    base = dict(depth=2, d_model=128, n_head=2, head_dim=64, n_kv_head=1, d_ff=512, vocab=512, batch=1, seq_len=8,
                dtype="f32")
    base.update(kw)
    return Config(**base)


SHAPES = {
    # Wq, Wo square; Wk, Wv wide (64 x 128); W1 tall (512 x 128); W2 wide
    "tiny_f32": _cfg(),
    "tiny_bf16": _cfg(dtype="bf16"),
    # Wq, Wk tall (512 / 256 x 192), Wo wide (192 x 512), W1 tall, W2 wide; 192-wide rows
    "gqa_d128_bf16": _cfg(d_model=192, n_head=4, head_dim=128, n_kv_head=2, d_ff=256, vocab=264, dtype="bf16"),
    "gqa_d128_f32": _cfg(d_model=192, n_head=4, head_dim=128, n_kv_head=2, d_ff=256, vocab=264, dtype="f32"),
}


def _params(cfg, seed):
    return synth.init_params(cfg.depth, cfg.d_model, cfg.n_head, cfg.head_dim, cfg.n_kv_head, cfg.d_ff, cfg.vocab,
                             std=0.05, seed=seed, dtype=cfg.dtype, out=np.float64)


def _grads(cfg, seed):
    return synth.init_params(cfg.depth, cfg.d_model, cfg.n_head, cfg.head_dim, cfg.n_kv_head, cfg.d_ff, cfg.vocab,
                             std=1.0, seed=seed, dtype="f32", out=np.float64)


def _run_gpu(cfg, p, grads, hps):
    params = dev(flat_params(cfg, p), cfg)
    sz = lib.opt_query_sizes(cfg)
    state = torch.full((sz.state // 4,), float("nan"), dtype=torch.float32, device="cuda")
    ws = lib.alloc_bytes(sz.workspace)
    lib.opt_init(cfg, params, state)
    for t, (g, hp) in enumerate(zip(grads, hps), 1):
        gd = torch.from_numpy(flat_params(cfg, g).astype(np.float32)).cuda()
        lib.opt_step(cfg, lib.opt_hparams(step=t, **hp), params, gd, state, ws)
    torch.cuda.synchronize()
    return params, state


def _split(cfg, flat):
    """Flat parameter-layout vector -> dict shaped like the params."""
    offs, _ = lib.param_layout(cfg)
    d, V, F = cfg.d_model, cfg.vocab, cfg.d_ff
    H, G, D = cfg.n_head, cfg.n_kv_head, cfg.head_dim
    out = dict(wte=flat[offs[0]:offs[0] + V * d].reshape(V, d), layers=[],
               wlm=flat[offs[-1]:offs[-1] + V * d].reshape(V, d))
    for l in range(cfg.depth):
        qkv = flat[offs[1 + 4 * l]:offs[2 + 4 * l]].reshape(-1, d)
        out["layers"].append(dict(wq=qkv[:H * D], wk=qkv[H * D:(H + G) * D], wv=qkv[(H + G) * D:],
                                  wo=flat[offs[2 + 4 * l]:offs[3 + 4 * l]].reshape(d, H * D),
                                  w1=flat[offs[3 + 4 * l]:offs[4 + 4 * l]].reshape(F, d),
                                  w2=flat[offs[4 + 4 * l]:offs[4 + 4 * l] + d * F].reshape(d, F)))
    return out


def _check(cfg, p, params, state, st):
    _, n = lib.param_layout(cfg)
    s = host(state)
    master, s1, s2 = _split(cfg, s[:n]), _split(cfg, s[n:2 * n]), s[2 * n:]
    vd = cfg.vocab * cfg.d_model
    tol = TOL[cfg.dtype]["grad"]
    for name in ("wte", "wlm"):  # AdamW: float32 arithmetic in both modes
        assert_close(master[name] - p[name], st["master"][name] - p[name], 1e-4, f"{name} update")
        assert_close(s1[name], st["adam"][name][0], 1e-5, f"{name} first moment")
    assert_close(s2[:vd].reshape(cfg.vocab, -1), st["adam"]["wte"][1], 1e-5, "wte second moment")
    assert_close(s2[vd:].reshape(cfg.vocab, -1), st["adam"]["wlm"][1], 1e-5, "wlm second moment")
    for l in range(cfg.depth):
        for k in MATS:
            w0 = p["layers"][l][k]
            assert_close(master["layers"][l][k] - w0, st["master"]["layers"][l][k] - w0, tol, f"layer {l} {k} update")
            assert_close(s1["layers"][l][k], st["mom"][l][k], 1e-5, f"layer {l} {k} momentum")
    # the stored parameters are the master weights rounded to the storage type
    want = torch.from_numpy(s[:n].astype(np.float32)).to(lib.torch_dtype(cfg)).float().numpy()
    assert np.array_equal(host(params).astype(np.float32), want)


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_opt_steps_match_oracle(name):
    cfg = SHAPES[name]
    p = _params(cfg, 3)
    grads = [_grads(cfg, 10 + t) for t in range(3)]
    params, state = _run_gpu(cfg, p, grads, HP_STEPS)
    st = optim.init_state(p)
    for t, (g, hp) in enumerate(zip(grads, HP_STEPS), 1):
        st = optim.opt_step(st, g, t, hp)
    _check(cfg, p, params, state, st)


def test_opt_step_is_deterministic():
    cfg = SHAPES["gqa_d128_bf16"]
    p = _params(cfg, 4)
    grads = [_grads(cfg, 20 + t) for t in range(2)]
    a = _run_gpu(cfg, p, grads, HP_STEPS[:2])
    b = _run_gpu(cfg, p, grads, HP_STEPS[:2])
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_depth20_opt_step_sampled():
    """One step of the depth-20 model (502M parameters, bf16) on seeded
    gradients; checked: every matrix of layers 0 and 19 (Wq and Wo square, Wk
    and Wv wide 128 x 1280, W1 tall 5120 x 1280, W2 wide 1280 x 5120) against
    the oracle's Muon, and 512 rows of each of Wte and Wlm against AdamW."""
    cfg = DEPTH20
    p = synth.init_params(cfg.depth, cfg.d_model, cfg.n_head, cfg.head_dim, cfg.n_kv_head, cfg.d_ff, cfg.vocab,
                          std=0.02, seed=0, dtype="bf16", out=np.float32)
    offs, n = lib.param_layout(cfg)
    params = torch.from_numpy(flat_params(cfg, p)).to("cuda", torch.bfloat16)
    del p
    gen = torch.Generator(device="cuda").manual_seed(5)
    grads = torch.randn(n, generator=gen, device="cuda", dtype=torch.float32) * 1e-3
    w0 = params.float()
    sz = lib.opt_query_sizes(cfg)
    state = torch.empty(sz.state // 4, dtype=torch.float32, device="cuda")
    ws = lib.alloc_bytes(sz.workspace)
    lib.opt_init(cfg, params, state)
    lib.opt_step(cfg, lib.opt_hparams(step=1, **HP), params, grads, state, ws)
    torch.cuda.synchronize()
    d, F, V = cfg.d_model, cfg.d_ff, cfg.vocab
    HD, GD = cfg.n_head * cfg.head_dim, cfg.n_kv_head * cfg.head_dim
    for l in (0, 19):
        q = offs[1 + 4 * l]
        mats = dict(wq=(q, HD, d), wk=(q + HD * d, GD, d), wv=(q + (HD + GD) * d, GD, d), wo=(offs[2 + 4 * l], d, HD),
                    w1=(offs[3 + 4 * l], F, d), w2=(offs[4 + 4 * l], d, F))
        for k, (o, R, C) in mats.items():
            W = host(w0[o:o + R * C]).reshape(R, C)
            G = host(grads[o:o + R * C]).reshape(R, C)
            Wn, M = optim.muon_update(W, G, np.zeros_like(G), HP["lr_matrix"], HP["momentum"])
            assert_close(host(state[o:o + R * C]).reshape(R, C) - W, Wn - W, TOL["bf16"]["grad"], f"layer {l} {k}")
            assert_close(host(state[n + o:n + o + R * C]).reshape(R, C), M, 1e-6, f"layer {l} {k} momentum")
    rows = np.random.default_rng(9).choice(V, 512, replace=False)
    for name, o, lr in (("wte", offs[0], HP["lr_embed"]), ("wlm", offs[-1], HP["lr_unembed"])):
        idx = torch.from_numpy((o + rows[:, None] * d + np.arange(d)[None, :]).reshape(-1)).cuda()
        W, G = host(w0[idx]), host(grads[idx])
        Wn, _, _ = optim.adamw_update(W, G, 0 * G, 0 * G, 1, lr, HP["beta1"], HP["beta2"], HP["eps"])
        assert_close(host(state[idx]) - W, Wn - W, 1e-4, f"{name} rows")
