"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test checks the oracle against a closed form, an invariant the
architecture implies, an independent library routine, or finite differences,
chosen so that a dropped term, a wrong sign or index or a transposed operand
fails at least one of them.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import Cfg
from dense_pretraining_amd import synth

TINY = Cfg(depth=2, d_model=128, n_head=2, head_dim=64, n_kv_head=1, d_ff=512,
           vocab=512, batch=2, seq_len=64)
MICRO = Cfg(depth=2, d_model=32, n_head=4, head_dim=8, n_kv_head=2, d_ff=64,
            vocab=48, batch=2, seq_len=7)


def _params(cfg, seed=0, std=0.02, dtype="f32"):
    return synth.init_params(cfg.depth, cfg.d_model, cfg.n_head, cfg.head_dim, cfg.n_kv_head,
                             cfg.d_ff, cfg.vocab, std=std, seed=seed, dtype=dtype)


def _tokens(cfg):
    return synth.zipf_tokens(cfg.vocab, cfg.batch, cfg.seq_len)


# ---------------------------------------------------------------- RMSNorm (P3, P6)

def test_rmsnorm_unit_rms_exact_form():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 33)) * np.array([1e-3, 0.02, 1, 5, 1e2, 3, 0.5])[:, None]
    eps = 1e-6
    y, r = oracle.rms_norm(x, eps)
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), ms / (ms + eps), rtol=1e-12)


def test_rmsnorm_matches_torch_library():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((5, 40))
    y, _ = oracle.rms_norm(x, 1e-6)
    yt = F.rms_norm(torch.from_numpy(x), (40,), eps=1e-6).numpy()
    np.testing.assert_allclose(y, yt, rtol=1e-13, atol=1e-15)


def test_rmsnorm_bwd_scale_invariance_and_autograd():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((6, 24)) * 0.3
    dy = rng.standard_normal((6, 24))
    eps = 1e-6
    y, r = oracle.rms_norm(x, eps)
    dx = oracle.rms_norm_bwd(dy, y, r)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    lhs = np.sum(dx * x, axis=-1)
    rhs = (r * eps / (ms + eps))[:, 0] * np.sum(dy * x, axis=-1)
    np.testing.assert_allclose(lhs, rhs, atol=1e-12)
    xt = torch.from_numpy(x).requires_grad_(True)
    F.rms_norm(xt, (24,), eps=eps).backward(torch.from_numpy(dy))
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------- RoPE (P4, P5)

def test_rope_matches_complex_rotation():
    T, D, base = 9, 16, 10000.0
    rng = np.random.default_rng(8)
    x = rng.standard_normal((T, 3, D))
    cos, sin = oracle.rope_tables(T, D, base)
    y = oracle.rope_apply(x, cos, sin)
    z = x[..., : D // 2] + 1j * x[..., D // 2:]
    t = np.arange(T)[:, None, None]
    i = np.arange(D // 2)[None, None, :]
    zr = z * np.exp(1j * t * base ** (-2.0 * i / D))
    np.testing.assert_allclose(y[..., : D // 2], zr.real, atol=1e-12)
    np.testing.assert_allclose(y[..., D // 2:], zr.imag, atol=1e-12)


def test_rope_identity_at_zero_norm_preserving_and_inverse():
    T, D = 11, 32
    rng = np.random.default_rng(9)
    x = rng.standard_normal((T, 2, D))
    cos, sin = oracle.rope_tables(T, D, 10000.0)
    y = oracle.rope_apply(x, cos, sin)
    np.testing.assert_allclose(y[0], x[0], atol=0)
    pair_in = x[..., : D // 2] ** 2 + x[..., D // 2:] ** 2
    pair_out = y[..., : D // 2] ** 2 + y[..., D // 2:] ** 2
    np.testing.assert_allclose(pair_out, pair_in, rtol=1e-12)
    np.testing.assert_allclose(oracle.rope_apply_t(y, cos, sin), x, atol=1e-12)


def test_rope_scores_depend_only_on_relative_position():
    T, D, s = 40, 64, 13
    rng = np.random.default_rng(10)
    q = rng.standard_normal(D)
    k = rng.standard_normal(D)
    cos, sin = oracle.rope_tables(T, D, 10000.0)
    Q = oracle.rope_apply(np.broadcast_to(q, (T, 1, D)).copy(), cos, sin)[:, 0]
    K = oracle.rope_apply(np.broadcast_to(k, (T, 1, D)).copy(), cos, sin)[:, 0]
    for t, u in [(5, 2), (20, 20), (9, 0), (3, 11)]:
        np.testing.assert_allclose(Q[t] @ K[u], Q[t + s] @ K[u + s], rtol=1e-10, atol=1e-12)


def test_qknorm_commutes_with_rope():
    T, D = 12, 32
    rng = np.random.default_rng(11)
    x = rng.standard_normal((T, 3, D)) * 2
    cos, sin = oracle.rope_tables(T, D, 10000.0)
    a = oracle.rope_apply(oracle.rms_norm(x, 1e-6)[0], cos, sin)
    b = oracle.rms_norm(oracle.rope_apply(x, cos, sin), 1e-6)[0]
    np.testing.assert_allclose(a, b, atol=1e-12)


# ---------------------------------------------------------------- attention (P7-P10)

def _attn_inputs(B, T, H, G, D, seed=12):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, T, H, D)), rng.standard_normal((B, T, G, D)),
            rng.standard_normal((B, T, G, D)))


def test_attention_first_position_and_single_token():
    q, k, v = _attn_inputs(2, 6, 4, 1, 8)
    o, _ = oracle.attention_fwd(q, k, v)
    for h in range(4):
        np.testing.assert_allclose(o[:, 0, h], v[:, 0, 0], atol=1e-14)
    o1, lse1 = oracle.attention_fwd(q[:, :1], k[:, :1], v[:, :1])
    np.testing.assert_allclose(o1[:, 0, 2], v[:, 0, 0], atol=1e-14)


def test_attention_matches_torch_sdpa_per_head():
    B, T, H, G, D = 2, 17, 6, 2, 16
    q, k, v = _attn_inputs(B, T, H, G, D, seed=13)
    o, lse = oracle.attention_fwd(q, k, v)
    for h in range(H):
        g = h * G // H
        qt = torch.from_numpy(q[:, :, h]).unsqueeze(1)
        kt = torch.from_numpy(k[:, :, g]).unsqueeze(1)
        vt = torch.from_numpy(v[:, :, g]).unsqueeze(1)
        ot = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True)[:, 0]
        np.testing.assert_allclose(o[:, :, h], ot.numpy(), rtol=1e-11, atol=1e-12)
        s = (qt @ kt.transpose(-1, -2))[:, 0] / np.sqrt(D)
        s = s.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), float("-inf"))
        np.testing.assert_allclose(lse[:, :, h], torch.logsumexp(s, -1).numpy(), rtol=1e-12)


def test_attention_bwd_matches_autograd():
    B, T, H, G, D = 2, 13, 4, 1, 8
    q, k, v = _attn_inputs(B, T, H, G, D, seed=14)
    do = np.random.default_rng(15).standard_normal((B, T, H, D))
    o, lse = oracle.attention_fwd(q, k, v)
    dq, dk, dv = oracle.attention_bwd(q, k, v, o, lse, do)
    qt, kt, vt = (torch.from_numpy(a).requires_grad_(True) for a in (q, k, v))
    ot = F.scaled_dot_product_attention(
        qt.transpose(1, 2), kt.transpose(1, 2).expand(B, H, T, D),
        vt.transpose(1, 2).expand(B, H, T, D), is_causal=True).transpose(1, 2)
    ot.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, vt.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_mqa_equals_mha_with_replicated_kv():
    B, T, H, D = 2, 9, 4, 8
    q, k, v = _attn_inputs(B, T, H, 1, D, seed=16)
    do = np.random.default_rng(17).standard_normal((B, T, H, D))
    o1, l1 = oracle.attention_fwd(q, k, v)
    kr, vr = np.repeat(k, H, axis=2), np.repeat(v, H, axis=2)
    o2, l2 = oracle.attention_fwd(q, kr, vr)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    _, dk1, dv1 = oracle.attention_bwd(q, k, v, o1, l1, do)
    _, dk2, dv2 = oracle.attention_bwd(q, kr, vr, o2, l2, do)
    np.testing.assert_allclose(dk1[:, :, 0], dk2.sum(axis=2), atol=1e-12)
    np.testing.assert_allclose(dv1[:, :, 0], dv2.sum(axis=2), atol=1e-12)


def test_attention_score_bound_after_qknorm():
    cfg = TINY
    p = _params(cfg, std=0.5)
    x = np.random.default_rng(18).standard_normal((2, 16, cfg.d_model))
    c = dict(cfg.__dict__)
    c["seq_len"] = 16
    _, cache = oracle.block_fwd(Cfg(**c), p["layers"][0], x)
    D = cfg.head_dim
    s = np.einsum("btd,bud->btu", cache["qr"][:, :, 0], cache["kr"][:, :, 0]) / np.sqrt(D)
    assert np.max(np.abs(s)) <= np.sqrt(D)


# ---------------------------------------------------------------- causality (P9)

def test_causality_of_logits():
    cfg = TINY
    p = _params(cfg)
    idx, _ = _tokens(cfg)
    z1 = oracle.model_forward_logits(cfg, p, idx)
    idx2 = idx.copy()
    t = 30
    idx2[:, t + 1] = (idx2[:, t + 1] + 17) % cfg.vocab
    z2 = oracle.model_forward_logits(cfg, p, idx2)
    assert np.array_equal(z1[:, : t + 1], z2[:, : t + 1])
    assert not np.allclose(z1[:, t + 1], z2[:, t + 1])


# ---------------------------------------------------------------- softcap / loss (P11, P13, P15)

def test_softcap_bound():
    cfg = TINY
    p = _params(cfg, std=1.0)
    idx, _ = _tokens(cfg)
    z = oracle.model_forward_logits(cfg, p, idx)
    assert np.max(np.abs(z)) < cfg.softcap


def test_zero_unembedding_closed_form():
    cfg = TINY
    p = _params(cfg)
    p["wlm"] = np.zeros_like(p["wlm"])
    idx, tgt = _tokens(cfg)
    loss, g = oracle.model_loss_and_grad(cfg, p, idx, tgt)
    assert abs(loss - np.log(cfg.vocab)) < 1e-12
    assert abs(np.log(512) - 6.238324625039508) < 1e-12
    for lg in g["layers"]:
        for a in lg.values():
            assert np.all(a == 0)
    assert np.all(g["wte"] == 0)
    # dWlm = dz^T xf with dz = (1/V - onehot)/Nv
    x, _ = oracle.embed_fwd(cfg, idx, p["wte"])
    for w in p["layers"]:
        x, _ = oracle.block_fwd(cfg, w, x)
    xf, _ = oracle.rms_norm(x.reshape(-1, cfg.d_model), cfg.norm_eps)
    n = xf.shape[0]
    dz = np.full((n, cfg.vocab), 1.0 / cfg.vocab)
    dz[np.arange(n), tgt.reshape(-1)] -= 1.0
    dz /= n
    np.testing.assert_allclose(g["wlm"], dz.T @ xf, atol=1e-14)


def test_identical_unembedding_rows_give_zero_input_grad():
    # all logits equal -> softmax uniform; each row of the softmax-minus-onehot
    # gradient sums to zero, so dxf = dz Wlm = 0 when every Wlm row is the same.
    cfg = TINY
    p = _params(cfg)
    row = np.random.default_rng(19).standard_normal(cfg.d_model) * 0.02
    p["wlm"] = np.tile(row, (cfg.vocab, 1))
    idx, tgt = _tokens(cfg)
    x, _ = oracle.embed_fwd(cfg, idx, p["wte"])
    loss, cache = oracle.lmhead_softcap_xent_fwd(cfg, x, p["wlm"], tgt)
    assert abs(loss - np.log(cfg.vocab)) < 1e-12
    dx, _ = oracle.lmhead_softcap_xent_bwd(cfg, x, p["wlm"], cache)
    assert np.max(np.abs(dx)) < 1e-15


def test_xent_matches_torch_cross_entropy_with_ignore():
    cfg = TINY
    rng = np.random.default_rng(20)
    x = rng.standard_normal((2, 64, cfg.d_model))
    wlm = rng.standard_normal((cfg.vocab, cfg.d_model)) * 0.3
    _, tgt = _tokens(cfg)
    tgt = tgt.copy()
    tgt[0, ::3] = -1
    loss, cache = oracle.lmhead_softcap_xent_fwd(cfg, x, wlm, tgt)
    dx, dwlm = oracle.lmhead_softcap_xent_bwd(cfg, x, wlm, cache, dloss=0.7)
    xt = torch.from_numpy(x).requires_grad_(True)
    wt = torch.from_numpy(wlm).requires_grad_(True)
    xf = F.rms_norm(xt, (cfg.d_model,), eps=cfg.norm_eps)
    z = cfg.softcap * torch.tanh(xf @ wt.T / cfg.softcap)
    lt = F.cross_entropy(z.reshape(-1, cfg.vocab), torch.from_numpy(tgt).long().reshape(-1),
                         ignore_index=-1)
    (0.7 * lt).backward()
    assert abs(loss - lt.item()) < 1e-12
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-9, atol=1e-14)
    np.testing.assert_allclose(dwlm, wt.grad.numpy(), rtol=1e-9, atol=1e-14)


# ---------------------------------------------------------------- embedding grad (P14)

def test_embedding_grad_absent_rows_zero_and_total():
    cfg = TINY
    p = _params(cfg)
    idx, _ = _tokens(cfg)
    x0, r0 = oracle.embed_fwd(cfg, idx, p["wte"])
    dx0 = np.random.default_rng(21).standard_normal(x0.shape)
    dwte = oracle.embed_bwd(cfg, idx, x0, r0, dx0, cfg.vocab)
    absent = np.setdiff1d(np.arange(cfg.vocab), np.unique(idx))
    assert absent.size > 0 and np.all(dwte[absent] == 0)
    de = oracle.rms_norm_bwd(dx0, x0, r0)
    np.testing.assert_allclose(dwte.sum(0), de.reshape(-1, cfg.d_model).sum(0), atol=1e-12)
    # brute force: per id, sum the rows in position order
    for v in np.unique(idx)[:20]:
        m = np.nonzero(idx.reshape(-1) == v)[0]
        np.testing.assert_allclose(dwte[v], de.reshape(-1, cfg.d_model)[m].sum(0), atol=1e-13)


# ---------------------------------------------------------------- whole model (P1, P2, P12, P16)

def _flat(g):
    out = [("wte", g["wte"])]
    for i, lg in enumerate(g["layers"]):
        for k in ("wq", "wk", "wv", "wo", "w1", "w2"):
            out.append((f"{k}{i}", lg[k]))
    out.append(("wlm", g["wlm"]))
    return out


def _perturbed(p, name, delta):
    q = dict(wte=p["wte"].copy(), wlm=p["wlm"].copy(),
             layers=[{k: v.copy() for k, v in lw.items()} for lw in p["layers"]])
    if name in ("wte", "wlm"):
        q[name] = q[name] + delta
    else:
        q["layers"][int(name[2:])][name[:2]] = q["layers"][int(name[2:])][name[:2]] + delta
    return q


def test_whole_model_finite_differences():
    cfg = MICRO
    p = _params(cfg, std=0.3, dtype="f32")
    rng = np.random.default_rng(22)
    idx = rng.integers(0, cfg.vocab, (cfg.batch, cfg.seq_len)).astype(np.int32)
    tgt = rng.integers(0, cfg.vocab, (cfg.batch, cfg.seq_len)).astype(np.int32)
    tgt[1, 2] = -1
    loss, g = oracle.model_loss_and_grad(cfg, p, idx, tgt)
    h = 1e-5
    for name, gt in _flat(g):
        base = _flat(p)
        shape = dict(base)[name].shape
        u = rng.standard_normal(shape)
        u /= np.linalg.norm(u)
        lp, _ = oracle.model_loss_and_grad(cfg, _perturbed(p, name, h * u), idx, tgt)
        lm, _ = oracle.model_loss_and_grad(cfg, _perturbed(p, name, -h * u), idx, tgt)
        fd = (lp - lm) / (2 * h)
        an = float(np.sum(gt * u))
        assert abs(fd - an) <= 1e-6 * max(1e-3, abs(an)) + 1e-9, (name, fd, an)


def test_whole_model_matches_torch_autograd():
    cfg = MICRO
    p = _params(cfg, std=0.3, dtype="f32")
    rng = np.random.default_rng(23)
    idx = rng.integers(0, cfg.vocab, (cfg.batch, cfg.seq_len)).astype(np.int32)
    tgt = rng.integers(0, cfg.vocab, (cfg.batch, cfg.seq_len)).astype(np.int32)
    loss, g = oracle.model_loss_and_grad(cfg, p, idx, tgt)
    B, T, d, H, G, D = cfg.batch, cfg.seq_len, cfg.d_model, cfg.n_head, cfg.n_kv_head, cfg.head_dim
    tp = {n: torch.from_numpy(a.copy()).requires_grad_(True) for n, a in _flat(p)}
    eps = cfg.norm_eps
    x = F.rms_norm(tp["wte"][torch.from_numpy(idx).long()], (d,), eps=eps)
    pos = torch.arange(T, dtype=torch.float64)
    inv = cfg.rope_base ** (-torch.arange(0, D, 2, dtype=torch.float64) / D)
    ang = pos[:, None] * inv[None]
    cs, sn = torch.cos(ang)[None, :, None], torch.sin(ang)[None, :, None]

    def rot(t):
        a, b = t[..., : D // 2], t[..., D // 2:]
        return torch.cat([a * cs - b * sn, a * sn + b * cs], -1)

    for i in range(cfg.depth):
        hh = F.rms_norm(x, (d,), eps=eps)
        q = rot(F.rms_norm((hh @ tp[f"wq{i}"].T).view(B, T, H, D), (D,), eps=eps))
        k = rot(F.rms_norm((hh @ tp[f"wk{i}"].T).view(B, T, G, D), (D,), eps=eps))
        v = (hh @ tp[f"wv{i}"].T).view(B, T, G, D)
        rep = H // G
        kk = k.repeat_interleave(rep, dim=2)
        vv = v.repeat_interleave(rep, dim=2)
        o = F.scaled_dot_product_attention(q.transpose(1, 2), kk.transpose(1, 2),
                                           vv.transpose(1, 2), is_causal=True)
        x = x + o.transpose(1, 2).reshape(B, T, H * D) @ tp[f"wo{i}"].T
        h2 = F.rms_norm(x, (d,), eps=eps)
        x = x + torch.relu(h2 @ tp[f"w1{i}"].T).square() @ tp[f"w2{i}"].T
    xf = F.rms_norm(x, (d,), eps=eps)
    z = cfg.softcap * torch.tanh(xf @ tp["wlm"].T / cfg.softcap)
    lt = F.cross_entropy(z.reshape(-1, cfg.vocab), torch.from_numpy(tgt).long().reshape(-1))
    lt.backward()
    assert abs(loss - lt.item()) < 1e-12
    for name, ga in _flat(g):
        np.testing.assert_allclose(ga, tp[name].grad.numpy(), rtol=1e-8, atol=1e-13, err_msg=name)


def test_qk_projection_grads_nearly_orthogonal_to_weights():
    cfg = TINY
    p = _params(cfg)
    idx, tgt = _tokens(cfg)
    _, g = oracle.model_loss_and_grad(cfg, p, idx, tgt)
    H, D = cfg.n_head, cfg.head_dim
    for lw, lg in zip(p["layers"], g["layers"]):
        for h in range(H):
            w = lw["wq"][h * D:(h + 1) * D]
            gw = lg["wq"][h * D:(h + 1) * D]
            assert abs(np.sum(w * gw)) / (np.linalg.norm(w) * np.linalg.norm(gw)) < 1e-3
        assert abs(np.sum(lw["wk"] * lg["wk"])) / (np.linalg.norm(lw["wk"]) * np.linalg.norm(lg["wk"])) < 1e-3


def test_batch_permutation_invariance():
    cfg = TINY
    p = _params(cfg)
    idx, tgt = _tokens(cfg)
    l1, g1 = oracle.model_loss_and_grad(cfg, p, idx, tgt)
    l2, g2 = oracle.model_loss_and_grad(cfg, p, idx[::-1].copy(), tgt[::-1].copy())
    assert abs(l1 - l2) < 1e-12
    for (n, a), (_, b) in zip(_flat(g1), _flat(g2)):
        np.testing.assert_allclose(a, b, atol=1e-12, err_msg=n)


def test_block_split_matches_whole_model():
    # the per-function entry points compose to the whole-model result
    cfg = TINY
    p = _params(cfg)
    idx, tgt = _tokens(cfg)
    loss, g = oracle.model_loss_and_grad(cfg, p, idx, tgt, dloss=2.0)
    x0, r0 = oracle.embed_fwd(cfg, idx, p["wte"])
    xs = [x0]
    for w in p["layers"]:
        xs.append(oracle.block_fwd(cfg, w, xs[-1])[0])
    l2, hc = oracle.lmhead_softcap_xent_fwd(cfg, xs[-1], p["wlm"], tgt)
    dx, dwlm = oracle.lmhead_softcap_xent_bwd(cfg, xs[-1], p["wlm"], hc, 2.0)
    assert l2 == loss
    np.testing.assert_allclose(dwlm, g["wlm"], rtol=0, atol=0)
    dx1, g1 = oracle.block_bwd(cfg, p["layers"][1], xs[1], dx)
    np.testing.assert_allclose(g1["w1"], g["layers"][1]["w1"], atol=0)
