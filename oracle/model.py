"""Plain fp64 NumPy forward and backward of the nanochat decoder (oracle).

Test infrastructure only (see the package docstring). Nothing here is tuned;
every step is the textbook definition, written so that it can be checked by
eye against the pages.

Citation keys used below:
  [arch]  page "安德烈·卡帕西推出nanochat：极简全栈AI训练项目..." (vpshk.cn),
          Q&A section "卡帕西亲自揭秘背后技术", the list of architecture
          features (dense Transformer, rotary embeddings without a position
          table, QK norm, untied embedding/unembedding, a norm right after the
          token embedding, ReLU^2 MLP, RMSNorm without parameters, bias-free
          linears, multi-query attention, logit softcap).
  [pre]   page "100美元成本、8000行代码纯手搓克隆ChatGPT!..." (imeisheng.com),
          section "预训练": next-token prediction, 32 rows x 2048 tokens per
          GPU per forward/backward, 20 layers, 1280 channels, 10 heads of 128,
          no trainable parameters other than the matrices.

Readings where the pages are silent (each also listed in the design notes):
  * RMSNorm epsilon: one constant ``norm_eps`` for every norm (default 1e-6).
  * Norm placement: after the embedding [arch], before attention and before
    the MLP of every block, and once before the unembedding.
  * RoPE: theta = rope_base, positions 0..T-1 within each row, split-half
    pairing (i, i + D/2), rotation (a, b) -> (a cos - b sin, a sin + b cos).
  * QK norm: parameter-free RMSNorm over each head's D values, same epsilon;
    applied before the rotation (the two commute exactly, since the rotation
    keeps the 2-norm).
  * Attention scale 1/sqrt(D); causal mask u <= t; query head h uses KV head
    floor(h * G / H).
  * ReLU^2: max(u, 0)^2.
  * Residuals: x + f(N(x)), no scaling.
  * Softcap: z' = c * tanh(z / c).
  * Loss: mean over targets != -1 of logsumexp(z') - z'[target].
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Cfg:
    """Model and batch shape, in the pages' terms ([pre]: depth, channels,
    heads x head dim; [arch]: multi-query attention -> n_kv_head KV heads)."""

    depth: int
    d_model: int
    n_head: int
    head_dim: int
    n_kv_head: int
    d_ff: int
    vocab: int
    batch: int
    seq_len: int
    softcap: float = 15.0
    rope_base: float = 10000.0
    norm_eps: float = 1e-6


# --------------------------------------------------------------------------
# Parameter-free RMSNorm ([arch]: no learnable norm parameters; a norm follows
# the token embedding and precedes each sublayer)
# --------------------------------------------------------------------------

def rms_norm(x, eps):
    """y = x / sqrt(mean(x^2) + eps) over the last axis; returns (y, r) with
    r = 1/sqrt(mean(x^2) + eps) (shape [..., 1])."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(ms + eps)
    return x * r, r


def rms_norm_bwd(dy, y, r):
    """Gradient of rms_norm wrt its input, written in terms of the output y
    and r: dx = r * (dy - y * mean(dy * y))."""
    return r * (dy - y * np.mean(dy * y, axis=-1, keepdims=True))


# --------------------------------------------------------------------------
# Rotary embeddings ([arch]: rotary position encoding, no position table)
# --------------------------------------------------------------------------

def rope_tables(T, D, base):
    """cos/sin of the angle t * base^(-2i/D), t in [0,T), i in [0,D/2)."""
    i = np.arange(D // 2, dtype=np.float64)
    omega = base ** (-2.0 * i / D)
    phi = np.arange(T, dtype=np.float64)[:, None] * omega[None, :]
    return np.cos(phi), np.sin(phi)


def rope_apply(x, cos, sin):
    """Rotate pairs (i, i+D/2) of x[..., T, n, D] by the angle of position t.
    cos/sin are [T, D/2]."""
    half = x.shape[-1] // 2
    a, b = x[..., :half], x[..., half:]
    c = cos[:, None, :]
    s = sin[:, None, :]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def rope_apply_t(dx, cos, sin):
    """Transpose (= inverse) rotation, used by the backward pass."""
    half = dx.shape[-1] // 2
    a, b = dx[..., :half], dx[..., half:]
    c = cos[:, None, :]
    s = sin[:, None, :]
    return np.concatenate([a * c + b * s, -a * s + b * c], axis=-1)


# --------------------------------------------------------------------------
# Causal multi-query attention ([arch]: MQA; [pre]: next-token prediction,
# hence causal)
# --------------------------------------------------------------------------

def attention_fwd(q, k, v):
    """q [B,T,H,D], k/v [B,T,G,D] -> (o [B,T,H,D], lse [B,T,H]).

    Per batch row and query head h (KV head g = floor(h*G/H)):
    S = q k^T / sqrt(D), S[t,u] = -inf for u > t, P = softmax over u, o = P v.
    """
    B, T, H, D = q.shape
    G = k.shape[2]
    o = np.zeros_like(q)
    lse = np.zeros((B, T, H))
    mask = np.triu(np.ones((T, T), dtype=bool), k=1)
    scale = 1.0 / np.sqrt(D)
    for b in range(B):
        for h in range(H):
            g = (h * G) // H
            s = (q[b, :, h, :] @ k[b, :, g, :].T) * scale
            s[mask] = -np.inf
            m = np.max(s, axis=1, keepdims=True)
            e = np.exp(s - m)
            den = np.sum(e, axis=1, keepdims=True)
            p = e / den
            o[b, :, h, :] = p @ v[b, :, g, :]
            lse[b, :, h] = (m + np.log(den))[:, 0]
    return o, lse


def attention_bwd(q, k, v, o, lse, do):
    """Gradients of attention_fwd: returns (dq, dk, dv).

    With P recomputed from q, k and lse: dP = dO v^T, Delta = rowsum(dO * o),
    dS = P * (dP - Delta), dq = dS k / sqrt(D), dk = sum over the heads that
    share the KV head of dS^T q / sqrt(D), dv = the same sum of P^T dO.
    """
    B, T, H, D = q.shape
    G = k.shape[2]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    mask = np.triu(np.ones((T, T), dtype=bool), k=1)
    scale = 1.0 / np.sqrt(D)
    for b in range(B):
        for h in range(H):
            g = (h * G) // H
            s = (q[b, :, h, :] @ k[b, :, g, :].T) * scale
            s[mask] = -np.inf
            p = np.exp(s - lse[b, :, h][:, None])
            dob = do[b, :, h, :]
            dp = dob @ v[b, :, g, :].T
            delta = np.sum(dob * o[b, :, h, :], axis=1, keepdims=True)
            ds = p * (dp - delta)
            dq[b, :, h, :] = (ds @ k[b, :, g, :]) * scale
            dk[b, :, g, :] += (ds.T @ q[b, :, h, :]) * scale
            dv[b, :, g, :] += p.T @ dob
    return dq, dk, dv


# --------------------------------------------------------------------------
# Embedding + post-embedding norm ([arch]: untied embedding; norm right after
# the token embedding)
# --------------------------------------------------------------------------

def embed_fwd(cfg, idx, wte):
    """x0 = N(Wte[idx]); idx [B,T] ints, wte [V,d]. Returns (x0, r0)."""
    e = np.asarray(wte, dtype=np.float64)[np.asarray(idx)]
    return rms_norm(e, cfg.norm_eps)


def embed_bwd(cfg, idx, x0, r0, dx0, V):
    """dWte[v] = sum over positions m with idx[m] = v of N_bwd(dx0)[m]."""
    de = rms_norm_bwd(dx0, x0, r0)
    d = de.shape[-1]
    dwte = np.zeros((V, d))
    np.add.at(dwte, np.asarray(idx).reshape(-1), de.reshape(-1, d))
    return dwte


# --------------------------------------------------------------------------
# One transformer block ([arch]: dense, bias-free linears, RoPE + QK norm,
# MQA, ReLU^2 MLP, parameter-free pre-norms)
# --------------------------------------------------------------------------

def _split_heads(cfg, qkv_like, B, T):
    H, G, D = cfg.n_head, cfg.n_kv_head, cfg.head_dim
    q = qkv_like[..., : H * D].reshape(B, T, H, D)
    k = qkv_like[..., H * D: (H + G) * D].reshape(B, T, G, D)
    v = qkv_like[..., (H + G) * D:].reshape(B, T, G, D)
    return q, k, v


def block_fwd(cfg, w, x):
    """x [B,T,d] -> (x_out, cache). w holds wq [H*D,d], wk, wv [G*D,d],
    wo [d,H*D], w1 [F,d], w2 [d,F] (nn.Linear layout [out, in]).

    h = N(x); q,k,v = h Wq^T, h Wk^T, h Wv^T; q,k <- R(N_D(.));
    x1 = x + attn(q,k,v) Wo^T; h2 = N(x1); u = h2 W1^T; a = max(u,0)^2;
    x_out = x1 + a W2^T.
    """
    B, T, d = x.shape
    H, G, D = cfg.n_head, cfg.n_kv_head, cfg.head_dim
    eps = cfg.norm_eps
    cos, sin = rope_tables(T, D, cfg.rope_base)
    h, r1 = rms_norm(x, eps)
    q = (h @ w["wq"].T).reshape(B, T, H, D)
    k = (h @ w["wk"].T).reshape(B, T, G, D)
    v = (h @ w["wv"].T).reshape(B, T, G, D)
    qn, rq = rms_norm(q, eps)
    kn, rk = rms_norm(k, eps)
    qr = rope_apply(qn, cos, sin)
    kr = rope_apply(kn, cos, sin)
    o, lse = attention_fwd(qr, kr, v)
    y = o.reshape(B, T, H * D)
    x1 = x + y @ w["wo"].T
    h2, r2 = rms_norm(x1, eps)
    u = h2 @ w["w1"].T
    a = np.maximum(u, 0.0) ** 2
    x_out = x1 + a @ w["w2"].T
    cache = dict(h=h, r1=r1, qn=qn, rq=rq, kn=kn, rk=rk, qr=qr, kr=kr, v=v,
                 o=o, lse=lse, y=y, x1=x1, h2=h2, r2=r2, u=u, a=a, cos=cos, sin=sin)
    return x_out, cache


def block_bwd(cfg, w, x, dx_out, cache=None):
    """Gradients of block_fwd. Recomputes the forward when no cache is given.
    Returns (dx_in, grads) with grads keyed like w (fp64)."""
    if cache is None:
        _, cache = block_fwd(cfg, w, x)
    B, T, d = x.shape
    H, G, D = cfg.n_head, cfg.n_kv_head, cfg.head_dim
    c = cache
    g = {}
    # MLP: x_out = x1 + a W2^T, a = max(u,0)^2, u = h2 W1^T, h2 = N(x1)
    g["w2"] = dx_out.reshape(-1, d).T @ c["a"].reshape(-1, cfg.d_ff)
    da = dx_out @ w["w2"]
    du = da * 2.0 * np.maximum(c["u"], 0.0)
    g["w1"] = du.reshape(-1, cfg.d_ff).T @ c["h2"].reshape(-1, d)
    dh2 = du @ w["w1"]
    dx1 = dx_out + rms_norm_bwd(dh2, c["h2"], c["r2"])
    # attention output projection: x1 = x + y Wo^T
    g["wo"] = dx1.reshape(-1, d).T @ c["y"].reshape(-1, H * D)
    dy = (dx1 @ w["wo"]).reshape(B, T, H, D)
    dqr, dkr, dv = attention_bwd(c["qr"], c["kr"], c["v"], c["o"], c["lse"], dy)
    # rotation, then QK norm, backward
    dqn = rope_apply_t(dqr, c["cos"], c["sin"])
    dkn = rope_apply_t(dkr, c["cos"], c["sin"])
    dq = rms_norm_bwd(dqn, c["qn"], c["rq"])
    dk = rms_norm_bwd(dkn, c["kn"], c["rk"])
    hf = c["h"].reshape(-1, d)
    g["wq"] = dq.reshape(-1, H * D).T @ hf
    g["wk"] = dk.reshape(-1, G * D).T @ hf
    g["wv"] = dv.reshape(-1, G * D).T @ hf
    dh = (dq.reshape(B, T, H * D) @ w["wq"] + dk.reshape(B, T, G * D) @ w["wk"]
          + dv.reshape(B, T, G * D) @ w["wv"])
    dx = dx1 + rms_norm_bwd(dh, c["h"], c["r1"])
    return dx, g


# --------------------------------------------------------------------------
# Final norm + unembedding + softcap + cross-entropy ([arch]: untied
# unembedding, logit softcap; [pre]: next-token cross-entropy)
# --------------------------------------------------------------------------

def _lse_rows(zc):
    m = np.max(zc, axis=-1, keepdims=True)
    return (m + np.log(np.sum(np.exp(zc - m), axis=-1, keepdims=True)))[..., 0]


def lmhead_softcap_xent_fwd(cfg, x, wlm, targets, row_chunk=512):
    """x [B,T,d] (residual stream after the last block), wlm [V,d],
    targets [B,T] ints (-1 = ignored). Returns (loss, cache).

    xf = N(x); z = xf Wlm^T; z' = c tanh(z/c);
    loss = mean over valid targets of logsumexp(z') - z'[target].
    The logits are processed in row chunks to bound memory; the chunking only
    splits independent rows.
    """
    d = x.shape[-1]
    c = cfg.softcap
    xf, rf = rms_norm(x.reshape(-1, d), cfg.norm_eps)
    y = np.asarray(targets).reshape(-1)
    valid = y >= 0
    nv = int(np.count_nonzero(valid))
    lse = np.zeros(xf.shape[0])
    zt = np.zeros(xf.shape[0])
    wlm = np.asarray(wlm, dtype=np.float64)
    for s in range(0, xf.shape[0], row_chunk):
        e = min(s + row_chunk, xf.shape[0])
        zc = c * np.tanh((xf[s:e] @ wlm.T) / c)
        lse[s:e] = _lse_rows(zc)
        rows = np.arange(e - s)
        yy = np.where(valid[s:e], y[s:e], 0)
        zt[s:e] = zc[rows, yy]
    per_tok = np.where(valid, lse - zt, 0.0)
    loss = float(np.sum(per_tok) / nv) if nv > 0 else float("nan")
    cache = dict(xf=xf, rf=rf, lse=lse, nv=nv, valid=valid, y=y)
    return loss, cache


def lmhead_softcap_xent_bwd(cfg, x, wlm, cache, dloss=1.0, row_chunk=512):
    """Gradients of lmhead_softcap_xent_fwd (times dloss): returns (dx, dwlm).

    G = (softmax(z') - onehot(target)) * dloss / Nv on valid rows, 0 otherwise;
    dz = G * (1 - (z'/c)^2); dWlm = dz^T xf; dxf = dz Wlm; dx = N_bwd(dxf).
    """
    d = x.shape[-1]
    c = cfg.softcap
    xf, rf, lse, nv, valid, y = (cache[k] for k in ("xf", "rf", "lse", "nv", "valid", "y"))
    wlm = np.asarray(wlm, dtype=np.float64)
    dxf = np.zeros_like(xf)
    dwlm = np.zeros_like(wlm)
    scale = dloss / nv if nv > 0 else 0.0
    for s in range(0, xf.shape[0], row_chunk):
        e = min(s + row_chunk, xf.shape[0])
        zc = c * np.tanh((xf[s:e] @ wlm.T) / c)
        p = np.exp(zc - lse[s:e, None])
        rows = np.arange(e - s)
        vv = valid[s:e]
        p[rows[vv], y[s:e][vv]] -= 1.0
        gz = p * (scale * vv)[:, None]
        dz = gz * (1.0 - (zc / c) ** 2)
        dwlm += dz.T @ xf[s:e]
        dxf[s:e] = dz @ wlm
    dx = rms_norm_bwd(dxf, xf, rf).reshape(x.shape)
    return dx, dwlm


# --------------------------------------------------------------------------
# Whole model
# --------------------------------------------------------------------------

def model_forward_logits(cfg, params, idx):
    """Softcapped logits z' [B,T,V] of the whole model (small shapes only)."""
    x, _ = embed_fwd(cfg, idx, params["wte"])
    for w in params["layers"]:
        x, _ = block_fwd(cfg, w, x)
    d = x.shape[-1]
    xf, _ = rms_norm(x.reshape(-1, d), cfg.norm_eps)
    z = xf @ np.asarray(params["wlm"], dtype=np.float64).T
    return (cfg.softcap * np.tanh(z / cfg.softcap)).reshape(x.shape[0], x.shape[1], -1)


def model_loss_and_grad(cfg, params, idx, targets, dloss=1.0):
    """Loss and gradients of every parameter for one forward+backward.

    params: dict(wte [V,d], layers=[dict(wq,wk,wv,wo,w1,w2)], wlm [V,d]).
    Only each block's input is kept; block internals are recomputed in the
    backward pass, which keeps the full-size model within host memory.
    Returns (loss, grads) with grads shaped like params.
    """
    x0, r0 = embed_fwd(cfg, idx, params["wte"])
    xs = [x0]
    for w in params["layers"]:
        xs.append(block_fwd(cfg, w, xs[-1])[0])
    loss, hc = lmhead_softcap_xent_fwd(cfg, xs[-1], params["wlm"], targets)
    dx, dwlm = lmhead_softcap_xent_bwd(cfg, xs[-1], params["wlm"], hc, dloss)
    glayers = [None] * len(params["layers"])
    for li in range(len(params["layers"]) - 1, -1, -1):
        dx, glayers[li] = block_bwd(cfg, params["layers"][li], xs[li], dx)
    dwte = embed_bwd(cfg, idx, x0, r0, dx, params["wte"].shape[0])
    return loss, dict(wte=dwte, layers=glayers, wlm=dwlm)
