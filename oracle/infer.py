"""Greedy generation with a key/value cache (oracle).

Test infrastructure only, like the rest of this package. Plain fp64 NumPy.

Sources:
  [infer-a] page "100美元成本、8000行代码纯手搓克隆ChatGPT!..." (imeisheng.com):
            the feature list at its start (an inference engine with a KV
            cache and a simple prefill/decode flow) and the end of section
            "预训练" (the Engine class runs prefill and decode over a KV cache).
  [infer-b] page "如何低成本训练AI对话模型？NanoChat开源项目详解" (geoz.com.cn),
            sections "推理与部署" and "高效推理引擎与交互界面": keys and values
            are cached during inference so that earlier positions are not
            recomputed.

Readings where the pages are silent (also listed in the design notes):
  * The cache holds, per layer, the keys after QK norm and rotation and the
    values, for every position seen so far.
  * Prefill runs the prompt through the model and fills the cache; each
    decode step feeds one token per sequence at the next position.
  * Decoding is greedy: the next token is the argmax of the softcapped
    logits at the last position, ties going to the lowest id.

Two implementations, so that one pins the other:
  * ``greedy_reference`` recomputes the whole prefix with
    ``model.model_forward_logits`` at every step (the plain definition);
  * ``prefill`` / ``decode_step`` keep the cache and attend a single query
    over it, the way an inference engine does.
"""

from __future__ import annotations

import numpy as np

from .model import block_fwd, embed_fwd, rms_norm, rope_tables, model_forward_logits


def argmax_lowest(z):
    """Index of the largest value along the last axis; the first (lowest)
    index among equal maxima."""
    return np.argmax(z, axis=-1)


def softcap_logits(cfg, x, wlm):
    """z' = c tanh((N(x) Wlm^T) / c) for x [..., d]."""
    xf, _ = rms_norm(x, cfg.norm_eps)
    z = xf @ np.asarray(wlm, dtype=np.float64).T
    return cfg.softcap * np.tanh(z / cfg.softcap)


def greedy_reference(cfg, params, prompt, n_steps):
    """Greedy continuation of prompt [B, Tp] by full recomputation.
    Returns (tokens [B, n_steps + 1], logits [n_steps + 1, B, V]): tokens[:, 0]
    follows the prompt, tokens[:, s] follows prompt + tokens[:, :s]."""
    seq = np.asarray(prompt)
    toks, logs = [], []
    for _ in range(n_steps + 1):
        z = model_forward_logits(cfg, params, seq)[:, -1, :]
        t = argmax_lowest(z)
        toks.append(t)
        logs.append(z)
        seq = np.concatenate([seq, t[:, None]], axis=1)
    return np.stack(toks, axis=1), np.stack(logs)


def prefill(cfg, params, prompt):
    """Run prompt [B, Tp]; returns (cache, logits of the last position [B, V]).
    cache[l] = (k [B, Tp, G, D] after QK norm and rotation, v [B, Tp, G, D])."""
    x, _ = embed_fwd(cfg, np.asarray(prompt), params["wte"])
    cache = []
    for w in params["layers"]:
        x, c = block_fwd(cfg, w, x)
        cache.append((c["kr"], c["v"]))
    return cache, softcap_logits(cfg, x[:, -1, :], params["wlm"])


def decode_step(cfg, params, cache, tok, pos):
    """One token per sequence, tok [B], at position pos = the cache length.
    Returns (cache with position pos appended, logits [B, V])."""
    H, G, D = cfg.n_head, cfg.n_kv_head, cfg.head_dim
    eps = cfg.norm_eps
    B = len(tok)
    x, _ = embed_fwd(cfg, np.asarray(tok)[:, None], params["wte"])  # [B, 1, d]
    x = x[:, 0, :]
    cos, sin = rope_tables(pos + 1, D, cfg.rope_base)
    c_t, s_t = cos[pos], sin[pos]  # [D/2]

    def rotate(u):  # u [..., D] at position pos: pairs (i, i + D/2)
        a, b = u[..., : D // 2], u[..., D // 2:]
        return np.concatenate([a * c_t - b * s_t, a * s_t + b * c_t], axis=-1)

    new_cache = []
    for w, (kc, vc) in zip(params["layers"], cache):
        h, _ = rms_norm(x, eps)
        q = (h @ w["wq"].T).reshape(B, H, D)
        k = (h @ w["wk"].T).reshape(B, G, D)
        v = (h @ w["wv"].T).reshape(B, G, D)
        q = rotate(rms_norm(q, eps)[0])
        k = rotate(rms_norm(k, eps)[0])
        kc = np.concatenate([kc, k[:, None]], axis=1)  # [B, pos+1, G, D]
        vc = np.concatenate([vc, v[:, None]], axis=1)
        new_cache.append((kc, vc))
        o = np.zeros((B, H, D))
        for hh in range(H):
            g = hh * G // H
            s = np.einsum("bd,btd->bt", q[:, hh], kc[:, :, g]) / np.sqrt(D)  # every cached key is <= pos
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            o[:, hh] = np.einsum("bt,btd->bd", p, vc[:, :, g])
        x1 = x + o.reshape(B, H * D) @ w["wo"].T
        h2, _ = rms_norm(x1, eps)
        a = np.maximum(h2 @ w["w1"].T, 0.0) ** 2
        x = x1 + a @ w["w2"].T
    return new_cache, softcap_logits(cfg, x, params["wlm"])
