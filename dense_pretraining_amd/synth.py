"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle.

This module only draws random numbers and rounds them to the storage type; it
contains none of the model's arithmetic. Both sides receive exactly the same
host arrays, so a parity comparison measures compute error, not input
quantisation.

Recipe (the pages train on FineWeb-EDU tokens, 32 rows x 2048 tokens per GPU;
seeded Zipf rows stand in for them):
  * tokens: finite Zipf law p(r) ~ r^-s over ranks 1..V (s = 1.1), sampled by
    inverse CDF from ``default_rng(seed_rank)``, mapped to ids through
    ``default_rng(seed_perm).permutation(V)``; B x (T+1) draws, idx = [:, :T],
    targets = [:, 1:].
  * parameters: ``default_rng(seed)`` standard normals times std, drawn in the
    order Wte, then per layer Wq, Wk, Wv, Wo, W1, W2, then Wlm.
"""

from __future__ import annotations

import numpy as np


def round_bf16(x):
    """Round to the nearest bfloat16 (ties to even); returns float32 values.
    (Finite inputs; NaN stays NaN.)"""
    f = np.array(x, dtype=np.float32, copy=True, order="C")
    nan = np.isnan(f)
    u = f.view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    if nan.any():
        f[nan] = np.nan
    return f


def bf16_bits(x):
    """uint16 bit patterns of round_bf16(x)."""
    return (round_bf16(x).view(np.uint32) >> 16).astype(np.uint16)


def from_bf16_bits(b):
    """float32 values of uint16 bfloat16 bit patterns."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to(x, dtype, out=np.float64):
    """Round to the storage type ('bf16' or 'f32'); returns `out` values
    (float64 by default; float32 holds them exactly too)."""
    if dtype == "bf16":
        return round_bf16(x).astype(out, copy=False)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(out, copy=False)
    raise ValueError(dtype)


def zipf_tokens(vocab, batch, seq_len, s=1.1, seed_rank=1, seed_perm=2):
    """Seeded Zipf(s) token rows: returns (idx, targets), int32 [B, T]."""
    ranks = np.arange(1, vocab + 1, dtype=np.float64)
    p = ranks ** (-s)
    cdf = np.cumsum(p)
    cdf /= cdf[-1]
    u = np.random.default_rng(seed_rank).random(batch * (seq_len + 1))
    r = np.minimum(np.searchsorted(cdf, u, side="right"), vocab - 1)
    perm = np.random.default_rng(seed_perm).permutation(vocab)
    ids = perm[r].reshape(batch, seq_len + 1).astype(np.int32)
    return np.ascontiguousarray(ids[:, :seq_len]), np.ascontiguousarray(ids[:, 1:])


def normal(shape, std, rng, dtype, out=np.float64):
    """std * N(0,1) of the given shape, rounded to dtype, as `out` values."""
    x = rng.standard_normal(shape, dtype=np.float32)
    x *= np.float32(std)
    return round_to(x, dtype, out)


def init_params(depth, d_model, n_head, head_dim, n_kv_head, d_ff, vocab,
                std=0.02, seed=0, dtype="bf16", fan_in_std=False, out=np.float64):
    """Model parameters as float64 arrays holding storage-rounded values.

    With fan_in_std=True every matrix uses std = 1/sqrt(fan_in) instead of std.
    Returns dict(wte, layers=[dict(wq, wk, wv, wo, w1, w2)], wlm)."""
    rng = np.random.default_rng(seed)
    H, G, D, d, F, V = n_head, n_kv_head, head_dim, d_model, d_ff, vocab

    def draw(shape):
        sd = 1.0 / np.sqrt(shape[1]) if fan_in_std else std
        return normal(shape, sd, rng, dtype, out)

    wte = draw((V, d))
    layers = []
    for _ in range(depth):
        layers.append(dict(wq=draw((H * D, d)), wk=draw((G * D, d)), wv=draw((G * D, d)),
                           wo=draw((d, H * D)), w1=draw((F, d)), w2=draw((d, F))))
    wlm = draw((V, d))
    return dict(wte=wte, layers=layers, wlm=wlm)


def block_inputs(batch, seq_len, d_model, seed_x=3, seed_dy=4, dtype="bf16"):
    """Block-level inputs: x ~ N(0,1) and upstream grad dY ~ N(0,1) [B,T,d]."""
    x = normal((batch, seq_len, d_model), 1.0, np.random.default_rng(seed_x), dtype)
    dy = normal((batch, seq_len, d_model), 1.0, np.random.default_rng(seed_dy), dtype)
    return x, dy
