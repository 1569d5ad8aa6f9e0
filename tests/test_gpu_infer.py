"""Greedy generation with the key/value cache (nc_prefill, nc_decode_step) on
the GPU against the inference oracle.

The next token is an argmax taken in floating point, so a GPU choice is
checked for validity rather than identity: fed the same prefix (the GPU's own
tokens), the oracle's fp64 softcapped logit of the chosen token must lie
within the precision's tolerance of the largest one. The cache (K after QK
norm and rotation, V) is compared element by element with the oracle's."""

import numpy as np
import pytest
import torch

import oracle
from oracle import infer
from dense_pretraining_amd import lib, synth
from dense_pretraining_amd.config import Config
from gpu_util import TOL, assert_close, dev, flat_params, ocfg

pytestmark = pytest.mark.gpu

# argmax validity margin, relative to the largest |logit|
MARGIN = {"bf16": 4e-2, "f32": 1e-4}


def _cfg(**kw):
    base = dict(depth=2, d_model=256, n_head=4, head_dim=64, n_kv_head=1, d_ff=512, vocab=1000, batch=3,
                seq_len=48, dtype="bf16")
    base.update(kw)
    return Config(**base)


SHAPES = {
    "tiny_f32": _cfg(d_model=128, n_head=2, d_ff=512, vocab=512, batch=2, seq_len=32, dtype="f32"),
    "mqa_d64_bf16": _cfg(),
    "gqa_d128_bf16": _cfg(n_head=4, head_dim=128, n_kv_head=2, vocab=520, batch=2, seq_len=40),
    "mqa_d128_f32": _cfg(d_model=256, n_head=2, head_dim=128, vocab=264, batch=2, seq_len=24, dtype="f32"),
    # 24 query heads on one KV head: 24 of the 32 score-tile columns in use
    "rep24_d64_bf16": _cfg(n_head=24, vocab=776, batch=2, seq_len=40),
}


def _params(cfg, seed=0):
    p = synth.init_params(cfg.depth, cfg.d_model, cfg.n_head, cfg.head_dim, cfg.n_kv_head, cfg.d_ff, cfg.vocab,
                          std=0.05, seed=seed, dtype=cfg.dtype, out=np.float64)
    # logits of a few units, so that the greedy choice is decided by real gaps
    rng = np.random.default_rng(seed + 7)
    p["wlm"] = synth.round_to(rng.standard_normal(p["wlm"].shape) * (2.5 / np.sqrt(cfg.d_model)), cfg.dtype)
    return p


class Gen:
    def __init__(self, cfg, p):
        self.cfg = cfg
        self.params = dev(flat_params(cfg, p), cfg)
        sz = lib.infer_query_sizes(cfg)
        self.cache = lib.alloc_bytes(sz.cache)
        self.cache.zero_()
        self.ws = lib.alloc_bytes(sz.workspace)
        lib.clear_status(self.ws)
        self.nxt = torch.zeros(cfg.batch, dtype=torch.int32, device="cuda")

    def run(self, prompt, n_steps):
        cfg = self.cfg
        idx = torch.from_numpy(np.ascontiguousarray(prompt, dtype=np.int32).reshape(-1)).cuda()
        lib.prefill(cfg, self.params, idx, prompt.shape[1], self.cache, self.nxt, self.ws)
        toks = [self.nxt.clone()]
        for s in range(n_steps):
            tok = toks[-1].clone()
            lib.decode_step(cfg, self.params, tok, prompt.shape[1] + s, self.cache, self.nxt, self.ws)
            toks.append(self.nxt.clone())
        torch.cuda.synchronize()
        return np.stack([t.cpu().numpy() for t in toks], axis=1)

    def cache_np(self):
        cfg = self.cfg
        es = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        c = self.cache.view(es)[: cfg.depth * 2 * cfg.batch * cfg.seq_len * cfg.n_kv_head * cfg.head_dim]
        c = c.float().cpu().numpy().astype(np.float64)
        return c.reshape(cfg.depth, 2, cfg.batch, cfg.seq_len, cfg.n_kv_head, cfg.head_dim)


def _check_valid(z, tok, margin, what):
    """tok [B] must be within margin * max|z| of the row maxima of z [B, V]."""
    best = z.max(axis=1)
    got = z[np.arange(len(tok)), tok]
    slack = margin * max(1.0, np.abs(z).max())
    assert np.all(best - got <= slack), f"{what}: chosen {tok} gap {best - got} > {slack:.3e}"


def _run_and_check(cfg, p, prompt, n_steps, seed_note=""):
    g = Gen(cfg, p)
    toks = g.run(prompt, n_steps)
    assert lib.read_status(g.ws) == 0
    oc = ocfg(cfg)
    cache, z = infer.prefill(oc, p, prompt)
    _check_valid(z, toks[:, 0], MARGIN[cfg.dtype], f"prefill {seed_note}")
    for s in range(n_steps):
        cache, z = infer.decode_step(oc, p, cache, toks[:, s], prompt.shape[1] + s)
        _check_valid(z, toks[:, s + 1], MARGIN[cfg.dtype], f"decode step {s} {seed_note}")
    n = prompt.shape[1] + n_steps
    gc = g.cache_np()
    tol = TOL[cfg.dtype]["act"]
    for l, (k, v) in enumerate(cache):
        assert_close(gc[l, 0, :, :n], k, tol, f"K cache layer {l}")
        assert_close(gc[l, 1, :, :n], v, tol, f"V cache layer {l}")
    return g, toks


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_prefill_and_decode_match_oracle(name):
    cfg = SHAPES[name]
    p = _params(cfg)
    n_prompt = cfg.seq_len // 3 + 1
    prompt, _ = synth.zipf_tokens(cfg.vocab, cfg.batch, n_prompt)
    _run_and_check(cfg, p, prompt, n_steps=6, seed_note=name)


def test_prompt_of_one_token_and_full_capacity():
    cfg = SHAPES["mqa_d64_bf16"].with_(seq_len=16)
    p = _params(cfg, seed=3)
    prompt, _ = synth.zipf_tokens(cfg.vocab, cfg.batch, 1)
    # 1 prompt position + 15 decode steps fill all 16 positions of the cache
    _run_and_check(cfg, p, prompt, n_steps=cfg.seq_len - 1, seed_note="T=1")


def test_generation_is_deterministic():
    cfg = SHAPES["gqa_d128_bf16"]
    p = _params(cfg, seed=4)
    prompt, _ = synth.zipf_tokens(cfg.vocab, cfg.batch, 11)
    g = Gen(cfg, p)
    t1 = g.run(prompt, 5)
    c1 = g.cache.clone()
    t2 = g.run(prompt, 5)
    assert np.array_equal(t1, t2) and torch.equal(g.cache, c1)


def test_depth20_generation_sampled():
    """Depth-20 model at the inference benchmark's batch (64 sequences), a
    256-token prompt and 4 decode steps; sequence 0 checked against the oracle."""
    cfg = Config(depth=20, d_model=1280, n_head=10, head_dim=128, n_kv_head=1, d_ff=5120, vocab=65536, batch=64,
                 seq_len=264, dtype="bf16")
    p = synth.init_params(cfg.depth, cfg.d_model, cfg.n_head, cfg.head_dim, cfg.n_kv_head, cfg.d_ff, cfg.vocab,
                          std=0.02, seed=0, dtype="bf16", out=np.float32)
    rng = np.random.default_rng(11)
    p["wlm"] = synth.round_to(rng.standard_normal(p["wlm"].shape) * (2.5 / np.sqrt(cfg.d_model)), "bf16",
                              out=np.float32)
    prompt, _ = synth.zipf_tokens(cfg.vocab, cfg.batch, 256)
    g = Gen(cfg, p)
    toks = g.run(prompt, 4)
    assert lib.read_status(g.ws) == 0
    oc = ocfg(cfg.with_(batch=1))
    cache, z = infer.prefill(oc, p, prompt[:1])
    _check_valid(z, toks[:1, 0], MARGIN["bf16"], "depth20 prefill")
    for s in range(4):
        cache, z = infer.decode_step(oc, p, cache, toks[:1, s], 256 + s)
        _check_valid(z, toks[:1, s + 1], MARGIN["bf16"], f"depth20 decode {s}")
    gc = g.cache_np()
    for l in (0, 19):
        assert_close(gc[l, 0, :1, :260], cache[l][0], TOL["bf16"]["act"], f"K cache layer {l}")
        assert_close(gc[l, 1, :1, :260], cache[l][1], TOL["bf16"]["act"], f"V cache layer {l}")


def test_long_cache_multi_tile_chunks():
    """128 sequences x 2 KV heads over ~390 cached keys: the decode attention
    gives each block two 64-key tiles (the 2-stage ring) with a ragged last
    chunk."""
    cfg = _cfg(d_model=128, n_head=4, n_kv_head=2, d_ff=256, vocab=512, batch=128, seq_len=400)
    p = _params(cfg, seed=5)
    prompt, _ = synth.zipf_tokens(cfg.vocab, cfg.batch, 389)
    _run_and_check(cfg, p, prompt, n_steps=4, seed_note="long cache")


@pytest.mark.parametrize("pairing", ["adjacent", "far"])
def test_greedy_ties_go_to_the_lowest_id(pairing):
    """Exact ties: unembedding rows shared by two ids give both ids bitwise
    equal logits, so every greedy choice is a tie between twins and must be
    the lower id (the stated reading for an argmax tie). "adjacent": ids 2i
    and 2i + 1 (the same 32-column tile of the logit kernel), so every token
    must be even; "far": ids i and i + V/2 (different tiles, decided by the
    cross-tile reduction), so every token must be below V/2."""
    cfg = SHAPES["mqa_d64_bf16"]
    p = _params(cfg, seed=6)
    V = cfg.vocab
    w = p["wlm"]
    if pairing == "adjacent":
        w[1::2] = w[0::2]
    else:
        w[V // 2:] = w[: V // 2]
    prompt, _ = synth.zipf_tokens(cfg.vocab, cfg.batch, 9)
    g, toks = _run_and_check(cfg, p, prompt, n_steps=8, seed_note=f"ties {pairing}")
    if pairing == "adjacent":
        assert np.all(toks % 2 == 0), toks
    else:
        assert np.all(toks < V // 2), toks


def test_depth20_generation_benchmark_shape_sampled():
    """The inference benchmark's shape: 64 sequences, a 1024-token prompt, then
    decode steps up to position 1279 (cache capacity 1280). Sequence 0 is
    checked against the oracle in one forward pass over its 1279 positions
    (the prompt and the GPU's own tokens): every one of its 256 greedy tokens
    against the oracle's logits at that position, and its cache rows in
    layers 0 and 19 (positions 0 .. 1023 written by the prefill, 1024 .. 1278
    by the decode steps). Full recomputation equals cached decoding in exact
    arithmetic (pinned in the oracle's own tests)."""
    n_prompt, n_steps = 1024, 256
    cfg = Config(depth=20, d_model=1280, n_head=10, head_dim=128, n_kv_head=1, d_ff=5120, vocab=65536, batch=64,
                 seq_len=n_prompt + n_steps, dtype="bf16")
    p = synth.init_params(cfg.depth, cfg.d_model, cfg.n_head, cfg.head_dim, cfg.n_kv_head, cfg.d_ff, cfg.vocab,
                          std=0.02, seed=0, dtype="bf16", out=np.float32)
    rng = np.random.default_rng(11)
    p["wlm"] = synth.round_to(rng.standard_normal(p["wlm"].shape) * (2.5 / np.sqrt(cfg.d_model)), "bf16",
                              out=np.float32)
    prompt, _ = synth.zipf_tokens(cfg.vocab, cfg.batch, n_prompt)
    g = Gen(cfg, p)
    # positions 1024 .. 1278 are decoded: the last step appends position 1278 and
    # picks the token for 1279, the capacity's last position
    print("GPU prefill and decode ...", flush=True)
    toks = g.run(prompt, n_steps - 1)
    assert lib.read_status(g.ws) == 0
    print("oracle forward over 1279 positions ...", flush=True)
    oc = ocfg(cfg.with_(batch=1, seq_len=n_prompt + n_steps - 1))
    seq = np.concatenate([prompt[:1], toks[:1, :-1]], axis=1)  # [1, 1279]
    x, _ = oracle.embed_fwd(oc, seq, p["wte"])
    ks, vs = [], []
    for w in p["layers"]:
        x, c = oracle.block_fwd(oc, w, x)
        ks.append(c["kr"])
        vs.append(c["v"])
    z = infer.softcap_logits(oc, x[0, n_prompt - 1:, :], p["wlm"])  # positions 1023 .. 1278: [256, V]
    for s in range(n_steps):
        _check_valid(z[s:s + 1], toks[:1, s], MARGIN["bf16"], f"depth20 token after position {n_prompt - 1 + s}")
    gc = g.cache_np()
    n = n_prompt + n_steps - 1
    for l in (0, 19):
        assert_close(gc[l, 0, :1, :n], ks[l], TOL["bf16"]["act"], f"K cache layer {l}")
        assert_close(gc[l, 1, :1, :n], vs[l], TOL["bf16"]["act"], f"V cache layer {l}")
