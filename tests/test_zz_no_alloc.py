"""nc_decode_step_noalloc (the decode step with its scratch in the library's
static device array) against nc_decode_step (the same kernels on a caller
workspace), through the C ABI: two calls in a row, the second with a smaller
input (fewer sequences, a shorter cache), must give bitwise the same next
tokens and cache as the workspace entry point."""

import numpy as np
import pytest
import torch

from dense_pretraining_amd import lib, synth
from dense_pretraining_amd.config import Config
from gpu_util import dev, flat_params

pytestmark = pytest.mark.gpu


def _cfg(batch, seq_len):
    return Config(depth=2, d_model=256, n_head=4, head_dim=64, n_kv_head=1, d_ff=512, vocab=1000, batch=batch,
                  seq_len=seq_len, dtype="bf16")


def _decode_both(cfg, seed, n_prompt, n_steps):
    p = synth.init_params(cfg.depth, cfg.d_model, cfg.n_head, cfg.head_dim, cfg.n_kv_head, cfg.d_ff, cfg.vocab,
                          std=0.05, seed=seed, dtype="bf16", out=np.float64)
    p["wlm"] = synth.round_to(np.random.default_rng(seed + 7).standard_normal(p["wlm"].shape) * 2.5 / 16.0, "bf16")
    params = dev(flat_params(cfg, p), cfg)
    prompt, _ = synth.zipf_tokens(cfg.vocab, cfg.batch, n_prompt)
    idx = torch.from_numpy(np.ascontiguousarray(prompt, dtype=np.int32).reshape(-1)).cuda()
    sz = lib.infer_query_sizes(cfg)
    ws = lib.alloc_bytes(sz.workspace)
    lib.clear_status(ws)
    caches = [lib.alloc_bytes(sz.cache).zero_() for _ in range(2)]
    first = torch.zeros(cfg.batch, dtype=torch.int32, device="cuda")
    lib.prefill(cfg, params, idx, n_prompt, caches[0], first, ws)
    caches[1].copy_(caches[0])
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    toks = [[first.clone()], [first.clone()]]
    for s in range(n_steps):
        pos = n_prompt + s
        nxt = torch.zeros(cfg.batch, dtype=torch.int32, device="cuda")
        lib.decode_step(cfg, params, toks[0][-1], pos, caches[0], nxt, ws)
        toks[0].append(nxt)
        nxt2 = torch.full((cfg.batch,), -1, dtype=torch.int32, device="cuda")
        lib.decode_step_noalloc(cfg, params, toks[1][-1], pos, caches[1], nxt2, status)
        toks[1].append(nxt2)
    torch.cuda.synchronize()
    assert lib.read_status(ws) == 0 and int(status.item()) == 0
    a = torch.stack(toks[0]).cpu().numpy()
    b = torch.stack(toks[1]).cpu().numpy()
    assert np.array_equal(a, b), (a, b)
    assert torch.equal(caches[0], caches[1])
    return a


def test_noalloc_decode_matches_workspace_decode_twice():
    # first a larger call, then a smaller one on the same static scratch
    _decode_both(_cfg(batch=24, seq_len=160), seed=1, n_prompt=100, n_steps=5)
    _decode_both(_cfg(batch=3, seq_len=40), seed=2, n_prompt=17, n_steps=4)


def test_noalloc_decode_rejects_too_large_and_bad_arguments():
    # 4096 sequences of the depth-20 width need more than the static array holds
    big = Config(depth=1, d_model=1280, n_head=10, head_dim=128, n_kv_head=1, d_ff=5120, vocab=65536, batch=4096,
                 seq_len=64, dtype="bf16")
    t = torch.zeros(8, dtype=torch.int32, device="cuda")
    with pytest.raises(lib.NcError) as e:
        lib.decode_step_noalloc(big, t, t, 1, t, t)
    assert e.value.code == 4  # NC_ERR_WORKSPACE, before any launch
    with pytest.raises(lib.NcError) as e:
        lib.decode_step_noalloc(_cfg(batch=3, seq_len=40), t, t, 0, t, t)  # position 0 is the prompt's
    assert e.value.code == 2
