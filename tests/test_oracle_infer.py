"""Pins of the inference oracle (CPU): the cached single-query decode must
reproduce the plain definition -- the whole prefix recomputed -- and greedy
picks the lowest id among equal maxima."""

import numpy as np

import oracle
from oracle import infer
from dense_pretraining_amd import synth

CFG = oracle.Cfg(depth=2, d_model=128, n_head=4, head_dim=32, n_kv_head=1, d_ff=512, vocab=512, batch=3, seq_len=16)


def _params(cfg, seed=0):
    return synth.init_params(cfg.depth, cfg.d_model, cfg.n_head, cfg.head_dim, cfg.n_kv_head, cfg.d_ff, cfg.vocab,
                             std=0.05, seed=seed, dtype="f32", out=np.float64)


def test_argmax_lowest_breaks_ties_to_lowest_id():
    z = np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0], [0.0, -1.0, 7.0, 7.0]])
    assert list(infer.argmax_lowest(z)) == [1, 0, 2]


def test_cached_decode_equals_full_recompute():
    p = _params(CFG)
    prompt, _ = synth.zipf_tokens(CFG.vocab, CFG.batch, 7)
    cache, z = infer.prefill(CFG, p, prompt)
    seq = np.asarray(prompt)
    np.testing.assert_allclose(z, oracle.model_forward_logits(CFG, p, seq)[:, -1, :], atol=1e-12, rtol=0)
    for step in range(5):
        tok = infer.argmax_lowest(z)
        pos = seq.shape[1]
        cache, z = infer.decode_step(CFG, p, cache, tok, pos)
        seq = np.concatenate([seq, tok[:, None]], axis=1)
        ref = oracle.model_forward_logits(CFG, p, seq)[:, -1, :]
        assert np.max(np.abs(z - ref)) < 1e-10, step
        assert cache[0][0].shape[1] == pos + 1


def test_greedy_reference_matches_cached_generation():
    p = _params(CFG, seed=5)
    prompt, _ = synth.zipf_tokens(CFG.vocab, CFG.batch, 5, seed_rank=3, seed_perm=4)
    toks, logs = infer.greedy_reference(CFG, p, prompt, 4)
    cache, z = infer.prefill(CFG, p, prompt)
    got = [infer.argmax_lowest(z)]
    pos = prompt.shape[1]
    for s in range(4):
        cache, z = infer.decode_step(CFG, p, cache, got[-1], pos + s)
        got.append(infer.argmax_lowest(z))
    assert np.array_equal(np.stack(got, axis=1), toks)
    assert logs.shape == (5, CFG.batch, CFG.vocab)


def test_cache_holds_normed_rotated_keys():
    # keys in the cache have unit RMS per head (QK norm) at every position
    p = _params(CFG, seed=2)
    prompt, _ = synth.zipf_tokens(CFG.vocab, CFG.batch, 6)
    cache, _ = infer.prefill(CFG, p, prompt)
    for k, v in cache:
        rms = np.sqrt(np.mean(k ** 2, axis=-1))
        np.testing.assert_allclose(rms, 1.0, atol=1e-5)
        assert v.shape == k.shape
