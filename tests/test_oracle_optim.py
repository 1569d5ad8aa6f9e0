"""Pins of the optimizer oracle (oracle/optim.py) against closed forms, an
independent SVD route and torch's AdamW."""

import numpy as np
import pytest
import torch

from oracle import optim

RNG = np.random.default_rng(12)


def _poly_iter(s):
    a, b, c = optim.NS_COEFFS
    for _ in range(optim.NS_STEPS):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


@pytest.mark.parametrize("shape", [(48, 32), (32, 48), (40, 40), (200, 24), (8, 120)])
def test_newton_schulz_is_the_quintic_on_singular_values(shape):
    """X -> aX + b(XX^T)X + c(XX^T)^2 X acts on each singular value as
    s -> a s + b s^3 + c s^5 and keeps the singular vectors: after normalising
    G = U S V^T by its Frobenius norm, five steps give U p(S/|G|) V^T."""
    G = RNG.standard_normal(shape) * 3.0
    U, S, Vt = np.linalg.svd(G, full_matrices=False)
    want = (U * _poly_iter(S / (np.linalg.norm(G) + 1e-7))) @ Vt
    np.testing.assert_allclose(optim.newton_schulz5(G), want, rtol=0, atol=1e-10)


def test_newton_schulz_transpose_and_scale():
    G = RNG.standard_normal((30, 70))
    X = optim.newton_schulz5(G)
    np.testing.assert_allclose(optim.newton_schulz5(G.T), X.T, rtol=0, atol=1e-12)
    # the 1e-7 guard in the normalisation, amplified by up to a^5 = 484, is the only difference
    np.testing.assert_allclose(optim.newton_schulz5(G * 1e3), X, rtol=0, atol=1e-7)
    # a well-conditioned input ends with every singular value in the iteration's band around 1
    s = np.linalg.svd(X, compute_uv=False)
    assert s.min() > 0.6 and s.max() < 1.25


def test_muon_first_and_second_step():
    W = RNG.standard_normal((64, 16))
    G1, G2 = RNG.standard_normal((2, 64, 16))
    lr, mu = 0.05, 0.9
    W1, M1 = optim.muon_update(W, G1, np.zeros_like(W), lr, mu)
    # first step: M = G, U = (1 + mu) G, and the normalisation removes the scale
    np.testing.assert_allclose(M1, G1, atol=0)
    # (1 + mu) G normalises to G up to the 1e-7 guard
    np.testing.assert_allclose(W1, W - lr * 2.0 * optim.newton_schulz5(G1), atol=1e-9)
    W2, M2 = optim.muon_update(W1, G2, M1, lr, mu)
    np.testing.assert_allclose(M2, mu * G1 + G2, atol=1e-14)
    np.testing.assert_allclose(W2, W1 - lr * 2.0 * optim.newton_schulz5(G2 + mu * (mu * G1 + G2)), atol=1e-12)
    # without the look-ahead the direction is the momentum itself; decay scales W first
    W3, _ = optim.muon_update(W, G1, np.zeros_like(W), lr, mu, nesterov=False, wd=0.1)
    np.testing.assert_allclose(W3, W * (1 - lr * 0.1) - lr * 2.0 * optim.newton_schulz5(G1), atol=1e-9)


def test_adamw_matches_torch():
    W0 = RNG.standard_normal((20, 7))
    grads = RNG.standard_normal((5, 20, 7))
    hp = dict(lr=0.01, betas=(0.8, 0.95), eps=1e-10, weight_decay=0.05)
    p = torch.nn.Parameter(torch.from_numpy(W0.copy()))
    opt = torch.optim.AdamW([p], **hp)
    W, m, v = W0, np.zeros_like(W0), np.zeros_like(W0)
    for t, g in enumerate(grads, 1):
        p.grad = torch.from_numpy(g.copy())
        opt.step()
        W, m, v = optim.adamw_update(W, g, m, v, t, hp["lr"], *hp["betas"], hp["eps"], hp["weight_decay"])
        np.testing.assert_allclose(W, p.detach().numpy(), rtol=0, atol=1e-13)


def test_adamw_closed_forms():
    W0 = RNG.standard_normal(50)
    g = RNG.standard_normal(50)
    W, m, v = W0, np.zeros(50), np.zeros(50)
    for t in range(1, 8):  # a constant gradient: m_hat = g and v_hat = g^2 exactly
        W, m, v = optim.adamw_update(W, g, m, v, t, 0.1, 0.9, 0.99, 0.0)
    np.testing.assert_allclose(W, W0 - 0.7 * np.sign(g), atol=1e-12)
    W, m, v = W0, np.zeros(50), np.zeros(50)
    for t in range(1, 6):  # no gradient: only the decay
        W, m, v = optim.adamw_update(W, np.zeros(50), m, v, t, 0.1, 0.9, 0.99, 1e-8, wd=0.5)
    np.testing.assert_allclose(W, W0 * 0.95 ** 5, atol=1e-14)


def test_lr_schedule():
    assert [optim.lr_multiplier(s, 10, 0.2) for s in (0, 7, 8, 9, 10)] == [1.0, 1.0, 1.0, 0.5, 0.0]
    assert optim.lr_multiplier(5, 10, 0.0) == 1.0
    # 1/sqrt(dim): four times the width, half the learning rate
    assert optim.dim_scaled_lr(0.02, 3072, 768) == pytest.approx(0.01)


def test_opt_step_treats_each_matrix_separately():
    from dense_pretraining_amd import synth
    p = synth.init_params(2, 32, 2, 16, 1, 64, 40, std=0.1, seed=1, dtype="f32", out=np.float64)
    g = synth.init_params(2, 32, 2, 16, 1, 64, 40, std=1.0, seed=2, dtype="f32", out=np.float64)
    hp = dict(lr_matrix=0.02, lr_embed=0.3, lr_unembed=0.004, momentum=0.95, beta1=0.8, beta2=0.95, eps=1e-10)
    st = optim.opt_step(optim.init_state(p), g, 1, hp)
    for l, w in enumerate(p["layers"]):
        for k in ("wq", "wk", "wv", "wo", "w1", "w2"):
            want, _ = optim.muon_update(w[k], g["layers"][l][k], np.zeros_like(w[k]), 0.02, 0.95)
            np.testing.assert_allclose(st["master"]["layers"][l][k], want, atol=1e-13)
    want, _, _ = optim.adamw_update(p["wte"], g["wte"], 0 * p["wte"], 0 * p["wte"], 1, 0.3, 0.8, 0.95, 1e-10)
    np.testing.assert_allclose(st["master"]["wte"], want, atol=1e-13)
