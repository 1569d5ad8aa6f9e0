"""Pins of the per-product oracle (oracle/products.py) to facts outside it
(CPU only): adjoint identities, finite differences, closed forms and the
model oracle's own block, so that a transposed operand, a dropped factor or a
wrong sign fails one of them."""

import numpy as np

import oracle
from oracle import products as P

RNG = np.random.default_rng(2024)


def _r(*shape):
    return RNG.standard_normal(shape)


def test_xwt_identity_weight_and_residual():
    a = _r(5, 8)
    np.testing.assert_array_equal(P.xwt(a, np.eye(8)), a)
    aux = _r(5, 8)
    np.testing.assert_allclose(P.xwt(a, np.eye(8), aux), a + aux, rtol=0, atol=0)
    # a non-square weight: output rows follow w's rows ([out, in] layout)
    w = _r(3, 8)
    y = P.xwt(a, w)
    assert y.shape == (5, 3)
    np.testing.assert_allclose(y[:, 1], a @ w[1], rtol=1e-14)


def test_dyw_is_the_adjoint_of_xwt_in_a():
    # <dyw(g, w), da> = <g, xwt(da, w)> for all da: dyw is the gradient wrt a
    a, w, g = _r(6, 8), _r(4, 8), _r(6, 4)
    da = _r(*a.shape)
    np.testing.assert_allclose(np.sum(P.dyw(g, w) * da), np.sum(g * P.xwt(da, w)), rtol=1e-12)
    assert P.dyw(g, w).shape == a.shape


def test_dw_is_the_adjoint_of_xwt_in_w():
    a, w, g = _r(6, 8), _r(4, 8), _r(6, 4)
    dwt = _r(*w.shape)
    np.testing.assert_allclose(np.sum(P.dw(g, a) * dwt), np.sum(g * P.xwt(a, dwt)), rtol=1e-12)
    assert P.dw(g, a).shape == w.shape
    # token-additive: the gradient over rows [0, k) plus the one over [k, M) is the whole
    np.testing.assert_allclose(P.dw(g[:2], a[:2]) + P.dw(g[2:], a[2:]), P.dw(g, a), rtol=1e-12)


def test_drelusq_matches_finite_differences_of_relusq():
    # f(u) = <G, max(u, 0)^2> with G = dy w; its gradient is dyw_drelusq(dy, w, act)
    x, w1 = _r(5, 6), _r(7, 6)
    dy, w = _r(5, 3), _r(3, 7)
    u = P.xwt(x, w1)
    act = np.maximum(u, 0.0) ** 2
    np.testing.assert_allclose(P.xwt_relusq(x, w1), act, rtol=0, atol=0)
    G = P.dyw(dy, w)
    grad = P.dyw_drelusq(dy, w, act)
    d = _r(*u.shape)
    h = 1e-6
    fd = (np.sum(G * np.maximum(u + h * d, 0) ** 2) - np.sum(G * np.maximum(u - h * d, 0) ** 2)) / (2 * h)
    np.testing.assert_allclose(np.sum(grad * d), fd, rtol=1e-7)


def test_products_compose_to_the_block_mlp():
    # the block oracle's MLP output and weight gradients from the products
    cfg = oracle.Cfg(depth=1, d_model=16, n_head=2, head_dim=8, n_kv_head=1, d_ff=32, vocab=8, batch=1, seq_len=5)
    rng = np.random.default_rng(3)
    w = dict(wq=rng.standard_normal((16, 16)) * 0.2, wk=rng.standard_normal((8, 16)) * 0.2,
             wv=rng.standard_normal((8, 16)) * 0.2, wo=rng.standard_normal((16, 16)) * 0.2,
             w1=rng.standard_normal((32, 16)) * 0.2, w2=rng.standard_normal((16, 32)) * 0.2)
    x = rng.standard_normal((1, 5, 16))
    dy = rng.standard_normal((1, 5, 16))
    out, cache = oracle.block_fwd(cfg, w, x)
    _, g = oracle.block_bwd(cfg, w, x, dy, cache)
    # the MLP half from the block's x1 (after attention): x_out = x1 + relu^2(N(x1) W1^T) W2^T
    x1 = cache["x1"].reshape(5, 16)
    h2, _ = oracle.rms_norm(x1, cfg.norm_eps)
    act = P.xwt_relusq(h2, w["w1"])
    np.testing.assert_allclose(P.xwt(act, w["w2"], x1), out.reshape(5, 16), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(P.dw(dy.reshape(5, 16), act), g["w2"], rtol=1e-10, atol=1e-12)
    du = P.dyw_drelusq(dy.reshape(5, 16), w["w2"], act)
    np.testing.assert_allclose(P.dw(du, h2), g["w1"], rtol=1e-10, atol=1e-12)


def test_softcap_bound_small_logit_limit_and_zero_weights():
    a, w = _r(4, 16), _r(40, 16)
    zc = P.softcap_logits(a * 10, w, 15.0)
    assert np.all(np.abs(zc) < 15.0)
    small = P.softcap_logits(a * 1e-4, w, 15.0)
    np.testing.assert_allclose(small, P.xwt(a * 1e-4, w), rtol=1e-8)
    # zero weights: z' = 0, so each tile's sum of exp counts its columns
    s = P.tile_exp_sums(P.softcap_logits(a, np.zeros_like(w), 15.0), 16)
    np.testing.assert_array_equal(s, np.tile([16.0, 16.0, 8.0], (4, 1)))
    # the tile sums add up to the row's sum of exp
    s = P.tile_exp_sums(zc, 16)
    np.testing.assert_allclose(s.sum(axis=1), np.exp(zc).sum(axis=1), rtol=1e-13)


def test_axpby_and_gram():
    a, w, aux = _r(5, 6), _r(4, 6), _r(5, 4)
    np.testing.assert_allclose(P.axpby(a, w, 1.0), P.xwt(a, w), rtol=0, atol=0)
    np.testing.assert_allclose(P.axpby(a, w, 0.5, -2.0, aux), 0.5 * (a @ w.T) - 2.0 * aux, rtol=1e-14)
    g = P.gram(a)
    np.testing.assert_allclose(g, g.T, rtol=0, atol=0)
    assert np.all(np.linalg.eigvalsh(g) > -1e-10)
    np.testing.assert_allclose(np.diag(g), np.sum(a * a, axis=0), rtol=1e-13)
