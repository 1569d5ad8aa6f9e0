"""The step's linear-layer products one at a time, in fp64 (oracle; test
infrastructure only: see the package docstring).

Each function is the plain definition of one product the model runs:
  [arch]  page "安德烈·卡帕西推出nanochat：极简全栈AI训练项目..." (vpshk.cn),
          Q&A section "卡帕西亲自揭秘背后技术": linear layers without bias, a
          ReLU^2 MLP, an untied unembedding, a logit softcap.
  Muon    K. Jordan, "Muon: An optimizer for hidden layers in neural
          networks" (2024): the Newton-Schulz steps A = X X^T,
          B = b A + c A A, X <- a X + B X, written here as products with an
          optional scaled second term.
Operands are the exact values the GPU receives (already rounded to its
storage type); every product is formed in float64 with NumPy's matmul.

Pins (tests/test_oracle_products.py): the adjoint identities that make the
input- and weight-gradient products the derivatives of the forward product,
finite differences through ReLU^2, identity and zero weights, the softcap
bound and its small-logit limit, the Gram matrix's symmetry. No function here
is "parity unpinned".
"""

from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def xwt(a, w, aux=None):
    """y = a w^T (+ aux): a bias-free linear layer [arch] applied to the rows
    of a (w in the [out, in] layout); aux is the residual stream when the
    product feeds a residual add (the O and W2 products)."""
    y = _f64(a) @ _f64(w).T
    return y if aux is None else y + _f64(aux)


def xwt_relusq(a, w):
    """max(a w^T, 0)^2: the MLP's first product and its ReLU^2 activation [arch]."""
    return np.maximum(xwt(a, w), 0.0) ** 2


def dyw(dy, w):
    """dy w: the gradient of a w^T with respect to a, for upstream dy."""
    return _f64(dy) @ _f64(w)


def dyw_drelusq(dy, w, act):
    """(dy w) * 2 sqrt(act): the gradient through u -> max(u, 0)^2 given the
    stored activation act = max(u, 0)^2, since d/du max(u,0)^2 = 2 max(u,0)
    = 2 sqrt(act)."""
    return dyw(dy, w) * 2.0 * np.sqrt(_f64(act))


def dw(dy, x):
    """dy^T x: the gradient of x w^T with respect to w, summed over the rows
    (tokens)."""
    return _f64(dy).T @ _f64(x)


def softcap_logits(a, w, cap):
    """z' = cap * tanh(a w^T / cap): the softcapped logits of the untied
    unembedding [arch]."""
    return cap * np.tanh(xwt(a, w) / cap)


def tile_exp_sums(zc, tile):
    """Per row, the sum of exp(z') over each group of `tile` consecutive
    columns (the last group ragged): [M, ceil(N / tile)]."""
    zc = _f64(zc)
    n = zc.shape[1]
    return np.stack([np.exp(zc[:, j:j + tile]).sum(axis=1) for j in range(0, n, tile)], axis=1)


def axpby(a, w, alpha, beta=0.0, aux=None):
    """alpha a w^T (+ beta aux): a Newton-Schulz step as a product with a
    scaled second term (Muon)."""
    y = alpha * xwt(a, w)
    return y if aux is None else y + beta * _f64(aux)


def gram(a):
    """a^T a (Muon's A = X X^T for X stored as the transpose)."""
    a = _f64(a)
    return a.T @ a
