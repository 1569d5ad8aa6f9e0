"""The optimizer step (oracle): AdamW for the embedding and the unembedding,
Muon for every block matrix.

Test infrastructure only, like the rest of this package. Plain fp64 NumPy.

Sources:
  [arch]  page "安德烈·卡帕西推出nanochat..." (vpshk.cn), Q&A section
          "卡帕西亲自揭秘背后技术": the optimizer is Muon together with AdamW,
          after modded-nanoGPT.
  [pre]   page "100美元成本、8000行代码纯手搓克隆ChatGPT!..." (imeisheng.com),
          section "预训练": the learning rate is scaled by 1/sqrt(model dim);
          Muon updates the matrices, AdamW the embedding and the
          unembedding, and there are no other trainable parameters; the
          learning-rate multiplier "lrm" falls linearly to 0 near the end of
          training.
  [muon]  Muon's published definition (K. Jordan, "Muon: An optimizer for
          hidden layers in neural networks", 2024), which the pages name but
          do not define: SGD momentum with the Nesterov look-ahead; the
          update direction is the momentum-corrected gradient scaled to unit
          Frobenius norm and pushed towards the nearest semi-orthogonal
          matrix by five steps of the quintic Newton-Schulz map
          X <- a X + b (X X^T) X + c (X X^T)^2 X, (a, b, c) =
          (3.4445, -4.7750, 2.0315), run on the transpose when the matrix has
          more rows than columns; the step is scaled by max(1, rows/cols)^(1/2).
  [adamw] AdamW (Loshchilov and Hutter, decoupled weight decay) on Adam's
          bias-corrected moment estimates (Kingma and Ba).

Readings where the pages are silent (also listed in the design notes):
  * Hyperparameters (learning rates, betas, epsilon, momentum, weight decay)
    are inputs; the pages give only the 1/sqrt(dim) scaling and the linear
    end-of-run decay of the multiplier.
  * The multiplier is 1 until the last ``warmdown`` fraction of the steps
    and then falls linearly, reaching 0 after the last step.
  * Decoupled weight decay, where used, multiplies the weights by
    (1 - lr * wd) before the update. Muon's published form has none; it is
    an input here, 0 by default.
  * The optimizer keeps float32 master weights; the stored parameters are
    their rounding to the storage type after each step.
  * Wq, Wk and Wv are three matrices to Muon, as in the model's definition;
    packing them into one buffer for a single GEMM is a layout choice.
"""

from __future__ import annotations

import numpy as np

NS_COEFFS = (3.4445, -4.7750, 2.0315)
NS_STEPS = 5


def lr_multiplier(step: int, total_steps: int, warmdown: float) -> float:
    """lrm of step ``step`` (0-based) of ``total_steps``: 1, then linear to 0
    over the last ``warmdown`` fraction, 0 after the last step [pre]."""
    w = int(round(warmdown * total_steps))
    if w <= 0 or step < total_steps - w:
        return 1.0
    return max(0.0, (total_steps - step) / w)


def dim_scaled_lr(lr_ref: float, d_model: int, d_ref: int) -> float:
    """A learning rate tuned at width d_ref, scaled by 1/sqrt(dim) [pre]."""
    return lr_ref * (d_ref / d_model) ** 0.5


def newton_schulz5(G: np.ndarray, steps: int = NS_STEPS, eps: float = 1e-7) -> np.ndarray:
    """[muon] the quintic Newton-Schulz orthogonalization of G (any 2-D shape)."""
    a, b, c = NS_COEFFS
    X = np.asarray(G, dtype=np.float64)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    X = X / (np.linalg.norm(X) + eps)
    for _ in range(steps):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X.T if tall else X


def muon_update(W, G, Mom, lr, momentum, nesterov=True, wd=0.0):
    """[muon] one Muon step of the matrix W [rows, cols] with gradient G and
    momentum buffer Mom. Returns (W', Mom')."""
    W = np.asarray(W, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    Mom = momentum * np.asarray(Mom, dtype=np.float64) + G
    U = G + momentum * Mom if nesterov else Mom
    O = newton_schulz5(U)
    scale = max(1.0, W.shape[0] / W.shape[1]) ** 0.5
    W = W * (1.0 - lr * wd) - lr * scale * O
    return W, Mom


def adamw_update(W, G, m, v, step, lr, beta1, beta2, eps, wd=0.0):
    """[adamw] one AdamW step; ``step`` counts from 1. Returns (W', m', v')."""
    W = np.asarray(W, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    m = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * G
    v = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * G * G
    mhat = m / (1.0 - beta1 ** step)
    vhat = v / (1.0 - beta2 ** step)
    W = W * (1.0 - lr * wd) - lr * mhat / (np.sqrt(vhat) + eps)
    return W, m, v


def init_state(params):
    """Optimizer state for a parameter dict shaped like ``synth.init_params``:
    fp64 master copies, Muon momentum for the block matrices, AdamW moments
    for the embedding and the unembedding."""
    st = {"master": {"wte": np.array(params["wte"], dtype=np.float64),
                     "wlm": np.array(params["wlm"], dtype=np.float64),
                     "layers": [{k: np.array(v, dtype=np.float64) for k, v in w.items()} for w in params["layers"]]},
          "mom": [{k: np.zeros_like(v, dtype=np.float64) for k, v in w.items()} for w in params["layers"]],
          "adam": {k: (np.zeros_like(params[k], dtype=np.float64), np.zeros_like(params[k], dtype=np.float64))
                   for k in ("wte", "wlm")}}
    return st


def opt_step(state, grads, step, hp):
    """One optimizer step over every tensor. ``grads`` is shaped like the
    params (``layers`` with wq, wk, wv, wo, w1, w2); each of the six is one
    matrix to Muon (the library packs wq, wk, wv into one buffer for its
    projection GEMM, which is a layout, not a different model). ``hp`` holds
    lr_matrix, lr_embed, lr_unembed (already multiplied by lrm), momentum,
    nesterov, beta1, beta2, eps, wd_matrix, wd_adam. ``step`` counts from 1.
    Returns the new state."""
    ms = state["master"]
    for name, lr in (("wte", hp["lr_embed"]), ("wlm", hp["lr_unembed"])):
        m, v = state["adam"][name]
        ms[name], m, v = adamw_update(ms[name], grads[name], m, v, step, lr, hp["beta1"], hp["beta2"], hp["eps"],
                                      hp.get("wd_adam", 0.0))
        state["adam"][name] = (m, v)
    for w, g, mo in zip(ms["layers"], grads["layers"], state["mom"]):
        for k in ("wq", "wk", "wv", "wo", "w1", "w2"):
            w[k], mo[k] = muon_update(w[k], g[k], mo[k], hp["lr_matrix"], hp["momentum"], hp.get("nesterov", True),
                                      hp.get("wd_matrix", 0.0))
    return state
