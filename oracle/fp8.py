"""FP8 forward products (oracle): the block's four projections with both
operands rounded to FP8 E4M3 under one scale per tensor.

Test infrastructure only, like the rest of this package. NumPy.

Source: the page "nanochat：用 100 美元复刻 GPT-2 的 AI 训练实验台" (pomoai.com)
says the newest version of the project trains with FP8; no page gives a
recipe. Readings (also listed in the design notes):
  * Format: E4M3 with no infinities (1 sign bit, 4 exponent bits with bias 7,
    3 mantissa bits; largest finite value 448, subnormals down to 2^-9),
    round to nearest, ties to even.
  * Which products: the four forward projections of every block (QKV, O, W1,
    W2). The unembedding and every backward product stay in bf16; the
    backward treats the rounding as the identity (it uses the bf16
    activations and weights).
  * Scaling: one scale per tensor, from its largest magnitude a:
    inv = fp32(448 / a), y = clip(fp32(v * inv), -448, 448), q = E4M3(y), and
    the product is (q_x q_w^T) * s_x * s_w with s = fp32(a / 448); a = 0
    gives inv = s = 1. The arithmetic is stated in float32 so that the
    rounded codes are exactly defined.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3(y):
    """Round to the nearest E4M3 value (ties to even); |y| <= 448 expected."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    # spacing of the E4M3 grid around a: 2^-9 below 2^-6 (subnormals), else 2^(e - 3)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8)
    step = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (e - 3))
    q = np.rint(a / step) * step  # np.rint rounds half to even
    return np.sign(y) * np.minimum(q, E4M3_MAX)


def tensor_scale(v):
    """(inv, s) of the per-tensor scaling, in float32 arithmetic."""
    a = np.float32(np.max(np.abs(np.asarray(v, dtype=np.float32)))) if np.size(v) else np.float32(0)
    if a == 0:
        return np.float32(1), np.float32(1)
    return np.float32(448.0) / a, a / np.float32(448.0)


def quantize(v):
    """(codes as float64, dequantisation scale s) of a tensor."""
    inv, s = tensor_scale(v)
    y = np.clip(np.asarray(v, dtype=np.float32) * inv, np.float32(-448.0), np.float32(448.0))
    return e4m3(y.astype(np.float64)), float(s)


def fp8_matmul(x, w):
    """x [M, K] w [N, K]^T with both operands rounded to E4M3 under per-tensor scales."""
    qx, sx = quantize(x)
    qw, sw = quantize(w)
    return (qx @ qw.T) * (sx * sw)
