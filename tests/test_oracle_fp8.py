"""Pins of the FP8 oracle (oracle/fp8.py): the E4M3 rounding against torch's
float8_e4m3fn over every finite bf16 value in range, the format's closed
forms, and the scaled product against exact arithmetic."""

import numpy as np
import torch

from oracle import fp8


def test_e4m3_rounding_matches_torch_on_every_bf16_value():
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    v = bits.float()
    v = v[torch.isfinite(v) & (v.abs() <= 448)]
    want = v.to(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = fp8.e4m3(v.numpy().astype(np.float64))
    assert np.array_equal(got, want)


def test_e4m3_closed_forms():
    # every E4M3 value maps to itself: 2^-9 m (subnormals) and 2^(e-7) (1 + m/8)
    vals = [m * 2.0 ** -9 for m in range(8)] + [2.0 ** (e - 7) * (1 + m / 8) for e in range(1, 16)
                                                for m in range(8)]
    vals = np.array([x for x in vals if x <= 448])
    assert np.array_equal(fp8.e4m3(vals), vals) and np.array_equal(fp8.e4m3(-vals), -vals)
    # ties go to the even mantissa: 1 + 1/16 -> 1, 1 + 3/16 -> 1.25; 2^-10 -> 0
    assert list(fp8.e4m3(np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10]))) == [1.0, 1.25, 0.0, 2.0 ** -8]
    assert fp8.e4m3(np.array([448.0]))[0] == 448.0


def test_scaled_product():
    rng = np.random.default_rng(3)
    # operands already on the grid after scaling are exact: amax 448 gives inv = s = 1
    qx = fp8.e4m3(rng.uniform(-448, 448, (5, 16)))
    qx[0, 0] = 448.0
    qw = fp8.e4m3(rng.uniform(-448, 448, (7, 16)))
    qw[0, 0] = -448.0
    np.testing.assert_array_equal(fp8.fp8_matmul(qx, qw), qx @ qw.T)
    # a zero tensor has scale 1 and gives zeros
    assert np.all(fp8.fp8_matmul(np.zeros((2, 8)), qw[:, :8]) == 0)
    # scale invariance by a power of two, and the error bound: each rounding within 2^-4 relative
    x, w = rng.standard_normal((9, 64)), rng.standard_normal((11, 64))
    np.testing.assert_array_equal(fp8.fp8_matmul(x * 8, w), 8 * fp8.fp8_matmul(x, w))
    qv, s = fp8.quantize(x)
    assert np.all(np.abs(qv * s - x) <= 2.0 ** -4 * np.abs(x) + 2.0 ** -9 * s * 1.0001)
