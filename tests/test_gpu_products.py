"""Each linear-layer product of the step through nc_gemm (the kernels and
epilogues the block, head and optimizer launch), against the fp64 product of
the same rounded inputs (oracle/products.py), element by element.

Tolerance, derived from the arithmetic rather than the model-level bar:
  * float32 accumulation: a k-sum of n terms carries at most about
    n * 2^-24 * sum_k |a_k b_k|. The MFMA adds 16 (bf16) or 2 (float32)
    products per instruction into a chain of K/16 (K/2) instructions, a split
    reduction adds one term per split: n = K/16 + 48 (K/2 + 48), doubled.
  * one rounding of the output: 2^-8 of it in bf16 (8-bit significand, round
    to nearest even), 2^-24 in float32.
  * the epilogue's own float32 arithmetic: squares and square roots
    (relative 2^-22), the softcap's hardware exp2 and reciprocal (absolute
    2^-16 * c around z' = 0, where c - 2c/(2^x + 1) cancels).
Every element must lie within that bound (a worst case, linear in n), and the
relative Frobenius error must stay below the output rounding (2^-8 bf16, 1e-5
float32) plus 4 * 2^-24 * sqrt(n), the typical growth of n independent
roundings with a wide margin. A k-tile of 32 dropped at K = 1280 moves a product by
about 16 % of its RMS, far outside both.

Shapes cover the three operand layouts (NT forward, NN input gradient, TN
weight gradient), ragged M, N and K tails against the 256 x 256 x 32 tile,
K = 1280 and 5120, a weight gradient reduced over 65,536 tokens in 16 splits,
the column-panelled logit operand, accumulate, and the full-size depth-20
products in the benchmark's launch configuration (sampled rows)."""

import numpy as np
import pytest
import torch

from oracle import products as P
from dense_pretraining_amd import lib, synth

pytestmark = pytest.mark.gpu

U_OUT = {"bf16": 2.0 ** -8, "f32": 2.0 ** -24}
FRO = {"bf16": 2.0 ** -8, "f32": 1e-5}
KPER = {"bf16": 16, "f32": 2}
PANEL = 32


def _rand(shape, dt, seed, scale=1.0):
    return synth.normal(shape, scale, np.random.default_rng(seed), dt, np.float32)


def _dev(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda",
                                                                         torch.bfloat16 if dt == "bf16" else
                                                                         torch.float32)


def _host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _acc_bound(k, absprod, dt):
    return 2.0 * (k / KPER[dt] + 48) * 2.0 ** -24 * absprod


def _check(got, ref, bound, dt, name, k, in_dt, fro_extra=0.0):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), name
    err = np.abs(got - ref)
    lim = U_OUT[dt] * 1.01 * np.abs(ref) + 1.01 * bound
    bad = err > lim
    assert not bad.any(), (f"{name}: {bad.sum()} elements outside the bound, worst excess "
                           f"{np.max(err - lim):.3e} at {np.unravel_index(np.argmax(err - lim), err.shape)}")
    # rounding errors of a chain of n additions grow like sqrt(n) on average,
    # relative to the result: 4 * 2^-24 * sqrt(n) leaves a wide margin
    den = np.linalg.norm(ref)
    rel = np.linalg.norm(got - ref) / den if den > 0 else np.linalg.norm(got)
    lim_f = FRO[dt] + 4 * 2.0 ** -24 * np.sqrt(k / KPER[in_dt] + 48) + fro_extra
    assert rel <= lim_f, f"{name}: relative Frobenius error {rel:.3e} > {lim_f:.3e}"
    return rel


def to_panels(a):
    """[M, N] -> the column-panel layout (N/32 panels of [M, 32]), flat."""
    M, N = a.shape
    n_p = (N + PANEL - 1) // PANEL
    out = np.zeros((n_p, M, PANEL), dtype=a.dtype)
    for p in range(n_p):
        c = a[:, p * PANEL:(p + 1) * PANEL]
        out[p, :, :c.shape[1]] = c
    return out.reshape(-1)


def from_panels(flat, M, N):
    n_p = (N + PANEL - 1) // PANEL
    x = flat[: n_p * M * PANEL].reshape(n_p, M, PANEL)
    return np.concatenate([x[p] for p in range(n_p)], axis=1)[:, :N]


def _run(args, scratch=None):
    lib.gemm(args, scratch)
    torch.cuda.synchronize()


DTS = ["bf16", "f32"]
# (M, N, K): ragged M against 256-row tiles, ragged N, K a multiple of 32 or not
NT_SHAPES = [(300, 264, 1280), (513, 520, 1288), (256, 512, 5120), (40, 8, 8)]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("M,N,K", NT_SHAPES)
def test_forward_products(dt, M, N, K):
    x, w, res = _rand((M, K), dt, 1), _rand((N, K), dt, 2, 1 / np.sqrt(K)), _rand((M, N), dt, 3)
    absp = np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T
    acc = _acc_bound(K, absp, dt)
    xd, wd, rd = _dev(x, dt), _dev(w, dt), _dev(res, dt)
    y = torch.empty(M, N, dtype=xd.dtype, device="cuda")
    _run(lib.gemm_args("xwt", dt, M, N, K, xd, wd, y))
    _check(_host(y), P.xwt(x, w), acc, dt, "x w^T", K, dt)
    _run(lib.gemm_args("xwt", dt, M, N, K, xd, wd, y, aux=rd))
    _check(_host(y), P.xwt(x, w, res), acc, dt, "x w^T + residual", K, dt)
    _run(lib.gemm_args("xwt_relusq", dt, M, N, K, xd, wd, y))
    u = P.xwt(x, w)
    _check(_host(y), P.xwt_relusq(x, w), 2 * np.maximum(u, 0) * acc + acc ** 2 + 2.0 ** -22 * u * u, dt,
           "max(x w^T, 0)^2", K, dt, 2.0 ** -21)
    _run(lib.gemm_args("axpby", dt, M, N, K, xd, wd, y, aux=rd, alpha=0.75, beta=-1.5))
    _check(_host(y), P.axpby(x, w, 0.75, -1.5, res), 0.75 * acc + 2.0 ** -23 * np.abs(res), dt, "axpby", K, dt,
           2.0 ** -21)


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("M,N,K", [(300, 1280, 264), (513, 1288, 520), (256, 5120, 256), (40, 8, 8)])
def test_input_gradient_products(dt, M, N, K):
    # y[M,K] = dy[M,N] w[N,K]: the weight read K-outer
    dy, w = _rand((M, N), dt, 4), _rand((N, K), dt, 5, 1 / np.sqrt(N))
    act = synth.round_to(np.maximum(_rand((M, K), dt, 6), 0) ** 2, dt, np.float32)
    absp = np.abs(dy.astype(np.float64)) @ np.abs(w.astype(np.float64))
    acc = _acc_bound(N, absp, dt)
    dyd, wd, ad = _dev(dy, dt), _dev(w, dt), _dev(act, dt)
    y = torch.empty(M, K, dtype=dyd.dtype, device="cuda")
    _run(lib.gemm_args("dyw", dt, M, N, K, dyd, wd, y))
    _check(_host(y), P.dyw(dy, w), acc, dt, "dy w", N, dt)
    _run(lib.gemm_args("dyw_drelusq", dt, M, N, K, dyd, wd, y, aux=ad))
    ref = P.dyw_drelusq(dy, w, act)
    _check(_host(y), ref, 2 * np.sqrt(act) * acc + 2.0 ** -22 * np.abs(ref), dt, "(dy w) 2 sqrt(act)", N, dt,
           2.0 ** -21)


def _dw_case(dt, M, N, K, seed, panels=False, accumulate=False, expect_split=None):
    dy, x = _rand((M, N), dt, seed), _rand((M, K), dt, seed + 1)
    dyd = _dev(to_panels(dy) if panels else dy, dt)
    xd = _dev(x, dt)
    out = torch.empty(N, K, dtype=torch.float32, device="cuda")
    init = _rand((N, K), "f32", seed + 2) if accumulate else None
    if accumulate:
        out.copy_(torch.from_numpy(init))
    args = lib.gemm_args("dw", dt, M, N, K, dyd, xd, yf=out, a_panels=panels, accumulate=accumulate)
    need = lib.gemm_scratch_size(args)
    if expect_split is not None:
        assert (need > 0) == expect_split, need
    scratch = lib.alloc_bytes(need) if need else None
    _run(args, scratch)
    absp = np.abs(dy.astype(np.float64)).T @ np.abs(x.astype(np.float64))
    ref = P.dw(dy, x)
    bound = _acc_bound(M, absp, dt)
    if accumulate:
        ref = ref + init
        bound = bound + 2.0 ** -23 * np.abs(ref)
    # the gradient is float32 whatever the operands' storage type
    return _check(_host(out), ref, bound, "f32", f"dy^T x {M}x{N}x{K}", M, dt, 2.0 ** -22 if accumulate else 0.0)


@pytest.mark.parametrize("dt", DTS)
def test_weight_gradient_products(dt):
    # ragged token count (one split), ragged N and K
    _dw_case(dt, 300, 264, 520, 10, expect_split=False)
    # 65,536 tokens over a small output: 16 splits of 4096, summed in a fixed order
    _dw_case(dt, 65536, 264, 256, 20, expect_split=True)
    # accumulate into an existing gradient, split and unsplit
    _dw_case(dt, 65536, 256, 264, 30, accumulate=True, expect_split=True)
    _dw_case(dt, 100, 256, 264, 40, accumulate=True, expect_split=False)
    # the logit gradient's column panels (ragged last panel: 520 = 16 * 32 + 8)
    _dw_case(dt, 1000, 520, 128, 50, panels=True)
    _dw_case(dt, 65536, 520, 64, 60, panels=True)


@pytest.mark.parametrize("dt", DTS)
def test_input_gradient_from_panelled_logits(dt):
    M, N, K = 700, 520, 264
    dz, w = _rand((M, N), dt, 70), _rand((N, K), dt, 71, 0.05)
    y = torch.empty(M, K, dtype=torch.bfloat16 if dt == "bf16" else torch.float32, device="cuda")
    _run(lib.gemm_args("dyw", dt, M, N, K, _dev(to_panels(dz), dt), _dev(w, dt), y, a_panels=True))
    absp = np.abs(dz.astype(np.float64)) @ np.abs(w.astype(np.float64))
    _check(_host(y), P.dyw(dz, w), _acc_bound(N, absp, dt), dt, "dz w (panels)", N, dt)


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("M,N,K,scale", [(300, 520, 256, 2.5), (257, 1000, 128, 40.0), (64, 8, 64, 0.0)])
def test_softcap_product(dt, M, N, K, scale):
    # scale 40: most |z| are several times c, deep in the softcap's saturation
    cap = 15.0
    x, w = _rand((M, K), dt, 80), _rand((N, K), dt, 81, scale / np.sqrt(K))
    tile = 256 if dt == "bf16" else 128
    n_t = (N + tile - 1) // tile
    z = torch.empty((N + PANEL - 1) // PANEL * PANEL * M, dtype=torch.bfloat16 if dt == "bf16" else torch.float32,
                    device="cuda")
    part = torch.empty(M, n_t, dtype=torch.float32, device="cuda")
    _run(lib.gemm_args("softcap", dt, M, N, K, _dev(x, dt), _dev(w, dt), z, yf=part, softcap=cap))
    ref = P.softcap_logits(x, w, cap)
    absp = np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T
    u = P.xwt(x, w)
    # d z'/dz = 1 - tanh^2 <= 1: the accumulation error passes through damped
    bound = _acc_bound(K, absp, dt) * (1 - np.tanh(u / cap) ** 2) + 2.0 ** -16 * cap
    zc = from_panels(_host(z), M, N)
    fro_abs = 2.0 ** -16 * cap * np.sqrt(ref.size) / max(np.linalg.norm(ref), 1e-30)
    _check(zc, ref, bound, dt, "c tanh(x w^T / c)", K, dt, fro_abs)
    assert np.all(np.abs(zc) <= cap)
    s_ref = P.tile_exp_sums(ref, tile)
    # exp(z') of the unrounded z': relative error about the absolute error of z'
    rel = np.abs(_host(part) - s_ref) / s_ref
    assert np.max(rel) <= 1e-4, np.max(rel)


@pytest.mark.parametrize("dt", DTS)
def test_gram_product(dt):
    M, K = 300, 264
    x = _rand((M, K), dt, 90, 0.1)
    y = torch.empty(K, K, dtype=torch.bfloat16 if dt == "bf16" else torch.float32, device="cuda")
    _run(lib.gemm_args("gram", dt, M, 0, K, _dev(x, dt), y=y))
    xa = np.abs(x.astype(np.float64))
    _check(_host(y), P.gram(x), _acc_bound(M, xa.T @ xa, dt), dt, "x^T x", M, dt)


def test_full_size_products_sampled_rows():
    """The depth-20 block's products at their benchmark shapes (65,536
    tokens, bf16, the same launches as the training step: W1 forward with
    ReLU^2, the dReLU^2 input gradient, dWo over 10 splits of 6,554 tokens,
    dW1 over 5), checked on sampled rows of each output."""
    dt = "bf16"
    M, d, F = 65536, 1280, 5120
    rows = np.random.default_rng(99).choice(M, 48, replace=False)
    rows = np.sort(np.concatenate([rows, [0, 255, 256, M - 1]]))
    h = _rand((M, d), dt, 100)
    w1 = _rand((F, d), dt, 101, 1 / np.sqrt(d))
    hd, w1d = _dev(h, dt), _dev(w1, dt)
    act = torch.empty(M, F, dtype=torch.bfloat16, device="cuda")
    _run(lib.gemm_args("xwt_relusq", dt, M, F, d, hd, w1d, act))
    u = P.xwt(h[rows], w1)
    acc = _acc_bound(d, np.abs(h[rows].astype(np.float64)) @ np.abs(w1.astype(np.float64)).T, dt)
    act_rows = _host(act[torch.from_numpy(rows).cuda()])
    _check(act_rows, np.maximum(u, 0) ** 2, 2 * np.maximum(u, 0) * acc + acc ** 2 + 2.0 ** -22 * u * u, dt,
           "W1 + ReLU^2 (65536 x 5120 x 1280)", d, dt, 2.0 ** -21)
    # input gradient through ReLU^2: du = (dx W2) 2 sqrt(act), K = d = 1280 reduction, output [M, F]
    dx = _rand((M, d), dt, 102)
    w2 = _rand((d, F), dt, 103, 1 / np.sqrt(F))
    du = torch.empty(M, F, dtype=torch.bfloat16, device="cuda")
    _run(lib.gemm_args("dyw_drelusq", dt, M, d, F, _dev(dx, dt), _dev(w2, dt), du, aux=act))
    ref = P.dyw_drelusq(dx[rows], w2, act_rows)
    acc = _acc_bound(d, np.abs(dx[rows].astype(np.float64)) @ np.abs(w2.astype(np.float64)), dt)
    _check(_host(du[torch.from_numpy(rows).cuda()]), ref, 2 * np.sqrt(act_rows) * acc + 2.0 ** -22 * np.abs(ref), dt,
           "dReLU^2 input gradient (65536 x 1280 -> 5120)", d, dt, 2.0 ** -21)
    del act, du
    # weight gradients over all 65,536 tokens, checked on sampled output rows
    for name, N, K, a_np, b_np in (("dWo", d, d, dx, h), ("dW1", F, d, None, h)):
        if a_np is None:
            a_np = _rand((M, F), dt, 104)
        out = torch.empty(N, K, dtype=torch.float32, device="cuda")
        ad, bd = _dev(a_np, dt), _dev(b_np, dt)
        args = lib.gemm_args("dw", dt, M, N, K, ad, bd, yf=out)
        need = lib.gemm_scratch_size(args)
        assert need > 0, f"{name}: expected a split reduction"
        _run(args, lib.alloc_bytes(need))
        orow = np.sort(np.random.default_rng(7).choice(N, 24, replace=False))
        ref = P.dw(a_np[:, orow], b_np)
        absp = np.abs(a_np[:, orow].astype(np.float64)).T @ np.abs(b_np.astype(np.float64))
        _check(_host(out)[orow], ref, _acc_bound(M, absp, dt), "f32", f"{name} (65536 tokens, split)", M, dt)
        del ad, bd
