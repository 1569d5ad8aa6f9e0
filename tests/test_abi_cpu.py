"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every symbol the header declares, validates configurations, and rejects bad
arguments before queueing anything."""

import ctypes as C
import os
import re

import pytest

from dense_pretraining_amd import config as cfgmod
from dense_pretraining_amd import lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nc.h")

pytestmark = pytest.mark.skipif(not os.path.exists(lib.LIB_PATH), reason="libnc.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nc_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported():
    L = lib.load()
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n
    assert sorted(lib.EXPORTED) == names


def test_abi_version():
    assert lib.load().nc_abi_version() == 1


@pytest.mark.parametrize("cfg", [cfgmod.TINY, cfgmod.BLOCK_D20, cfgmod.DEPTH20, cfgmod.DEPTH30,
                                 cfgmod.TINY.with_(dtype="bf16")])
def test_named_configs_validate(cfg):
    assert lib.validate(cfg) == 0


@pytest.mark.parametrize("change,code", [
    (dict(n_head=3, n_kv_head=2), 2),       # H % G != 0
    (dict(d_model=0), 2),
    (dict(batch=-1), 2),
    (dict(head_dim=96), 5),
    (dict(d_model=100), 5),
    (dict(vocab=50257), 5),
    (dict(d_ff=100), 5),
    (dict(softcap=0.0), 2),
    (dict(depth=0), 2),
    (dict(batch=256, seq_len=2048), 5),     # 2^19 tokens: the logit panel stride exceeds 24 bits
])
def test_bad_configs_rejected(change, code):
    assert lib.validate(cfgmod.TINY.with_(**change)) == code


def test_param_layout_matches_formula():
    for cfg in (cfgmod.TINY, cfgmod.DEPTH20):
        offs, n = lib.param_layout(cfg)
        assert n == cfgmod.param_count(cfg)
        d, V = cfg.d_model, cfg.vocab
        assert offs[0] == 0 and offs[1] == V * d
        per = cfg.qkv_dim * d + d * cfg.n_head * cfg.head_dim + 2 * d * cfg.d_ff
        for l in range(cfg.depth):
            assert offs[1 + 4 * l] == V * d + l * per
        assert offs[-1] == n - V * d
        assert lib.query_sizes(cfg).n_params == n


def test_sizes_grow_with_batch():
    a = lib.query_sizes(cfgmod.DEPTH20.with_(batch=8))
    b = lib.query_sizes(cfgmod.DEPTH20)
    assert b.model_workspace > a.model_workspace > 0
    assert b.block_saved > a.block_saved
    # the depth-20 step fits an MI355X (288 GB) with room to spare
    assert b.model_workspace < 100e9


def test_workspace_size_agrees_with_query_sizes():
    for cfg in (cfgmod.TINY, cfgmod.DEPTH20):
        s = lib.query_sizes(cfg)
        assert lib.workspace_size(cfg) == (s.model_workspace, s.block_saved, s.scratch)
    L = lib.load()
    c = lib.to_nc_config(cfgmod.TINY)
    assert L.nc_workspace_size(C.byref(c), None, None, None) == 0
    bad = lib.to_nc_config(cfgmod.TINY.with_(head_dim=96))
    assert L.nc_workspace_size(C.byref(bad), None, None, None) != 0


def _fake(addr):
    return C.c_void_p(addr)


def test_null_and_misaligned_pointers_rejected_before_launch():
    L = lib.load()
    c = lib.to_nc_config(cfgmod.TINY)
    ok = _fake(0x100000)
    bad = _fake(0x100001)
    assert L.nc_embed_fwd(C.byref(c), None, ok, ok, ok, ok, None) == 1
    assert L.nc_embed_fwd(C.byref(c), ok, ok, bad, ok, ok, None) == 3
    assert L.nc_clear_status(None, None) == 1
    assert L.nc_clear_status(bad, None) == 3
    f = C.c_float(1.0)
    assert L.nc_lmhead_softcap_xent_bwd(C.byref(c), ok, ok, ok, ok, f, ok, None, 0, ok, None) == 1
    bp = lib.NcBlockParams(0x100000, 0x100000, 0x100000, 0x100000)
    assert L.nc_block_fwd(C.byref(c), C.byref(bp), ok, ok, ok, ok, None) == 1  # x_in == x_out
    bp0 = lib.NcBlockParams(0x100000, None, 0x100000, 0x100000)
    assert L.nc_block_fwd(C.byref(c), C.byref(bp0), ok, _fake(0x200000), ok, ok, None) == 1


def test_small_workspace_rejected():
    L = lib.load()
    c = lib.to_nc_config(cfgmod.TINY)
    need = lib.query_sizes(cfgmod.TINY).model_workspace
    ok = _fake(0x100000)
    r = L.nc_model_loss_and_grad(C.byref(c), ok, ok, ok, ok, ok, C.c_float(1.0), 0, ok, need - 1, None)
    assert r == 4


def test_status_strings():
    L = lib.load()
    assert L.nc_status_str(0) == b"ok"
    assert L.nc_status_str(4) == b"workspace too small"
    assert L.nc_status_str(99) == b"unknown status"


def test_inference_arguments_checked_before_launch():
    L = lib.load()
    cfg = cfgmod.TINY.with_(seq_len=32)
    c = lib.to_nc_config(cfg)
    sz = lib.infer_query_sizes(cfg)
    # cache: [depth][2][batch][seq_len][G*D] in the storage dtype
    es = 2 if cfg.dtype == "bf16" else 4
    assert sz.cache == cfg.depth * 2 * cfg.batch * cfg.seq_len * cfg.n_kv_head * cfg.head_dim * es
    assert sz.workspace > 0
    ok, bad = _fake(0x100000), _fake(0x100001)
    W = sz.workspace
    assert L.nc_prefill(C.byref(c), ok, None, 4, ok, ok, ok, W, None) == 1
    assert L.nc_prefill(C.byref(c), ok, ok, 0, ok, ok, ok, W, None) == 2          # empty prompt
    assert L.nc_prefill(C.byref(c), ok, ok, 33, ok, ok, ok, W, None) == 2         # beyond the capacity
    assert L.nc_prefill(C.byref(c), ok, ok, 4, bad, ok, ok, W, None) == 3
    assert L.nc_prefill(C.byref(c), ok, ok, 4, ok, ok, ok, W - 1, None) == 4
    assert L.nc_decode_step(C.byref(c), ok, ok, 0, ok, ok, ok, W, None) == 2      # nothing cached yet
    assert L.nc_decode_step(C.byref(c), ok, ok, 32, ok, ok, ok, W, None) == 2     # cache full
    assert L.nc_decode_step(C.byref(c), ok, None, 5, ok, ok, ok, W, None) == 1
    assert L.nc_decode_step(C.byref(c), ok, ok, 5, ok, ok, ok, W - 1, None) == 4
    # more than 32 query heads per KV head is not implemented by the decode attention
    assert L.nc_infer_query_sizes(C.byref(lib.to_nc_config(cfg.with_(n_head=32, d_model=256))),
                                  C.byref(lib.NcInferSizes())) == 0
    wide = cfg.with_(n_head=64, d_model=256)
    assert L.nc_infer_query_sizes(C.byref(lib.to_nc_config(wide)), C.byref(lib.NcInferSizes())) == 5


def test_optimizer_arguments_checked_before_launch():
    L = lib.load()
    cfg = cfgmod.TINY
    c = lib.to_nc_config(cfg)
    sz = lib.opt_query_sizes(cfg)
    _, n = lib.param_layout(cfg)
    # master [n] + s1 [n] + s2 [2 V d], all float32
    assert sz.state == 4 * (2 * n + 2 * cfg.vocab * cfg.d_model)
    assert sz.workspace > 0
    ok, bad = _fake(0x100000), _fake(0x100001)
    W = sz.workspace
    good = lib.opt_hparams(0.02, 0.3, 0.004, 1)
    assert L.nc_opt_step(C.byref(c), None, ok, ok, ok, ok, W, None) == 1
    for field, value in [("lr_matrix", -1.0), ("lr_embed", float("nan")), ("momentum", 1.0), ("beta1", 1.0),
                         ("beta2", -0.1), ("eps", 0.0), ("wd_matrix", -0.5), ("step", 0), ("nesterov", 2)]:
        hp = lib.opt_hparams(0.02, 0.3, 0.004, 1)
        setattr(hp, field, value)
        assert L.nc_opt_step(C.byref(c), C.byref(hp), ok, ok, ok, ok, W, None) == 1, field
    assert L.nc_opt_step(C.byref(c), C.byref(good), ok, None, ok, ok, W, None) == 1
    assert L.nc_opt_step(C.byref(c), C.byref(good), ok, ok, bad, ok, W, None) == 3
    assert L.nc_opt_step(C.byref(c), C.byref(good), ok, ok, ok, ok, W - 1, None) == 4
    assert L.nc_opt_init(C.byref(c), None, ok, None) == 1
    assert L.nc_opt_init(C.byref(c), ok, bad, None) == 3
    # the optimizer needs the layers: depth 0 is a shape error
    assert L.nc_opt_query_sizes(C.byref(lib.to_nc_config(cfg.with_(depth=0))), C.byref(lib.NcOptSizes())) == 2
