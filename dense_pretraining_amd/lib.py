"""ctypes binding of libnc.so: the same entry points as include/nc.h.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI. Torch tensors provide device memory; their data
pointers and the current HIP stream are passed through unchanged. Loading
fails loudly when the library has not been built.
"""

from __future__ import annotations

import ctypes as C
import os

import torch

from .config import Config, NC_BF16, NC_F32

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnc.so")

NC_OK = 0
# storage modes of nc_config.dtype: bf16, float32 (check mode), bf16 with FP8 E4M3 forward block products
_DTYPES = {"bf16": 0, "f32": 1, "bf16_fp8": 2}
STATUS_NAMES = {
    0: "NC_OK", 1: "NC_ERR_INVALID_ARG", 2: "NC_ERR_SHAPE", 3: "NC_ERR_ALIGN", 4: "NC_ERR_WORKSPACE",
    5: "NC_ERR_UNSUPPORTED", 6: "NC_ERR_HIP", 7: "NC_ERR_DEVICE_DATA",
}
STATUS_BAD_TOKEN = 0x1
STATUS_BAD_TARGET = 0x2
STATUS_NONFINITE_LOSS = 0x4
STATUS_NO_TARGETS = 0x8

EXPORTED = [
    "nc_abi_version", "nc_status_str", "nc_last_hip_error", "nc_validate", "nc_param_layout",
    "nc_query_sizes", "nc_workspace_size", "nc_read_status", "nc_clear_status", "nc_embed_fwd", "nc_embed_bwd",
    "nc_block_fwd", "nc_block_bwd", "nc_lmhead_softcap_xent_fwd", "nc_lmhead_softcap_xent_bwd",
    "nc_model_loss_and_grad", "nc_infer_query_sizes", "nc_prefill", "nc_decode_step", "nc_opt_query_sizes",
    "nc_opt_init", "nc_opt_step", "nc_profile_enable", "nc_profile_only", "nc_profile_summary",
    "nc_gemm_scratch_size", "nc_gemm", "nc_decode_step_noalloc",
]


class NcError(RuntimeError):
    def __init__(self, code, where, detail=""):
        self.code = code
        msg = f"{where}: {STATUS_NAMES.get(code, code)}"
        if detail:
            msg += f" ({detail})"
        super().__init__(msg)


class NcConfig(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("depth", "d_model", "n_head", "head_dim", "n_kv_head", "d_ff",
                                         "vocab", "batch", "seq_len")] + [
        ("softcap", C.c_float), ("rope_base", C.c_float), ("norm_eps", C.c_float), ("dtype", C.c_int32)]


class NcBlockParams(C.Structure):
    _fields_ = [("wqkv", C.c_void_p), ("wo", C.c_void_p), ("w1", C.c_void_p), ("w2", C.c_void_p)]


class NcBlockGrads(C.Structure):
    _fields_ = [("wqkv", C.c_void_p), ("wo", C.c_void_p), ("w1", C.c_void_p), ("w2", C.c_void_p)]


class NcSizes(C.Structure):
    _fields_ = [("block_saved", C.c_size_t), ("lmhead_saved", C.c_size_t), ("scratch", C.c_size_t),
                ("model_workspace", C.c_size_t), ("n_params", C.c_size_t)]


class NcInferSizes(C.Structure):
    _fields_ = [("cache", C.c_size_t), ("workspace", C.c_size_t)]


class NcOptHparams(C.Structure):
    _fields_ = [("lr_matrix", C.c_float), ("lr_embed", C.c_float), ("lr_unembed", C.c_float),
                ("momentum", C.c_float), ("nesterov", C.c_int32), ("beta1", C.c_float), ("beta2", C.c_float),
                ("eps", C.c_float), ("wd_matrix", C.c_float), ("wd_adam", C.c_float), ("step", C.c_int32)]


class NcGemmArgs(C.Structure):
    _fields_ = [("kind", C.c_int32), ("dtype", C.c_int32), ("M", C.c_int32), ("N", C.c_int32), ("K", C.c_int32),
                ("a", C.c_void_p), ("b", C.c_void_p), ("aux", C.c_void_p), ("y", C.c_void_p), ("yf", C.c_void_p),
                ("a_panels", C.c_int32), ("accumulate", C.c_int32), ("alpha", C.c_float), ("beta", C.c_float),
                ("softcap", C.c_float)]


# nc_gemm_kind
GEMM_KINDS = {"xwt": 0, "xwt_relusq": 1, "dyw": 2, "dyw_drelusq": 3, "dw": 4, "softcap": 5, "axpby": 6, "gram": 7}


class NcOptSizes(C.Structure):
    _fields_ = [("state", C.c_size_t), ("workspace", C.c_size_t)]


_lib = None


def load(path=LIB_PATH):
    """Loads libnc.so once; raises if it is missing (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m dense_pretraining_amd.build`")
    lib = C.CDLL(path)
    P, I, F, S = C.c_void_p, C.c_int, C.c_float, C.c_size_t
    cfgp = C.POINTER(NcConfig)
    sig = {
        "nc_abi_version": ([], I),
        "nc_status_str": ([I], C.c_char_p),
        "nc_last_hip_error": ([], C.c_char_p),
        "nc_validate": ([cfgp], I),
        "nc_param_layout": ([cfgp, C.POINTER(S), S, C.POINTER(S)], I),
        "nc_query_sizes": ([cfgp, C.POINTER(NcSizes)], I),
        "nc_workspace_size": ([cfgp, C.POINTER(S), C.POINTER(S), C.POINTER(S)], I),
        "nc_read_status": ([P, C.POINTER(C.c_uint32), P], I),
        "nc_clear_status": ([P, P], I),
        "nc_embed_fwd": ([cfgp, P, P, P, P, P, P], I),
        "nc_embed_bwd": ([cfgp, P, P, P, P, P, I, P, P], I),
        "nc_block_fwd": ([cfgp, C.POINTER(NcBlockParams), P, P, P, P, P], I),
        "nc_block_bwd": ([cfgp, C.POINTER(NcBlockParams), P, P, P, P, C.POINTER(NcBlockGrads), I, P, P], I),
        "nc_lmhead_softcap_xent_fwd": ([cfgp, P, P, P, P, P, P, P], I),
        "nc_lmhead_softcap_xent_bwd": ([cfgp, P, P, P, P, F, P, P, I, P, P], I),
        "nc_model_loss_and_grad": ([cfgp, P, P, P, P, P, F, I, P, S, P], I),
        "nc_infer_query_sizes": ([cfgp, C.POINTER(NcInferSizes)], I),
        "nc_prefill": ([cfgp, P, P, I, P, P, P, S, P], I),
        "nc_decode_step": ([cfgp, P, P, I, P, P, P, S, P], I),
        "nc_decode_step_noalloc": ([cfgp, P, P, I, P, P, P, P], I),
        "nc_opt_query_sizes": ([cfgp, C.POINTER(NcOptSizes)], I),
        "nc_opt_init": ([cfgp, P, P, P], I),
        "nc_opt_step": ([cfgp, C.POINTER(NcOptHparams), P, P, P, P, S, P], I),
        "nc_gemm_scratch_size": ([C.POINTER(NcGemmArgs), C.POINTER(S)], I),
        "nc_gemm": ([C.POINTER(NcGemmArgs), P, S, P], I),
        "nc_profile_enable": ([I], I),
        "nc_profile_only": ([C.c_char_p], I),
        "nc_profile_summary": ([C.c_char_p, S, C.POINTER(S)], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def to_nc_config(cfg: Config) -> NcConfig:
    return NcConfig(cfg.depth, cfg.d_model, cfg.n_head, cfg.head_dim, cfg.n_kv_head, cfg.d_ff, cfg.vocab,
                    cfg.batch, cfg.seq_len, cfg.softcap, cfg.rope_base, cfg.norm_eps,
                    _DTYPES[cfg.dtype])


def _check(code, where):
    if code != NC_OK:
        detail = ""
        if code == 6:
            detail = load().nc_last_hip_error().decode()
        raise NcError(code, where, detail)


def _p(t):
    """Device pointer of a tensor (None -> NULL)."""
    if t is None:
        return None
    return C.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def torch_dtype(cfg: Config):
    """Storage type of weights and activations."""
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


# ------------------------------------------------------------------ queries

def validate(cfg: Config):
    c = to_nc_config(cfg)
    return load().nc_validate(C.byref(c))


def query_sizes(cfg: Config) -> NcSizes:
    c = to_nc_config(cfg)
    s = NcSizes()
    _check(load().nc_query_sizes(C.byref(c), C.byref(s)), "nc_query_sizes")
    return s


def workspace_size(cfg: Config):
    """(model workspace, one block's saved, scratch) bytes."""
    c = to_nc_config(cfg)
    out = [C.c_size_t() for _ in range(3)]
    _check(load().nc_workspace_size(C.byref(c), *[C.byref(o) for o in out]), "nc_workspace_size")
    return tuple(o.value for o in out)


def param_layout(cfg: Config):
    c = to_nc_config(cfg)
    n = 2 + 4 * cfg.depth
    offs = (C.c_size_t * n)()
    total = C.c_size_t()
    _check(load().nc_param_layout(C.byref(c), offs, n, C.byref(total)), "nc_param_layout")
    return list(offs), total.value


def read_status(scratch, stream=None):
    """Returns the device status bits (synchronises the stream)."""
    flags = C.c_uint32()
    code = load().nc_read_status(_p(scratch), C.byref(flags), _stream(stream))
    if code not in (NC_OK, 7):
        _check(code, "nc_read_status")
    return flags.value


def clear_status(scratch, stream=None):
    _check(load().nc_clear_status(_p(scratch), _stream(stream)), "nc_clear_status")


def alloc_bytes(n, device="cuda"):
    """A 256-byte aligned device buffer of n bytes (torch's caching allocator)."""
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=device)


def new_scratch(cfg: Config, device="cuda"):
    s = alloc_bytes(query_sizes(cfg).scratch, device)
    clear_status(s)
    return s


# ------------------------------------------------------------------ entry points

def embed_fwd(cfg, idx, wte, x0, r0, scratch, stream=None):
    c = to_nc_config(cfg)
    _check(load().nc_embed_fwd(C.byref(c), _p(idx), _p(wte), _p(x0), _p(r0), _p(scratch), _stream(stream)),
           "nc_embed_fwd")


def embed_bwd(cfg, idx, x0, r0, dx0, dwte, scratch, accumulate=False, stream=None):
    c = to_nc_config(cfg)
    _check(load().nc_embed_bwd(C.byref(c), _p(idx), _p(x0), _p(r0), _p(dx0), _p(dwte), int(accumulate),
                               _p(scratch), _stream(stream)), "nc_embed_bwd")


def _bp(w):
    return NcBlockParams(w["wqkv"].data_ptr(), w["wo"].data_ptr(), w["w1"].data_ptr(), w["w2"].data_ptr())


def block_fwd(cfg, w, x_in, x_out, saved, scratch, stream=None):
    c = to_nc_config(cfg)
    bp = _bp(w)
    _check(load().nc_block_fwd(C.byref(c), C.byref(bp), _p(x_in), _p(x_out), _p(saved), _p(scratch),
                               _stream(stream)), "nc_block_fwd")


def block_bwd(cfg, w, x_in, saved, dx_out, dx_in, grads, scratch, accumulate=False, stream=None):
    c = to_nc_config(cfg)
    bp = _bp(w)
    bg = NcBlockGrads(grads["wqkv"].data_ptr(), grads["wo"].data_ptr(), grads["w1"].data_ptr(),
                      grads["w2"].data_ptr())
    _check(load().nc_block_bwd(C.byref(c), C.byref(bp), _p(x_in), _p(saved), _p(dx_out), _p(dx_in),
                               C.byref(bg), int(accumulate), _p(scratch), _stream(stream)), "nc_block_bwd")


def lmhead_softcap_xent_fwd(cfg, x, wlm, targets, loss, saved, scratch, stream=None):
    c = to_nc_config(cfg)
    _check(load().nc_lmhead_softcap_xent_fwd(C.byref(c), _p(x), _p(wlm), _p(targets), _p(loss), _p(saved),
                                             _p(scratch), _stream(stream)), "nc_lmhead_softcap_xent_fwd")


def lmhead_softcap_xent_bwd(cfg, x, wlm, targets, saved, dloss, dx, dwlm, scratch, accumulate=False,
                            stream=None):
    c = to_nc_config(cfg)
    _check(load().nc_lmhead_softcap_xent_bwd(C.byref(c), _p(x), _p(wlm), _p(targets), _p(saved),
                                             float(dloss), _p(dx), _p(dwlm), int(accumulate), _p(scratch),
                                             _stream(stream)), "nc_lmhead_softcap_xent_bwd")


def model_loss_and_grad(cfg, params, idx, targets, loss, grads, workspace, dloss=1.0, accumulate=False,
                        stream=None):
    c = to_nc_config(cfg)
    _check(load().nc_model_loss_and_grad(C.byref(c), _p(params), _p(idx), _p(targets), _p(loss), _p(grads),
                                         float(dloss), int(accumulate), _p(workspace),
                                         workspace.numel() * workspace.element_size(), _stream(stream)),
           "nc_model_loss_and_grad")


# ------------------------------------------------------------------ products

def gemm_args(kind, dtype, M, N, K, a, b=None, y=None, yf=None, aux=None, a_panels=False, accumulate=False,
              alpha=1.0, beta=0.0, softcap=0.0) -> NcGemmArgs:
    """nc_gemm_args for one product (kind: a key of GEMM_KINDS; dtype 'bf16' or 'f32')."""
    return NcGemmArgs(GEMM_KINDS[kind], _DTYPES[dtype], int(M), int(N), int(K), _p(a), _p(b), _p(aux), _p(y),
                      _p(yf), int(bool(a_panels)), int(bool(accumulate)), float(alpha), float(beta), float(softcap))


def gemm_scratch_size(args: NcGemmArgs) -> int:
    n = C.c_size_t()
    _check(load().nc_gemm_scratch_size(C.byref(args), C.byref(n)), "nc_gemm_scratch_size")
    return n.value


def gemm(args: NcGemmArgs, scratch=None, stream=None):
    nbytes = scratch.numel() * scratch.element_size() if scratch is not None else 0
    _check(load().nc_gemm(C.byref(args), _p(scratch), nbytes, _stream(stream)), "nc_gemm")


# ------------------------------------------------------------------ tracing

def profile_enable(on=True):
    _check(load().nc_profile_enable(int(on)), "nc_profile_enable")


def profile_only(kernel_class=None):
    """Record only the launches of one kernel class (None: all of them)."""
    _check(load().nc_profile_only(kernel_class.encode() if kernel_class else None), "nc_profile_only")


def profile_summary():
    """Per-kernel {launches, ms, flops, bytes} of the launches recorded while
    profiling was on (waits for them)."""
    import json
    need = C.c_size_t()
    load().nc_profile_summary(None, 0, C.byref(need))
    buf = C.create_string_buffer(need.value)
    _check(load().nc_profile_summary(buf, need.value, C.byref(need)), "nc_profile_summary")
    return json.loads(buf.value.decode())


# ------------------------------------------------------------------ inference

def infer_query_sizes(cfg: Config) -> NcInferSizes:
    c = to_nc_config(cfg)
    s = NcInferSizes()
    _check(load().nc_infer_query_sizes(C.byref(c), C.byref(s)), "nc_infer_query_sizes")
    return s


def prefill(cfg, params, idx, n_prompt, cache, next_tok, workspace, stream=None):
    c = to_nc_config(cfg)
    _check(load().nc_prefill(C.byref(c), _p(params), _p(idx), int(n_prompt), _p(cache), _p(next_tok),
                             _p(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "nc_prefill")


def decode_step(cfg, params, tok, pos, cache, next_tok, workspace, stream=None):
    c = to_nc_config(cfg)
    _check(load().nc_decode_step(C.byref(c), _p(params), _p(tok), int(pos), _p(cache), _p(next_tok),
                                 _p(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "nc_decode_step")


def decode_step_noalloc(cfg, params, tok, pos, cache, next_tok, status=None, stream=None):
    """nc_decode_step with the library's static scratch (no workspace);
    status: an optional device uint32 tensor the bad-token bit is OR-ed into."""
    c = to_nc_config(cfg)
    _check(load().nc_decode_step_noalloc(C.byref(c), _p(params), _p(tok), int(pos), _p(cache), _p(next_tok),
                                         _p(status), _stream(stream)), "nc_decode_step_noalloc")


# ------------------------------------------------------------------ optimizer

def opt_hparams(lr_matrix, lr_embed, lr_unembed, step, momentum=0.95, nesterov=True, beta1=0.8, beta2=0.95,
                eps=1e-10, wd_matrix=0.0, wd_adam=0.0) -> NcOptHparams:
    return NcOptHparams(lr_matrix, lr_embed, lr_unembed, momentum, 1 if nesterov else 0, beta1, beta2, eps,
                        wd_matrix, wd_adam, int(step))


def opt_query_sizes(cfg: Config) -> NcOptSizes:
    c = to_nc_config(cfg)
    s = NcOptSizes()
    _check(load().nc_opt_query_sizes(C.byref(c), C.byref(s)), "nc_opt_query_sizes")
    return s


def opt_init(cfg, params, state, stream=None):
    c = to_nc_config(cfg)
    _check(load().nc_opt_init(C.byref(c), _p(params), _p(state), _stream(stream)), "nc_opt_init")


def opt_step(cfg, hp: NcOptHparams, params, grads, state, workspace, stream=None):
    c = to_nc_config(cfg)
    _check(load().nc_opt_step(C.byref(c), C.byref(hp), _p(params), _p(grads), _p(state), _p(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream)), "nc_opt_step")
