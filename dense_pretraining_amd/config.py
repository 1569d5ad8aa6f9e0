"""Model/batch configuration and the bookkeeping formulas (params, FLOPs).

The shape knobs follow the pretraining walkthrough on imeisheng.com (section
"预训练": depth 20 has 1280 channels and 10 heads of 128) and the single-knob
scaling it describes (width and heads follow from depth): d_model = 64*depth,
n_head = d_model/128, head_dim = 128, d_ff = 4*d_model; multi-query attention
(one KV head) from the architecture list on vpshk.cn.
"""

from __future__ import annotations

from dataclasses import dataclass, replace

NC_BF16 = 0
NC_F32 = 1


@dataclass(frozen=True)
class Config:
    depth: int
    d_model: int
    n_head: int
    head_dim: int
    n_kv_head: int
    d_ff: int
    vocab: int
    batch: int
    seq_len: int
    softcap: float = 15.0
    rope_base: float = 10000.0
    norm_eps: float = 1e-6
    # storage of weights and activations: "bf16", "f32" (check mode), or "bf16_fp8"
    # (bf16 storage, the block's forward products in FP8 E4M3)
    dtype: str = "bf16"

    @staticmethod
    def from_depth(depth, batch=32, seq_len=2048, vocab=65536, n_kv_head=1, dtype="bf16"):
        d = 64 * depth
        return Config(depth=depth, d_model=d, n_head=d // 128, head_dim=128, n_kv_head=n_kv_head,
                      d_ff=4 * d, vocab=vocab, batch=batch, seq_len=seq_len, dtype=dtype)

    def with_(self, **kw):
        return replace(self, **kw)

    @property
    def tokens(self):
        return self.batch * self.seq_len

    @property
    def qkv_dim(self):
        return (self.n_head + 2 * self.n_kv_head) * self.head_dim


# Named workloads (the tiny oracle model, one block at the real shape, the
# depth-20 and depth-30 models).
TINY = Config(depth=2, d_model=128, n_head=2, head_dim=64, n_kv_head=1, d_ff=512,
              vocab=512, batch=2, seq_len=64, dtype="f32")
BLOCK_D20 = Config.from_depth(20).with_(depth=1)
DEPTH20 = Config.from_depth(20)
DEPTH30 = Config.from_depth(30, batch=16)


def matmul_params(cfg):
    """Parameters that take part in a matmul per token (embedding excluded:
    it is a row gather)."""
    d, F, V = cfg.d_model, cfg.d_ff, cfg.vocab
    per_layer = d * cfg.qkv_dim + cfg.n_head * cfg.head_dim * d + 2 * d * F
    return cfg.depth * per_layer + V * d


def param_count(cfg):
    """All trainable parameters: Wte, per-layer matrices, Wlm."""
    return matmul_params(cfg) + cfg.vocab * cfg.d_model


def flops_per_token(cfg, convention="causal"):
    """Training (forward + backward) model FLOPs per token.

    6 * matmul params, plus attention: the score and value products cost
    2 * 2 * H * D * context per token forward, three times that with the
    backward. 'causal' counts the average context T/2, 'palm' the full T."""
    ctx = cfg.seq_len / 2 if convention == "causal" else cfg.seq_len
    attn = 3 * 4 * cfg.depth * cfg.n_head * cfg.head_dim * ctx
    return 6 * matmul_params(cfg) + attn


MI355X_BF16_DENSE_PEAK = 2.5166e15  # 256 CU x 2.4 GHz x 4096 flop/clk
MI355X_FP32_MFMA_PEAK = 157.3e12
MI355X_FP8_DENSE_PEAK = 5.0332e15  # twice the bf16 rate
MI355X_HBM_PEAK = 8.0e12
