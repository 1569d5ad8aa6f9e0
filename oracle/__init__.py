"""fp64 CPU oracle of one nanochat pretraining step (test infrastructure only).

This package is the slow, plainly written reference that the GPU library is
checked against. It is test infrastructure: only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it. The product path
(the HIP library and its Python binding) never imports, calls or links
anything here, and this package imports nothing from the product.

Every function follows the architecture list on the page "nanochat ...
卡帕西亲自揭秘背后技术" (vpshk.cn, Q&A section, architecture bullets) and the
pretraining walkthrough on imeisheng.com (section "预训练"). Where the pages
are silent, the reading adopted is stated beside the code.

Parity pins: every function here is pinned by tests in ``tests/test_oracle_*``
to closed forms, invariants, finite differences or an independent library
routine; no function is "parity unpinned".
"""

from .model import (  # noqa: F401
    Cfg,
    rope_tables,
    rms_norm,
    rms_norm_bwd,
    rope_apply,
    rope_apply_t,
    attention_fwd,
    attention_bwd,
    embed_fwd,
    embed_bwd,
    block_fwd,
    block_bwd,
    lmhead_softcap_xent_fwd,
    lmhead_softcap_xent_bwd,
    model_loss_and_grad,
    model_forward_logits,
)
from . import infer  # noqa: F401  (greedy generation with a key/value cache)
from . import optim  # noqa: F401  (the optimizer step: Muon and AdamW)
from . import fp8  # noqa: F401  (FP8 E4M3 forward products)
