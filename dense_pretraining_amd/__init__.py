"""MI355X-native nanochat pretraining step: a C-ABI HIP library and its binding.

Importing the package is cheap; the HIP library is loaded on first use by
``dense_pretraining_amd.lib`` and loading fails loudly when it is missing.
"""

from .config import Config, DEPTH20, DEPTH30, BLOCK_D20, TINY  # noqa: F401
