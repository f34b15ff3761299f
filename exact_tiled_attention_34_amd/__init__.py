"""Exact tiled (FlashAttention-2 style) attention for MI355X / gfx950.

The computation lives in ``libfa2.so`` (hand-written HIP kernels behind the C
ABI in ``include/fa2.h``); ``fa2`` is its thin ctypes binding.  Importing this
package does not load the library; the first call does, and fails loudly if
it has not been built (``python -m exact_tiled_attention_34_amd.build``).
"""

from . import fa2
from .fa2 import fwd, bwd, bwd_workspace_bytes, FA2Error

__all__ = ["fa2", "fwd", "bwd", "bwd_workspace_bytes", "FA2Error"]

# Submodules that need PyTorch autograd are imported explicitly:
#   from exact_tiled_attention_34_amd.autograd import attention
#   from exact_tiled_attention_34_amd import gpt_block
