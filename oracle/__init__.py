"""CPU oracle for exact softmax attention — TEST INFRASTRUCTURE, not product code.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import, call or run anything in this package.  The HIP library and its
Python binding never import it and share no code with it: no kernels, headers,
helpers, constants or pre/post-processing.

Contents
--------
``attention``  the plain definition of softmax attention and of its analytic
               gradient, materialised per (batch, head) in float64.
``tiled``      a float64 model of the tile-by-tile online-softmax algorithm,
               used only to show that tiling reaches exactly the plain result.
``bf16``       decoding of bfloat16 and float16 bit patterns to float64 (exact).

Pins: every function here is checked against facts fixed by the mathematics
(closed forms, finite differences, invariants, a library special case) in
``tests/test_oracle.py``; nothing is "parity unpinned".
"""

from .bf16 import bf16_bits_to_float64, fp16_bits_to_float64, bits_to_float64
from .attention import (
    causal_offset,
    scores,
    softmax_rows,
    forward,
    backward,
    forward_head,
    backward_head,
    forward_rows,
    row_stats,
    backward_rows,
    backward_cols,
)
from .tiled import tiled_forward_head, tiled_backward_head

__all__ = [
    "bf16_bits_to_float64",
    "fp16_bits_to_float64",
    "bits_to_float64",
    "causal_offset",
    "scores",
    "softmax_rows",
    "forward",
    "backward",
    "forward_head",
    "backward_head",
    "forward_rows",
    "row_stats",
    "backward_rows",
    "backward_cols",
    "tiled_forward_head",
    "tiled_backward_head",
]
