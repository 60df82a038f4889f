"""Oracle: a plain, slow, CPU-only statement of what the fused kernels compute.

This package is TEST INFRASTRUCTURE. Only the test suite, the smoke check in
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call it. The product path (the HIP library and its Python binding)
never imports it, and it imports nothing from the product path: the two share
no kernels, headers, helpers or constant tables. The only code both sides meet
is the seeded input generator, which holds none of the method's arithmetic.

Every result here is written as the *unfused* cascade the pages describe
(max, then sum of exponentials, then divide, then multiply; mean, then the
centred second moment), in float64 with
numpy, so a reader can check it against the pages by eye. Sources:

* "RedFuser episode transcript" (podcast.do-not-panic.com, episode of
  2026-10-13), cues 5, 9, 11, 15, 19, 21, 29, 31, 33, 39, 41, 47, 55.
* "RedFuser episode visual explainer" (same site, /viz/), the widgets
  "Online softmax, step by step", "Rescale the output accumulator too" and
  "Merging partial states across blocks (FlashDecoding-style)".
* "RedFuser: An Automatic Operator Fusion Framework for Cascaded Reductions on
  AI Accelerators" (bookshelf explainer), sections "Problem" and
  "This paper's idea".
* "Online normalizer calculation for softmax" (citation index page), abstract.

Parity status of each function is stated in its module docstring.
"""

from .attention import (
    attention,
    attention_online,
    decode_partials,
    merge_states,
    NEG_INF,
)
from .routing import softmax_rows, softmax_topk
from .codec import e4m3_decode, e4m3_encode, e4m3_table
from .quant import absmax_quant, quant_gemm, quant_gemm_running_scale
from .moments import row_inertia, row_variance

__all__ = [
    "attention",
    "attention_online",
    "decode_partials",
    "merge_states",
    "NEG_INF",
    "softmax_rows",
    "softmax_topk",
    "e4m3_decode",
    "e4m3_encode",
    "e4m3_table",
    "absmax_quant",
    "quant_gemm",
    "quant_gemm_running_scale",
    "row_inertia",
    "row_variance",
]
