"""CPU oracle for the fp8 mixture-of-experts grouped-matmul hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only the tests, the smoke check and the CPU-baseline leg of
the benchmark use it.  It is a plain, slow, obviously-correct restatement of
what the path computes, written from the pull-request pages it cites, in
NumPy with float64 accumulation.  It shares no code with the HIP library.

Pages cited (by title and section):

* "Quantize activations before EP all gather" (MaxText pull request 4812):
  the description (quantize activations before the expert-parallel
  all-gather, so that the collective and the activation sort move fp8),
  its "Testing strategy" section (equivalence of quantize-then-gather and
  gather-then-quantize) and the code-review comments on the prequantized
  ``gmm_v2`` test, on ``ragged_sort.py`` (the per-token scale is gathered
  only when its leading dimension is the token dimension) and on
  ``ragged_gather_reduce_v2.py`` (output dtype defaults to bf16).
* "Support quantization for tokamax gmm v2" (MaxText pull request 4451):
  "What this does" (gmm2 / tgmm2 quantization, forward/backward split) and
  the tolerance discussion with its quantization schemes (``fp8_dynamic`` =
  absmax for weight, activation and gradient; ``fp8_static_wa`` = fixed
  weight and activation scales plus absmax gradients) and the tables
  "relative_norm_diff Across All Cases" and "max_abs_diff Across All Cases".
* "Keep qwix out of tpu-inference's fused MoE kernel and pre-quantize
  weights" (MaxText pull request 5136): the Mosaic error showing that an
  fp8 x fp8 matmul needs a 32-bit accumulator, and "Changes in this PR"
  (weights pre-quantized to float8_e4m3fn with [E, blocks, 1, N] scales).

Every function is pinned by tests under ``tests/`` that check it against
textbook value sets, library routines (``numpy.argsort``, ``numpy.bincount``,
torch's CPU float8 / bfloat16 casts), brute force on tiny inputs, exact
rational arithmetic and the invariants the pages state.
"""

from .codec import (E4M3_MAX, bf16_decode, bf16_rne_from_f32, bf16_rne_from_f64,
                    e4m3_decode, e4m3_rne)
from .quantize import (SCALE_ROW_DYNAMIC, SCALE_TENSOR_DYNAMIC, SCALE_TENSOR_FROM_ROW_AMAX, SCALE_TENSOR_STATIC,
                       pinned_exp_f32, quantize_rows, quantize_weights, silu_mul_backward, silu_mul_backward_f32,
                       silu_mul_f32)
from .sort import sort_by_expert
from .gmm import gmm, tgmm
from .gather_reduce import gather_reduce, gather_reduce_backward

__all__ = [
    "E4M3_MAX", "bf16_decode", "bf16_rne_from_f32", "bf16_rne_from_f64", "e4m3_decode",
    "e4m3_rne", "SCALE_ROW_DYNAMIC", "SCALE_TENSOR_DYNAMIC", "SCALE_TENSOR_STATIC", "SCALE_TENSOR_FROM_ROW_AMAX",
    "pinned_exp_f32", "quantize_rows", "quantize_weights", "silu_mul_f32", "silu_mul_backward",
    "silu_mul_backward_f32",
    "sort_by_expert", "gmm", "tgmm", "gather_reduce", "gather_reduce_backward",
]
