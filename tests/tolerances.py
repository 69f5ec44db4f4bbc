"""Tolerances of the attention comparisons.

The contract bars are max-abs 1e-4 for fp32 outputs and 2e-2 for bf16
outputs.  For bf16 the contract bar is about the size of the outputs
themselves at long contexts (a few hundredths), so bf16 outputs are also held
to a per-element bound derived from the arithmetic:

* the kernel accumulates in fp32; against the exact result o its fp32 value
  o32 is off by at most delta = ACC_REL * sum_t w_t |V_t| (w the softmax
  weights over the attended rows).  The a-priori bound of the fp32 logit dot
  products over 128 coordinates, the exp2 approximation and the blocked
  weighted sums stays below 2^-13 of that sum; ACC_REL = 2^-12 allows twice
  that;
* rounding o32 to bf16 (8 significant bits, nearest even) moves it by at most
  half a unit in the last place, 2^-8 |o32| <= 2^-8 (|o| + delta).

Hence |o_bf16 - o| <= 2^-8 |o| + 2 delta per element.  Dropping one percent
of the attended rows, or attending to a wrong row set of that size, moves
some outputs far beyond it (see test_attention_bound.py).
"""
from __future__ import annotations

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}
BF16_HALF_ULP_REL = 2.0 ** -8
ACC_REL = 2.0 ** -12


def bf16_bound(o_ref: np.ndarray, w: np.ndarray, VA: np.ndarray) -> np.ndarray:
    """Per-element bound of |o_gpu - o_ref| for one head's bf16 output.

    o_ref [D] the exact output, w [|A|] its softmax weights, VA [|A|, D] the
    attended V rows (in the order of w)."""
    delta = ACC_REL * (np.asarray(w) @ np.abs(VA)) if len(w) else np.zeros_like(o_ref)
    return BF16_HALF_ULP_REL * np.abs(o_ref) + 2.0 * delta
