"""CPU oracle for the HyperAttention forward pass, its backward and the
row-norm-sampling variant of the product (``oracle.rownorm``) and the
method's fine-grained parameters as diagnostics (``oracle.diagnostics``).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (``approximate_long_context_amd``); the two are written
separately from the same definitions and meet only in the tests.

The oracle is plain, slow and meant to be read against the pages.  All
floating point is IEEE fp64, except where the method's definition fixes
another precision (the fp32 hash).  Sources cited below:

  [S] "HyperAttention: Long-context Attention in Near-Linear Time",
      atlas.scime.ai research-map summary page; sections "Approach",
      "Limitations", "Key results", "Experimental setup" ("Builds on").
  [A] "HyperAttention: Long-context Attention in Near-Linear Time",
      OpenReview forum page, "Abstract".
  [P] Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
      1, 2, 3", SC'11 (Philox4x32-10).
  [BM] Box & Muller, "A note on the generation of random normal deviates",
      Ann. Math. Stat. 1958.

Where the pages leave a step open, the reading used is stated at the
function that takes it.

Pins (see ``tests/test_oracle_*.py``): every function here is checked
against something other than itself -- a library implementation (rocRAND's
Philox, libm, ``scipy.special.softmax``, ``numpy.argsort``), a closed form,
an exhaustive enumeration or brute force on tiny inputs.  Parity unpinned:
none of the functions; the *approximation quality* of the method relative
to exact attention has no printed reference value on the pages and is only
reported, never asserted.
"""

from .philox import philox4x32_10, philox_words
from .gauss import neg2_log_u, sincos_2pi, sqrt_newton, box_muller, projections
from .hyperattn import (
    HAConfig,
    hash_codes,
    gray_inverse,
    ranks,
    sort_perm,
    sample_positions,
    block_part,
    sample_part,
    lse_merge,
    noncausal_problem,
    causal_problem,
    forward,
    forward_rows,
    exact_attention,
    causal_levels,
)

__all__ = [
    "philox4x32_10", "philox_words", "neg2_log_u", "sincos_2pi", "sqrt_newton",
    "box_muller", "projections", "HAConfig", "hash_codes", "gray_inverse",
    "ranks", "sort_perm", "sample_positions", "block_part", "sample_part",
    "lse_merge", "noncausal_problem", "causal_problem", "forward", "forward_rows",
    "exact_attention", "causal_levels",
]
from . import backward  # noqa: E402  (weighted-softmax backward, fp64)
from . import rownorm  # noqa: E402  (row-norm-sampling variant of the product)
from . import diagnostics  # noqa: E402  (alpha and the residual row-sum ratio)
