"""CPU oracle for chunkwise gated-delta linear attention (test infrastructure).

This package is test infrastructure, not part of the product.  Only the test
suite, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of
``bench.py`` may import it.  The GPU library never imports, links or calls
anything in here, and nothing in here imports the GPU library: the two share
no code.  Inputs reach both sides from the seeded generators in
``workloads/``, which hold none of the method's arithmetic.

Everything is float64 NumPy, written for a reader to check against the pages
by eye rather than for speed.

Sources (cited by title and section):

* [HA-1]  "混合注意力学习(1): 线性注意力" (hybrid-attention notes, part 1:
  linear attention), jsqmd.com.
* [LA-OV] "LinearAttention 概述" (linear attention overview), razer666.cn.
* [CS336] "【CS336】lecture4 线性注意力|Mamba|GDN|DSA" (lecture-4 notes),
  wsisp.com.

Modules:

* ``recurrence`` -- the token-by-token recurrence (the definition of what the
  method computes) and the single decode step.
* ``chunkwise``  -- the chunkwise-parallel algebra in float64 (masked intra-
  chunk products, WY/UT representation, decay folding); it is pinned to the
  recurrence by the exactness of the chunkwise form and is used to pin
  intermediates.
* ``prologue``   -- the steps in front of the op that the fused entry points
  take inside (q, k L2 normalisation, gate activations).
* ``epilogue``   -- the steps behind it (the residual in v, the output
  normalisation).
* ``noncausal``  -- the bidirectional form O = Q (S0 + K^T V).
* ``backward``   -- the gradients of every input, by the reverse of the token
  recurrence.

Parity status of each function is stated in its module header.
"""

from .recurrence import (  # noqa: F401
    ERASE_MODES,
    GATED_MODES,
    MODES,
    decode_steps,
    recurrent_fwd,
    recurrent_step,
)
from .prologue import l2_normalise, prepare, prologue_bwd, sigmoid, softplus  # noqa: F401
from .epilogue import add_dskip, out_norm  # noqa: F401
from .noncausal import noncausal_fwd  # noqa: F401
from .backward import recurrent_bwd  # noqa: F401
from .chunkwise import (  # noqa: F401
    chunkwise_bwd,
    chunkwise_fwd,
    forward_substitution_inverse,
    parallel_masked_linear,
    ut_transform,
    wy_transition,
)
