"""The bidirectional (non-causal) form of linear attention.

Test infrastructure (see the package docstring).  float64 NumPy only.

Without the causal mask every token reads the same state, the sum over the
whole sequence, so by the associativity of the matrix products O = (Q K^T) V
= Q (K^T V): two products in linear time, the form bidirectional models use
[LA-OV "快速预览"].  With an initial state S0 (the ``[dk, dv]`` convention of
``recurrence``): S = S0 + K^T V, o_t = S^T q_t.  This is the plain
definition written out; the two products are library matmuls.

Parity status: pinned in tests/test_oracle_pins.py against the other
evaluation order (Q K^T) V and against the causal recurrence, whose last
token and final state see the whole sequence too.
"""
import numpy as np


def noncausal_fwd(q, k, v, S0=None):
    """q, k [B, H, L, dk], v [B, H, L, dv], S0 [B, H, dk, dv] or None.
    Returns (out [B, H, L, dv], S [B, H, dk, dv])."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    S = np.matmul(np.swapaxes(k, -1, -2), v)
    if S0 is not None:
        S = S + np.asarray(S0, dtype=np.float64)
    return np.matmul(q, S), S
