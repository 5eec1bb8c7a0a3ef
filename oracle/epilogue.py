"""The steps behind the op that the fused entry points take inside: the
residual in v and the output normalisation.

Test infrastructure (see the package docstring).  float64 NumPy only.
Outputs and values are laid out [B, H, L, dv]; the per-head channel
parameters D and w are [H, dv].

* Residual in v: o_t + D * v_t per channel.  Mamba adds to the output a term
  in v next to the state's read-out, a residual path that lets the input
  reach the output without passing through the compressed state [CS336
  "继续改进：Mamba"].  Reading taken: one learned factor per (head, value
  channel), the usual shape of that term (the pages give no formula).
* Output normalisation: o_t / sqrt(mean over dv of o_t^2 + eps) * w.  With the
  denominator of linear attention dropped for its numerical trouble, a norm
  of the output takes its place, O = XNorm(Q (K^T V)) [LA-OV "The Devil in
  Linear Transformer"].  Reading taken: XNorm is the root-mean-square norm
  over the value channels of each (token, head) with a per-head channel
  weight (the pages name no particular norm); it comes after the residual.

Parity status: pinned in tests/test_oracle_pins.py by a worked example of
the residual and by the closed form of the normalised mean square.
"""
import numpy as np


def add_dskip(o, v, D):
    """o + D * v with D [H, dv] broadcast over batch and tokens."""
    D = np.asarray(D, dtype=np.float64)
    return np.asarray(o, dtype=np.float64) + D[None, :, None, :] * np.asarray(v, np.float64)


def out_norm(o, w=None, eps=1e-6):
    """o / sqrt(mean(o^2) + eps) per (b, h, t) over dv, times w [H, dv]."""
    o = np.asarray(o, dtype=np.float64)
    y = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    if w is not None:
        y = y * np.asarray(w, dtype=np.float64)[None, :, None, :]
    return y
