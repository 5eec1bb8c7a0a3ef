"""The steps in front of the op that the fused entry points take inside:
L2 normalisation of q and k and the gate activations.

Test infrastructure (see the package docstring).  float64 NumPy only.

* L2 normalisation, x / sqrt(|x|^2 + eps) per token (the last axis), eps =
  1e-6.  The delta rule's read-then-replace recovers a stored value exactly
  only when the key has unit length [HA-1 "Fast Weight Programmers与
  DeltaNet"]; queries are normalised the same way.  Reading taken: the
  small eps inside the root keeps an all-zero vector at zero instead of
  dividing by zero (the pages give no formula for the normalisation).
* Write strength beta = sigmoid(b) = 1 / (1 + e^-b): a value in (0, 1)
  produced by an activation from a learned score, as for the delta rule's
  learning-rate network [HA-1 "Fast Weight Programmers与DeltaNet"].
* Decay log alpha = -gate_scale * softplus(a), softplus(a) = log(1 + e^a):
  a non-negative rate through softplus, so alpha = exp(log alpha) is in
  (0, 1] -- the scalar weight decay of Mamba2 that Gated DeltaNet adopts
  [HA-1 "Gated DeltaNet"; CS336 "继续改进：Mamba"].  Reading taken: one
  positive scale per call (the pages fix no parametrisation of the rate).

The library routines ``scipy.special.expit`` (the logistic function) and
``numpy.logaddexp`` (log(e^x + e^y), here log(1 + e^a)) serve as steps.

Parity status: pinned in tests/test_oracle_pins.py by closed forms
(sigmoid(0) = 1/2, sigmoid(log 3) = 3/4, softplus(0) = log 2,
softplus(log(e - 1)) = 1, softplus(a) - softplus(-a) = a), by the norm of a
normalised vector in closed form, and by the scale invariance of the whole
op under normalisation.
"""
import numpy as np
import scipy.special

from .recurrence import ERASE_MODES, GATED_MODES

QK_NORM_EPS = 1e-6
GATES = 1        # flags: raw gate scores through the activations
QK_L2NORM = 2    # flags: q and k normalised per token


def l2_normalise(x, eps=QK_NORM_EPS):
    """x / sqrt(sum(x^2) + eps) along the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def sigmoid(x):
    return scipy.special.expit(np.asarray(x, dtype=np.float64))


def softplus(x):
    return np.logaddexp(0.0, np.asarray(x, dtype=np.float64))


def prepare(q, k, a, b, mode, flags, gate_scale):
    """The op's inputs after the prologue ``flags`` asks for: returns
    (q, k, log_alpha, beta).  Gates a mode does not read pass through
    unchanged (None stays None)."""
    if flags & QK_L2NORM:
        q, k = l2_normalise(q), l2_normalise(k)
    log_alpha, beta = a, b
    if flags & GATES:
        if mode in GATED_MODES:
            log_alpha = -gate_scale * softplus(a)
        if mode in ERASE_MODES:
            beta = sigmoid(b)
    return q, k, log_alpha, beta
