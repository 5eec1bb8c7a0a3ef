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

``prologue_bwd`` carries the gradients of the op's prepared inputs back to
the raw ones by the chain rule, one step per activation: for x_hat = x r,
r = (|x|^2 + eps)^(-1/2), dx = r (dx_hat - x_hat (x_hat . dx_hat)); for
beta = sigmoid(b), db = dbeta sigmoid(b) (1 - sigmoid(b)); for log alpha =
-gate_scale softplus(a), da = -gate_scale sigmoid(a) dlog_alpha (the
derivative of softplus is the logistic function).

Parity status: pinned in tests/test_oracle_pins.py by closed forms
(sigmoid(0) = 1/2, sigmoid(log 3) = 3/4, softplus(0) = log 2,
softplus(log(e - 1)) = 1, softplus(a) - softplus(-a) = a), by the norm of a
normalised vector in closed form, and by the scale invariance of the whole
op under normalisation; ``prologue_bwd`` composed with the recurrence's
backward by central finite differences of the loss in the raw inputs, for
every mode and flag set.
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


def prologue_bwd(q, k, a, b, mode, flags, gate_scale, dq, dk, dlog_alpha, dbeta):
    """Gradients of the raw inputs of ``prepare`` from those of its outputs.

    ``q, k, a, b`` are the raw inputs (as for ``prepare``); ``dq, dk,
    dlog_alpha, dbeta`` the gradients of the prepared q, k, log alpha and
    beta (None where the mode has none).  Returns (dq_raw, dk_raw, da, db).
    """
    dq = np.asarray(dq, dtype=np.float64)
    dk = np.asarray(dk, dtype=np.float64)
    if flags & QK_L2NORM:
        out = []
        for x, dx in ((q, dq), (k, dk)):
            x = np.asarray(x, dtype=np.float64)
            r = 1.0 / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + QK_NORM_EPS)
            xh = x * r
            out.append(r * (dx - xh * np.sum(xh * dx, axis=-1, keepdims=True)))
        dq, dk = out
    da, db = dlog_alpha, dbeta
    if flags & GATES:
        if mode in GATED_MODES and dlog_alpha is not None:
            da = -gate_scale * sigmoid(a) * np.asarray(dlog_alpha, dtype=np.float64)
        if mode in ERASE_MODES and dbeta is not None:
            sb = sigmoid(b)
            db = sb * (1.0 - sb) * np.asarray(dbeta, dtype=np.float64)
    return dq, dk, da, db
