"""Token-by-token recurrence: the definition the GPU path must reproduce.

Test infrastructure (see the package docstring).  float64 NumPy only.

State convention.  For one (batch, head) the state ``S`` is a ``dk x dv``
matrix; a key ``k`` (length dk) addresses rows and a value ``v`` (length dv)
fills columns, so a write is the outer product ``k v^T`` and a read with a
query is ``S^T q`` (a length-dv vector).  [CS336 "朴素线性注意力"] describes the
(d, d) state accumulated from per-token ``k_t v_t^T`` and read with ``q_t``;
[LA-OV "Lightning Attention"] writes the same sum as ``k_j^T v_j`` with row
vectors.

Update rules, one token at a time (the first three are special cases of
``gated_delta``, the first of ``gated_linear``):

* ``linear``      S <- S + k v^T.  Plain causal linear attention without
  feature map or normaliser: [HA-1 "线性注意力"] drops the denominator as
  numerically unstable and uses the numerator alone; [LA-OV "The Devil in
  Linear Transformer"] says the same and adds that q and k need no
  activation.  Nothing is ever forgotten [HA-1 "Fast Weight Programmers与
  DeltaNet"].
* ``delta``       read the value currently stored under k, ``s = S^T k``,
  then replace it by a beta-blend of the new and the old value:
  S <- S - beta k s^T + beta k v^T.  This is the delta rule of [HA-1 "Fast
  Weight Programmers与DeltaNet"] (read, learning-rate-controlled blend,
  write), i.e. one gradient step of size beta on the reconstruction loss
  0.5 ||S^T k - v||^2.
* ``gated_delta`` S <- alpha (I - beta k k^T) S + beta k v^T with
  alpha = exp(log_alpha) in (0, 1]: the delta rule preceded by a scalar
  weight decay of the whole state [HA-1 "Gated DeltaNet"; CS336 "继续改进：
  GDN"].  The decay multiplies the old state and the erase term, not the new
  write.  Evaluating ``k^T S`` first keeps the step O(dk dv) instead of
  forming the dk x dk matrix [CS336 "继续改进：GDN"].
* ``gated_linear`` S <- alpha S + k v^T: plain linear attention whose state
  is multiplied by a scalar gate before each write -- the weight decay by
  which Mamba2 forgets the past [HA-1 "Gated DeltaNet"], a gate on the naive
  linear attention's state update that costs a constant factor [CS336
  "继续改进：Mamba"].  No erase and no beta.  Reading taken: the gate is per
  token, alpha = exp(log_alpha) as in ``gated_delta`` (a constant gate is
  the special case of equal log_alpha).

Output.  ``o_t = S_t^T q_t`` with the state *after* token t's update, so a
token sees itself: the causal mask of [LA-OV "快速预览"] includes the diagonal
(j <= t), as does the four-token cumulative-sum example of [LA-OV "Lightning
Attention"].

Gates are scalars per (batch, head, token).  No scaling (1/sqrt(dk)), feature
map, denominator or output norm is applied inside the op.

Parity status: pinned.  ``linear`` is pinned to the masked parallel form
(QK^T * M) V and to the pages' four-token example; ``gated_linear`` to the
same sum with each term weighted by the product of the gates after it
(evaluated by explicit loops), to ``linear`` at alpha = 1, to its alpha -> 0
closed form and to a hand-expanded scalar case; ``delta`` and
``gated_delta`` to a finite-difference gradient step on the reconstruction
loss, exact retrieval with orthonormal keys, the Householder norm invariant,
closed forms for beta = 0 and alpha -> 0, and a hand-expanded scalar case
(tests/test_oracle_pins.py).
"""

import numpy as np

MODES = ("linear", "delta", "gated_delta", "gated_linear")
GATED_MODES = ("gated_delta", "gated_linear")    # use log_alpha
ERASE_MODES = ("delta", "gated_delta")           # use beta (delta rule)


def _check_mode(mode):
    if mode not in MODES:
        raise ValueError(f"mode must be one of {MODES}, got {mode!r}")


def recurrent_step(S, q, k, v, log_alpha, beta, mode):
    """One token of the recurrence, batched over leading axes.

    Shapes: ``S [..., dk, dv]``, ``q, k [..., dk]``, ``v [..., dv]``,
    ``log_alpha, beta [...]`` (ignored where the mode does not use them).
    Returns ``(S_new, o)`` with ``o = S_new^T q`` of shape ``[..., dv]``.
    Inputs are converted to float64; ``S`` is not modified.
    """
    _check_mode(mode)
    S = np.asarray(S, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    write = k[..., :, None] * v[..., None, :]          # k v^T
    if mode == "linear":
        S_new = S + write
    elif mode == "gated_linear":
        alpha = np.exp(np.asarray(log_alpha, dtype=np.float64))[..., None, None]
        S_new = alpha * S + write
    else:
        beta = np.asarray(beta, dtype=np.float64)[..., None, None]
        if mode == "gated_delta":
            alpha = np.exp(np.asarray(log_alpha, dtype=np.float64))[..., None, None]
        else:
            alpha = 1.0
        # Read what is stored under k: s = S^T k, computed before any dk x dk
        # matrix would be formed.
        s = np.einsum("...ij,...i->...j", S, k)
        erase = k[..., :, None] * s[..., None, :]      # k (S^T k)^T = k k^T S
        S_new = alpha * S - alpha * beta * erase + beta * write
    o = np.einsum("...ij,...i->...j", S_new, q)
    return S_new, o


def recurrent_fwd(q, k, v, log_alpha, beta, S0, mode):
    """Causal forward over a whole sequence, one token at a time.

    Shapes: ``q, k [B, H, L, dk]``, ``v [B, H, L, dv]``,
    ``log_alpha, beta [B, H, L]`` (may be None where the mode ignores them),
    ``S0 [B, H, dk, dv]`` or None for a zero initial state.
    Returns ``(o [B, H, L, dv], S_final [B, H, dk, dv])`` in float64.
    """
    _check_mode(mode)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, L, dk = k.shape
    dv = v.shape[-1]
    if mode in ERASE_MODES and beta is None:
        raise ValueError("beta is required for the delta modes")
    if mode in GATED_MODES and log_alpha is None:
        raise ValueError(f"log_alpha is required for {mode}")
    la = None if log_alpha is None else np.asarray(log_alpha, dtype=np.float64)
    be = None if beta is None else np.asarray(beta, dtype=np.float64)
    S = (np.zeros((B, H, dk, dv)) if S0 is None
         else np.array(S0, dtype=np.float64, copy=True))
    o = np.empty((B, H, L, dv))
    for t in range(L):
        S, o[:, :, t] = recurrent_step(
            S, q[:, :, t], k[:, :, t], v[:, :, t],
            None if la is None else la[:, :, t],
            None if be is None else be[:, :, t],
            mode)
    return o, S


def decode_steps(S0, q, k, v, log_alpha, beta, mode):
    """A run of single-token decode steps on a batch of independent states.

    Shapes: ``S0 [B, H, dk, dv]``, ``q, k [N, B, H, dk]``, ``v [N, B, H, dv]``,
    ``log_alpha, beta [N, B, H]`` for N consecutive steps.  Step n consumes
    the state step n-1 produced (prefill hands its final state to decode,
    [HA-1 "Prefill、Decode与KVCache"]; [CS336 "朴素线性注意力"] runs the
    recurrent form at inference).  Returns ``(o [N, B, H, dv], S_N)``.
    """
    _check_mode(mode)
    S = np.array(S0, dtype=np.float64, copy=True)
    N = np.shape(q)[0]
    o = np.empty((N,) + np.shape(v)[1:])
    for n in range(N):
        S, o[n] = recurrent_step(
            S, q[n], k[n], v[n],
            None if log_alpha is None else log_alpha[n],
            None if beta is None else beta[n],
            mode)
    return o, S
