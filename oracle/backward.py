"""Gradients of the recurrence: the reverse of the token-by-token update.

Test infrastructure (see the package docstring).  float64 NumPy only.

Training runs the chunked (parallel) form and needs the gradients of every
input; the chunked form saves the per-chunk states for that [HA-1 "FWP分块
并行机制"; CS336 "朴素线性注意力": train with the parallel form, infer with the
recurrent one].  The pages print no usable gradient formulas (those that
[HA-1 "线性注意力"] derives for linear attention in training are lost in the
extraction), so this module differentiates the definition in
``recurrence`` itself: for a scalar
loss with upstream gradients dO (of every output) and dS_final (of the final
state), it walks the tokens backwards carrying dS = dLoss / dS_t.

With S = S_{t-1}, a = exp(log_alpha_t), b = beta_t and, in the delta modes,
S_t = a (S - b k k^T S) + b k v^T (a = 1 for ``delta``; ``linear`` and
``gated_linear`` have S_t = a S + k v^T), o_t = S_t^T q_t:

* dS_t += q_t do_t^T                       (o_t reads S_t)
* dq_t  = S_t do_t
* dv_t  = b dS_t^T k                       (b = 1 without erase)
* dk_t  = b dS_t v - a b (dS_t S^T k + S dS_t^T k)      (erase modes)
          dS_t v                                         (otherwise)
* dbeta_t      = k^T dS_t v - a k^T dS_t S^T k
* dlog_alpha_t = a <dS_t, S - b k k^T S>   (<A, B> = sum of the products;
  evaluated as a (<dS_t, S> - b k^T dS_t S^T k))
* dS_{t-1} = a (dS_t - b k (k^T dS_t))     (the update's matrix is
  symmetric), and dS0 = dS_0 at the end.

Each is the derivative of one term of the update by the product rule; the
erase term k k^T S contributes through both of its k factors.

Parity status: pinned in tests/test_oracle_pins.py by central finite
differences of the loss in every input and every mode, and by the closed
forms of causal linear attention's gradients, dV = (Q K^T * M)^T dO, dQ =
(dO V^T * M) K, dK = (dO V^T * M)^T Q.
"""
import numpy as np

from .recurrence import ERASE_MODES, GATED_MODES, _check_mode, recurrent_step


def recurrent_bwd(q, k, v, log_alpha, beta, S0, mode, dO, dS_final=None, checkpoint=None):
    """Gradients of sum(dO * O) + sum(dS_final * S_final).

    Shapes as in ``recurrent_fwd``; ``dO [B, H, L, dv]``, ``dS_final
    [B, H, dk, dv]`` or None.  Returns a dict with ``dq, dk, dv [B, H, L, d]``,
    ``dlog_alpha, dbeta [B, H, L]`` (None where the mode does not read the
    gate) and ``dS0 [B, H, dk, dv]``.

    ``checkpoint``: None keeps every state S_0 .. S_L of the forward (small
    cases); an integer n keeps only S_0, S_n, S_2n, ... and recomputes the
    states inside each run of n tokens from its first one just before the
    reverse walk crosses it, so memory is O(L / n + n) states instead of
    O(L).  The recomputation repeats the forward's own steps in the same
    order, so the gradients are bit-identical for every n.
    """
    _check_mode(mode)
    q, k, v, dO = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dO))
    B, H, L, dk = k.shape
    dv = v.shape[-1]
    erase, gated = mode in ERASE_MODES, mode in GATED_MODES
    la = np.asarray(log_alpha, dtype=np.float64) if gated else np.zeros((B, H, L))
    be = np.asarray(beta, dtype=np.float64) if erase else np.ones((B, H, L))
    span = L if checkpoint is None else int(checkpoint)
    if span < 1:
        raise ValueError("checkpoint must be a positive number of tokens")

    def run(S, t0, t1):
        """The forward's states S_t0 .. S_t1, starting from S = S_t0."""
        out = np.empty((t1 - t0 + 1, B, H, dk, dv))
        out[0] = S
        for t in range(t0, t1):
            out[t - t0 + 1], _ = recurrent_step(out[t - t0], q[:, :, t], k[:, :, t], v[:, :, t],
                                                la[:, :, t], be[:, :, t], mode)
        return out

    # forward: the state at the start of every run of `span` tokens
    starts = list(range(0, L, span))
    ckpt = {0: np.zeros((B, H, dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)}
    for i, t0 in enumerate(starts[:-1]):
        ckpt[starts[i + 1]] = run(ckpt[t0], t0, starts[i + 1])[-1]
    dS = np.zeros((B, H, dk, dv)) if dS_final is None else np.array(dS_final, dtype=np.float64)
    g = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v))}
    dla, dbe = np.zeros((B, H, L)), np.zeros((B, H, L))
    states, t0 = None, L
    for t in range(L - 1, -1, -1):
        if t < t0:
            # entering the run that holds token t: recompute its states
            t0 = (t // span) * span
            states = run(ckpt[t0], t0, min(t0 + span, L))
        S, St = states[t - t0], states[t - t0 + 1]
        qt, kt, vt, dot = q[:, :, t], k[:, :, t], v[:, :, t], dO[:, :, t]
        a = np.exp(la[:, :, t])[..., None]           # [B, H, 1]
        b = be[:, :, t][..., None]
        dS = dS + qt[..., :, None] * dot[..., None, :]
        g["dq"][:, :, t] = (St @ dot[..., :, None])[..., 0]
        kdS = (kt[..., None, :] @ dS)[..., 0, :]      # k^T dS        [dv]
        dSv = (dS @ vt[..., :, None])[..., 0]         # dS v          [dk]
        g["dv"][:, :, t] = b * kdS
        if erase:
            Sk = (kt[..., None, :] @ S)[..., 0, :]    # S^T k         [dv]
            dSSk = (dS @ Sk[..., :, None])[..., 0]    # dS S^T k      [dk]
            SdSk = (S @ kdS[..., :, None])[..., 0]    # S dS^T k      [dk]
            g["dk"][:, :, t] = b * dSv - a * b * (dSSk + SdSk)
            kdSv = np.sum(kt * dSv, axis=-1)          # k^T dS v
            kdSSk = np.sum(kdS * Sk, axis=-1)         # k^T dS S^T k
            dbe[:, :, t] = kdSv - a[..., 0] * kdSSk
            # <dS, S - b k k^T S> = <dS, S> - b k^T dS S^T k
            inner = np.sum(dS * S, axis=(-2, -1)) - b[..., 0] * kdSSk
        else:
            g["dk"][:, :, t] = dSv
            inner = np.sum(dS * S, axis=(-2, -1))
        if gated:
            dla[:, :, t] = a[..., 0] * inner
        # dS_{t-1} = a (dS - b k (k^T dS))
        if erase:
            dS = a[..., None] * (dS - b[..., None] * kt[..., :, None] * kdS[..., None, :])
        else:
            dS = a[..., None] * dS
    return dict(dq=g["dq"], dk=g["dk"], dv=g["dv"],
                dlog_alpha=dla if gated else None, dbeta=dbe if erase else None, dS0=dS)
