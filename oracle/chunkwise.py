"""Chunkwise-parallel form of the same recurrence, in float64.

Test infrastructure (see the package docstring).  It exists to pin the chunk
algebra that the GPU kernels implement -- the masked intra-chunk products,
the WY/UT representation and the decay folding -- against the token
recurrence in ``recurrence.py``, and to expose the per-chunk intermediates.

What the pages fix:

* Parallel form.  Stacking the rows of one sequence, plain causal linear
  attention is ``O = (Q K^T * M) V`` with ``M`` lower-triangular including the
  diagonal [HA-1 "传统FWP形式的线性注意力并行"; LA-OV "快速预览"].
* Chunkwise form.  Cut the sequence into chunks of C rows; inside a chunk use
  the masked product, across chunks carry the state.  With C = 1 it is the
  recurrent form and with C = L the parallel form; it is exact, so the chunk
  size does not change the output [HA-1 "FWP分块并行机制"; LA-OV "FLASH"].
* Delta rule in chunks.  Absorbing the erase term into per-token vectors that
  still need the previous state neither parallelises nor saves memory [HA-1
  "DeltaNet 分块并行机制"]; an inductive redefinition gives per-token vectors
  (here W and U) built from the chunk's own keys and values only, so no past
  state is stored [HA-1 "重新定义降低内存占用"].  The induction mirrors the
  WY representation: a product of rank-1 corrections (I - beta k k^T) equals
  the identity minus one low-rank product [HA-1 "HouseHolder变换和WY表示"].

Reading taken where the pages are silent (formulas for the gated chunk form
were lost in extraction).  Within a chunk with rows r = 1..C let
``g_r = sum_{i<=r} log_alpha_i``, ``gamma_r = exp(g_r)`` and
``Gamma_ri = exp(g_r - g_i)`` for i <= r.  Writing the recurrence as
``S_r = alpha_r S_{r-1} + k_r u_r^T`` with ``u_r = beta_r (v_r - alpha_r
S_{r-1}^T k_r)`` and unrolling inside the chunk from the chunk-entry state S
gives a unit lower-triangular system for the rows u_r:

    A = strict_lower(diag(beta) (K K^T) * Gamma)
    T = (I + A)^{-1}                       (forward substitution)
    W = T diag(beta * gamma) K,   U = T diag(beta) V
    U_new = U - W S                        (the true u_r rows)
    O = diag(gamma) Q S + (Q K^T * M * Gamma) U_new
    S' = gamma_C S + (diag(gamma_C / gamma) K)^T U_new

With alpha = 1 (``delta``) every gamma is 1 and this is the UT/WY form; in
``linear`` and ``gated_linear`` mode u_r = v_r and the system disappears:

    O = diag(gamma) Q S + (Q K^T * M * Gamma) V
    S' = gamma_C S + (diag(gamma_C / gamma) K)^T V

(``linear``: every gamma and Gamma entry is 1).  The chunk's state map
for V = 0 is ``S' = P S`` with ``P = gamma_C I - (diag(gamma_C/gamma) K)^T W``,
equal to the product of the per-token factors alpha_r (I - beta_r k_r k_r^T)
(latest factor on the left).

Parity status: pinned -- to the token recurrence for C = 1, C = L and ragged
chunkings in every mode (and through it to the pins of each mode), T to a
library triangular solve, P to the explicit product of dk x dk factors;
``chunkwise_bwd`` to the reverse of the token recurrence (``backward``,
itself pinned by finite differences) for every mode and chunking
(tests/test_oracle_pins.py).
"""

import numpy as np

from .recurrence import ERASE_MODES, GATED_MODES, MODES


def parallel_masked_linear(q, k, v):
    """``O = (Q K^T * M) V`` with the inclusive causal mask M.

    Shapes ``q, k [..., L, dk]``, ``v [..., L, dv]``; returns ``[..., L, dv]``.
    Quadratic in L; for pinning the linear recurrence only.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    L = k.shape[-2]
    M = np.tril(np.ones((L, L)))
    scores = np.matmul(q, np.swapaxes(k, -1, -2)) * M
    return np.matmul(scores, v)


def forward_substitution_inverse(A):
    """Inverse of ``I + A`` for strictly lower-triangular ``A [..., C, C]``.

    Row r of ``T = (I + A)^{-1}`` follows from row r of ``(I + A) T = I``:
    ``T_r = e_r - sum_{i<r} A_ri T_i``, using only rows already solved.
    """
    A = np.asarray(A, dtype=np.float64)
    C = A.shape[-1]
    T = np.zeros_like(A)
    for r in range(C):
        T[..., r, r] = 1.0
        for i in range(r):
            T[..., r, :] -= A[..., r, i, None] * T[..., i, :]
    return T


def _gates(log_alpha, beta, n, mode, lead_shape):
    """Per-row log-decay and write strength for one chunk of n rows."""
    if mode in GATED_MODES:
        la = np.asarray(log_alpha, dtype=np.float64)
    else:
        la = np.zeros(lead_shape + (n,))
    if mode in ERASE_MODES:
        be = np.asarray(beta, dtype=np.float64)
    else:
        be = np.ones(lead_shape + (n,))
    return la, be


def _decay(g):
    """gamma_r = exp(g_r) and Gamma_ri = exp(g_r - g_i) for i <= r (0 above).

    The exponent is masked before exponentiation so that no positive
    exponent (i > r) is ever evaluated.
    """
    n = g.shape[-1]
    lower = np.tril(np.ones((n, n), dtype=bool))
    diff = g[..., :, None] - g[..., None, :]
    Gamma = np.where(lower, np.exp(np.where(lower, diff, 0.0)), 0.0)
    return np.exp(g), Gamma


def ut_transform(k, v, log_alpha, beta, mode):
    """Per-chunk WY/UT quantities for ``delta`` and ``gated_delta``.

    Shapes: ``k [..., n, dk]``, ``v [..., n, dv]``, ``log_alpha, beta [..., n]``.
    Returns a dict with ``g, gamma, Gamma, A, T, W, U``.
    """
    if mode not in ("delta", "gated_delta"):
        raise ValueError("the UT transform applies to the delta modes only")
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = k.shape[-2]
    la, be = _gates(log_alpha, beta, n, mode, k.shape[:-2])
    g = np.cumsum(la, axis=-1)
    gamma, Gamma = _decay(g)
    KKt = np.matmul(k, np.swapaxes(k, -1, -2))
    A = np.tril(be[..., :, None] * KKt * Gamma, k=-1)
    T = forward_substitution_inverse(A)
    W = np.matmul(T, (be * gamma)[..., :, None] * k)
    U = np.matmul(T, be[..., :, None] * v)
    return dict(g=g, gamma=gamma, Gamma=Gamma, A=A, T=T, W=W, U=U)


def wy_transition(k, log_alpha, beta, mode):
    """The chunk's state map for zero values, ``P = gamma_C I - Kt^T W``.

    ``Kt = diag(gamma_C / gamma) K``.  Shape ``[..., dk, dk]``.
    """
    k = np.asarray(k, dtype=np.float64)
    n, dk = k.shape[-2:]
    ut = ut_transform(k, np.zeros(k.shape[:-1] + (1,)), log_alpha, beta, mode)
    g = ut["g"]
    gC = g[..., -1:]
    Kt = np.exp(gC - g)[..., :, None] * k
    return (np.exp(gC)[..., None] * np.eye(dk)
            - np.matmul(np.swapaxes(Kt, -1, -2), ut["W"]))


def chunkwise_fwd(q, k, v, log_alpha, beta, S0, mode, C):
    """Chunkwise forward, any chunk size C >= 1, ragged last chunk allowed.

    Same shapes and result as ``recurrence.recurrent_fwd``.
    """
    if mode not in MODES:
        raise ValueError(f"mode must be one of {MODES}, got {mode!r}")
    if C < 1:
        raise ValueError("chunk size must be >= 1")
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, L, dk = k.shape
    dv = v.shape[-1]
    S = (np.zeros((B, H, dk, dv)) if S0 is None
         else np.array(S0, dtype=np.float64, copy=True))
    o = np.empty((B, H, L, dv))
    for s in range(0, L, C):
        e = min(s + C, L)
        Q, K, V = q[:, :, s:e], k[:, :, s:e], v[:, :, s:e]
        n = e - s
        QKt = np.matmul(Q, np.swapaxes(K, -1, -2))
        if mode not in ERASE_MODES:
            la, _ = _gates(None if log_alpha is None else log_alpha[:, :, s:e],
                           None, n, mode, K.shape[:-2])
            g = np.cumsum(la, axis=-1)
            gamma, Gamma = _decay(g)
            o[:, :, s:e] = (gamma[..., :, None] * np.matmul(Q, S)
                            + np.matmul(QKt * Gamma, V))
            gC = g[..., -1:]
            Kt = np.exp(gC - g)[..., :, None] * K
            S = (np.exp(gC)[..., None] * S
                 + np.matmul(np.swapaxes(Kt, -1, -2), V))
            continue
        ut = ut_transform(K, V,
                          None if log_alpha is None else log_alpha[:, :, s:e],
                          beta[:, :, s:e], mode)
        g, gamma, Gamma = ut["g"], ut["gamma"], ut["Gamma"]
        U_new = ut["U"] - np.matmul(ut["W"], S)
        o[:, :, s:e] = (gamma[..., :, None] * np.matmul(Q, S)
                        + np.matmul(QKt * Gamma, U_new))
        gC = g[..., -1:]
        Kt = np.exp(gC - g)[..., :, None] * K
        S = (np.exp(gC)[..., None] * S
             + np.matmul(np.swapaxes(Kt, -1, -2), U_new))
    return o, S


def chunkwise_bwd(q, k, v, log_alpha, beta, S0, mode, C, dO, dS_final=None):
    """Gradients by the chunkwise form: the same result as
    ``backward.recurrent_bwd``, organised as a GPU backward would be.

    The forward keeps the state entering every chunk (the per-chunk states a
    training run saves [HA-1 "FWP分块并行机制"]).  Then, chunk by chunk in
    reverse, with dS' the gradient of the state leaving the chunk and the
    chunk's quantities as in ``chunkwise_fwd`` (f = gamma_C / gamma, P =
    Q K^T * M * Gamma):

        dU = P^T dO + diag(f) K dS'              (U = U_new; V without erase)
        dR = T^T dU                              (U = T R, R = diag(beta)(V -
                                                  diag(gamma) K S))
        dS = gamma_C dS' + Q^T diag(gamma) dO - K^T diag(beta gamma) dR

    is the only serial part -- the same shape as the forward's chain with T
    transposed and two terms that do not depend on dS.  Every other gradient
    of the chunk follows from S, dS', dO and the chunk's own inputs, in
    parallel over chunks:

        dQ = diag(gamma) dO S^T + (dO U^T * Gamma) K
        dK = diag(f) U dS'^T - diag(beta gamma) dR S^T + (dO U^T * Gamma)^T Q
             + H K + H^T K,   H = dA * beta_r * Gamma,  dA = strict_lower(-dR U^T)
        dV = diag(beta) dR        (dU without erase)
        dbeta_r = sum_j dR (V - diag(gamma) K S) + sum_i dA (K K^T) Gamma
        dg = the decay's gradient through gamma, gamma_C, f and Gamma
             (Gamma_ri = exp(g_r - g_i): +row sums, -column sums), and
        dlog_alpha_i = sum over r >= i of dg_r   (g is the in-chunk cumsum).

    The T factor's gradient uses d(I + A)^-1 = -T dA T, which with U = T R
    collapses to dA = -dR U^T on the strictly lower triangle A occupies.
    """
    if mode not in MODES:
        raise ValueError(f"mode must be one of {MODES}, got {mode!r}")
    q, k, v, dO = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dO))
    B, H, L, dk = k.shape
    dv = v.shape[-1]
    erase, gated = mode in ERASE_MODES, mode in GATED_MODES
    bounds = [(s, min(s + C, L)) for s in range(0, L, C)]
    # forward: the state entering each chunk
    entry = []
    S = np.zeros((B, H, dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    for s, e in bounds:
        entry.append(S)
        _, S = chunkwise_fwd(q[:, :, s:e], k[:, :, s:e], v[:, :, s:e],
                             None if log_alpha is None else log_alpha[:, :, s:e],
                             None if beta is None else beta[:, :, s:e], S, mode, e - s)
    dq, dk_, dv_ = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dla, dbe = np.zeros((B, H, L)), np.zeros((B, H, L))
    dS = np.zeros((B, H, dk, dv)) if dS_final is None else np.array(dS_final, dtype=np.float64)
    tr = lambda x: np.swapaxes(x, -1, -2)     # noqa: E731
    for (s, e), S in zip(reversed(bounds), reversed(entry)):
        n = e - s
        Q, K, V, dOc = q[:, :, s:e], k[:, :, s:e], v[:, :, s:e], dO[:, :, s:e]
        la, be = _gates(None if log_alpha is None else log_alpha[:, :, s:e],
                        None if beta is None else beta[:, :, s:e], n, mode, K.shape[:-2])
        g = np.cumsum(la, axis=-1)
        gamma, Gamma = _decay(g)
        gC = g[..., -1:]
        f = np.exp(gC - g)
        QKt = np.matmul(Q, tr(K))
        P = QKt * Gamma
        KS = np.matmul(K, S)
        if erase:
            KKt = np.matmul(K, tr(K))
            A = np.tril(be[..., :, None] * KKt * Gamma, k=-1)
            T = forward_substitution_inverse(A)
            R = be[..., :, None] * (V - gamma[..., :, None] * KS)
            U = np.matmul(T, R)
        else:
            U = V
        # the output's and the carried state's direct terms
        QS = np.matmul(Q, S)
        dQ = gamma[..., :, None] * np.matmul(dOc, tr(S))
        dS_in = np.matmul(tr(Q), gamma[..., :, None] * dOc) + np.exp(gC)[..., None] * dS
        dgamma = np.sum(dOc * QS, axis=-1)
        dgC = np.sum(dS * S, axis=(-2, -1))
        dP = np.matmul(dOc, tr(U))
        KdS = np.matmul(K, dS)
        dU = np.matmul(tr(P), dOc) + f[..., :, None] * KdS
        dK = f[..., :, None] * np.matmul(U, tr(dS))
        df = np.sum(KdS * U, axis=-1)
        dGamma = dP * QKt
        if erase:
            dR = np.matmul(tr(T), dU)
            dA = np.tril(-np.matmul(dR, tr(U)), k=-1)
            dV = be[..., :, None] * dR
            dbe[:, :, s:e] = (np.sum(dR * (V - gamma[..., :, None] * KS), axis=-1)
                              + np.sum(dA * KKt * Gamma, axis=-1))
            bg = (be * gamma)[..., :, None]
            dS_in = dS_in - np.matmul(tr(K), bg * dR)
            dK = dK - bg * np.matmul(dR, tr(S))
            dgamma = dgamma - be * np.sum(dR * KS, axis=-1)
            Hm = dA * be[..., :, None] * Gamma
            dK = dK + np.matmul(Hm, K) + np.matmul(tr(Hm), K)
            dGamma = dGamma + dA * be[..., :, None] * KKt
        else:
            dV = dU
        E = dP * Gamma
        dQ = dQ + np.matmul(E, K)
        dK = dK + np.matmul(tr(E), Q)
        GG = dGamma * Gamma
        dg = GG.sum(-1) - GG.sum(-2) + dgamma * gamma - df * f
        dg[..., -1] += dgC * np.exp(gC[..., 0]) + np.sum(df * f, axis=-1)
        dla[:, :, s:e] = np.flip(np.cumsum(np.flip(dg, -1), axis=-1), -1)
        dq[:, :, s:e], dk_[:, :, s:e], dv_[:, :, s:e] = dQ, dK, dV
        dS = dS_in
    return dict(dq=dq, dk=dk_, dv=dv_, dlog_alpha=dla if gated else None,
                dbeta=dbe if erase else None, dS0=dS)
