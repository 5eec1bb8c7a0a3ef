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
library triangular solve, P to the explicit product of dk x dk factors
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
