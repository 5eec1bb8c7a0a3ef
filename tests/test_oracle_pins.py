"""Pins of the float64 oracle to facts the pages and the mathematics fix.

Each test ties the oracle to something other than itself: an independent
formula (the masked parallel form, a finite-difference gradient, an explicit
product of dk x dk factors, a library triangular solve), a closed form, an
exact-integer expansion, or an invariant.  Shapes use dk != dv so that a
transposed operand cannot pass unnoticed.

Sources: [HA-1] "混合注意力学习(1): 线性注意力" (jsqmd.com); [LA-OV]
"LinearAttention 概述" (razer666.cn); [CS336] "【CS336】lecture4 线性注意力|
Mamba|GDN|DSA" (wsisp.com).
"""

import numpy as np
import pytest
import scipy.linalg

import oracle
from oracle import (chunkwise_fwd, decode_steps, forward_substitution_inverse,
                    parallel_masked_linear, recurrent_fwd, recurrent_step,
                    ut_transform, wy_transition)


def _rand(seed, B=2, H=3, L=13, dk=5, dv=3, unit_keys=True, s0=0.3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, L, dk))
    k = rng.standard_normal((B, H, L, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, L, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, H, L))))
    log_alpha = -np.log1p(np.exp(rng.standard_normal((B, H, L)))) / 4.0
    S0 = s0 * rng.standard_normal((B, H, dk, dv))
    return q, k, v, log_alpha, beta, S0


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# ---------------------------------------------------------------- linear mode

def test_linear_recurrence_equals_masked_parallel_form():
    """[HA-1 "传统FWP形式的线性注意力并行"; LA-OV "快速预览"]: stacking the
    rows, causal linear attention is (Q K^T * M) V; with a zero initial state
    the final state is K^T V (the sum of all writes)."""
    q, k, v, la, be, _ = _rand(1, L=17, dk=6, dv=4, unit_keys=False)
    o, S = recurrent_fwd(q, k, v, la, be, None, "linear")
    assert _rel(o, parallel_masked_linear(q, k, v)) < 1e-13
    assert _rel(S, np.swapaxes(k, -1, -2) @ v) < 1e-13


def test_linear_four_token_cumsum_example_exact_integers():
    """[LA-OV "Lightning Attention"] expands the causal sum for four tokens:
    output t is q_t times the running sum of k_j^T v_j over j <= t.  With
    small integer inputs float64 is exact, so the oracle must match the
    expansion evaluated in Python integers with equality."""
    rng = np.random.default_rng(7)
    d_k, d_v = 3, 2
    qi = rng.integers(-4, 5, size=(4, d_k))
    ki = rng.integers(-4, 5, size=(4, d_k))
    vi = rng.integers(-4, 5, size=(4, d_v))
    expect = []
    for t in range(4):
        row = []
        for c in range(d_v):
            # q_t (k_1^T v_1 + ... + k_t^T v_t), entry c
            row.append(sum(int(qi[t, a]) * int(ki[j, a]) * int(vi[j, c])
                           for j in range(t + 1) for a in range(d_k)))
        expect.append(row)
    o, _ = recurrent_fwd(qi[None, None].astype(float), ki[None, None].astype(float),
                         vi[None, None].astype(float), None, None, None, "linear")
    assert np.array_equal(o[0, 0], np.array(expect, dtype=float))


def test_linear_never_forgets_same_key_twice():
    """[HA-1 "Fast Weight Programmers与DeltaNet"]: the plain update only adds,
    so writing the same unit key twice returns the sum of both values, while
    the delta rule with beta = 1 returns the latest value."""
    k1 = np.array([0.0, 1.0, 0.0, 0.0])
    v1 = np.array([1.0, -2.0, 0.5])
    v2 = np.array([3.0, 0.25, -1.0])
    k = np.stack([k1, k1])[None, None]
    v = np.stack([v1, v2])[None, None]
    q = k.copy()
    beta = np.ones((1, 1, 2))
    o_lin, _ = recurrent_fwd(q, k, v, None, None, None, "linear")
    o_del, _ = recurrent_fwd(q, k, v, None, beta, None, "delta")
    assert np.allclose(o_lin[0, 0, 1], v1 + v2, rtol=0, atol=1e-15)
    assert np.allclose(o_del[0, 0, 1], v2, rtol=0, atol=1e-15)


# ---------------------------------------------------------------- delta rule

def _fd_grad(S, k, v, h=1e-6):
    """Central-difference gradient of 0.5 ||S^T k - v||^2 over S's entries."""
    G = np.zeros_like(S)
    for i in range(S.shape[0]):
        for j in range(S.shape[1]):
            Sp = S.copy()
            Sm = S.copy()
            Sp[i, j] += h
            Sm[i, j] -= h
            lp = 0.5 * np.sum((Sp.T @ k - v) ** 2)
            lm = 0.5 * np.sum((Sm.T @ k - v) ** 2)
            G[i, j] = (lp - lm) / (2 * h)
    return G


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_delta_step_is_gradient_step_on_reconstruction_loss(seed):
    """[HA-1 "Fast Weight Programmers与DeltaNet"]: the delta rule is one
    gradient-descent step, with the learned rate beta, on the reconstruction
    loss of the value from the key.  The gradient here comes from finite
    differences, not from the update formula."""
    rng = np.random.default_rng(seed)
    dk, dv = 5, 3
    S = rng.standard_normal((dk, dv))
    k = rng.standard_normal(dk)          # any norm: the identity is exact
    v = rng.standard_normal(dv)
    q = rng.standard_normal(dk)
    beta = 0.37
    S_new, o = recurrent_step(S, q, k, v, None, beta, "delta")
    expect = S - beta * _fd_grad(S, k, v)
    assert np.max(np.abs(S_new - expect)) < 1e-7
    assert np.max(np.abs(o - S_new.T @ q)) < 1e-14


@pytest.mark.parametrize("seed", [3, 4])
def test_gated_delta_step_is_decay_then_gradient_step(seed):
    """[HA-1 "Gated DeltaNet"; CS336 "继续改进：GDN"]: the gated rule decays the
    whole state by alpha (Mamba2-style weight decay) and then takes the delta
    step; equivalently a gradient step on the loss evaluated at alpha S.
    The decay therefore scales the erase term too, but not the new write."""
    rng = np.random.default_rng(seed)
    dk, dv = 4, 6
    S = rng.standard_normal((dk, dv))
    k = rng.standard_normal(dk)
    k /= np.linalg.norm(k)
    v = rng.standard_normal(dv)
    q = rng.standard_normal(dk)
    beta, log_alpha = 0.8, -0.3
    a = np.exp(log_alpha)
    S_new, _ = recurrent_step(S, q, k, v, log_alpha, beta, "gated_delta")
    expect = a * S - beta * _fd_grad(a * S, k, v)
    assert np.max(np.abs(S_new - expect)) < 1e-7


def test_delta_blend_reading_matches_update():
    """[HA-1 "Fast Weight Programmers与DeltaNet"] describes the rule as: read
    the old value under k, blend it with the new one by beta, remove the old
    association and write the blended one.  Written out step by step this
    equals the oracle's update for any key norm."""
    rng = np.random.default_rng(11)
    dk, dv = 6, 2
    S = rng.standard_normal((dk, dv))
    k = 1.7 * rng.standard_normal(dk)
    v = rng.standard_normal(dv)
    beta = 0.61
    v_old = S.T @ k
    v_new = beta * v + (1.0 - beta) * v_old
    S_blend = S - np.outer(k, v_old) + np.outer(k, v_new)
    S_new, _ = recurrent_step(S, np.zeros(dk), k, v, None, beta, "delta")
    assert np.max(np.abs(S_new - S_blend)) < 1e-13


def test_delta_exact_retrieval_with_orthonormal_keys():
    """With beta = 1 and orthonormal keys each write replaces exactly what is
    stored under its key and leaves the other keys untouched, so querying
    with an earlier key returns its value, whatever the initial state
    (the delta rule's erase-then-write, [HA-1 "Fast Weight Programmers与
    DeltaNet"]).  Plain linear attention fails this when S0 != 0."""
    rng = np.random.default_rng(5)
    dk, dv, n = 7, 3, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm[:, :n].T                                  # n orthonormal rows
    vals = rng.standard_normal((n, dv))
    S0 = rng.standard_normal((1, 1, dk, dv))
    # token t queries with key j(t) <= t
    j_of_t = [0, 0, 1, 2, 1, 4]
    q = keys[j_of_t][None, None]
    k = keys[None, None]
    v = vals[None, None]
    beta = np.ones((1, 1, n))
    o, _ = recurrent_fwd(q, k, v, None, beta, S0, "delta")
    assert np.max(np.abs(o[0, 0] - vals[j_of_t])) < 1e-13
    o_g, _ = recurrent_fwd(q, k, v, np.zeros((1, 1, n)), beta, S0, "gated_delta")
    assert np.max(np.abs(o_g - o)) < 1e-15             # alpha = 1
    o_lin, _ = recurrent_fwd(q, k, v, None, None, S0, "linear")
    assert np.max(np.abs(o_lin[0, 0] - vals[j_of_t])) > 1e-3


def test_householder_reflection_preserves_state_norm():
    """[HA-1 "HouseHolder变换和WY表示"]: I - 2 k k^T / (k^T k) is a Householder
    reflection, orthogonal.  With beta = 2, unit keys, alpha = 1 and zero
    values every delta step applies one reflection, so the Frobenius norm of
    every column of the state is preserved and a reflected key flips sign."""
    rng = np.random.default_rng(9)
    dk, dv, L = 6, 4, 11
    k = rng.standard_normal((1, 1, L, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    S0 = rng.standard_normal((1, 1, dk, dv))
    zeros_v = np.zeros((1, 1, L, dv))
    beta = 2.0 * np.ones((1, 1, L))
    _, S = recurrent_fwd(np.zeros((1, 1, L, dk)), k, zeros_v, None, beta, S0, "delta")
    assert np.allclose(np.linalg.norm(S, axis=-2), np.linalg.norm(S0, axis=-2),
                       rtol=1e-13, atol=0)
    kk = k[0, 0, 0]
    S1, _ = recurrent_step(kk[:, None] * np.ones((1, dv)), np.zeros(dk), kk,
                           np.zeros(dv), None, 2.0, "delta")
    assert np.allclose(S1, -kk[:, None] * np.ones((1, dv)), atol=1e-15)


def test_gate_closed_forms():
    """Closed forms of the gated rule: with beta = 0 nothing is written or
    erased, so o_t = gamma_t S0^T q_t with gamma_t the running product of the
    decays; with alpha -> 0 all history is dropped and o_t = beta_t
    (q_t . k_t) v_t."""
    q, k, v, la, be, S0 = _rand(21, L=9, dk=4, dv=5)
    o, S = recurrent_fwd(q, k, v, la, np.zeros_like(be), S0, "gated_delta")
    gamma = np.exp(np.cumsum(la, axis=-1))
    expect = gamma[..., None] * np.einsum("bhij,bhti->bhtj", S0, q)
    assert _rel(o, expect) < 1e-13
    assert _rel(S, gamma[..., -1, None, None] * S0) < 1e-13
    la_zero = np.full_like(la, -1e30)                    # exp -> exactly 0
    o2, _ = recurrent_fwd(q, k, v, la_zero, be, S0, "gated_delta")
    expect2 = be[..., None] * np.sum(q * k, axis=-1)[..., None] * v
    assert _rel(o2, expect2) < 1e-14


def test_scalar_state_by_hand():
    """dk = dv = 1: the gated rule reads s <- alpha (1 - beta k^2) s + beta k v
    and o = s q; evaluated here with plain Python floats."""
    rng = np.random.default_rng(13)
    L = 8
    q, k, v = (rng.standard_normal(L) for _ in range(3))
    la = -np.abs(rng.standard_normal(L)) / 3
    be = rng.uniform(0, 1, L)
    s = 0.7
    want = []
    for t in range(L):
        a = float(np.exp(la[t]))
        s = a * (1.0 - be[t] * k[t] * k[t]) * s + be[t] * k[t] * v[t]
        want.append(s * q[t])
    o, S = recurrent_fwd(q[None, None, :, None], k[None, None, :, None],
                         v[None, None, :, None], la[None, None], be[None, None],
                         np.array([[[[0.7]]]]), "gated_delta")
    assert np.allclose(o[0, 0, :, 0], want, rtol=1e-14, atol=0)
    assert abs(S[0, 0, 0, 0] - s) < 1e-14


# ---------------------------------------------------------------- gated linear

def _gated_linear_by_loops(q, k, v, la, S0):
    """o_t = (prod_{u<=t} alpha_u) S0^T q_t
             + sum_{s<=t} (prod_{s<u<=t} alpha_u) (q_t . k_s) v_s
    and the final state, evaluated with explicit loops over t and s and
    running products of the gates (no cumulative sums, no exponent
    differences)."""
    B, H, L, dk = k.shape
    dv = v.shape[-1]
    alpha = np.exp(la)
    o = np.zeros((B, H, L, dv))
    S = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            for t in range(L):
                w0 = 1.0
                for u in range(t + 1):
                    w0 *= alpha[b, h, u]
                acc = w0 * (S0[b, h].T @ q[b, h, t])
                for s_ in range(t + 1):
                    w = 1.0
                    for u in range(s_ + 1, t + 1):
                        w *= alpha[b, h, u]
                    acc = acc + w * float(q[b, h, t] @ k[b, h, s_]) * v[b, h, s_]
                o[b, h, t] = acc
            wL = 1.0
            for u in range(L):
                wL *= alpha[b, h, u]
            Sbh = wL * S0[b, h]
            for s_ in range(L):
                w = 1.0
                for u in range(s_ + 1, L):
                    w *= alpha[b, h, u]
                Sbh = Sbh + w * np.outer(k[b, h, s_], v[b, h, s_])
            S[b, h] = Sbh
    return o, S


def test_gated_linear_equals_gate_weighted_sum():
    """[HA-1 "Gated DeltaNet"; CS336 "继续改进：Mamba"]: multiplying the state
    by alpha_t before each write makes output t the causal sum of the writes,
    each weighted by the product of the gates applied after it, plus the
    initial state decayed by all gates so far."""
    q, k, v, la, be, S0 = _rand(61, B=1, H=2, L=11, dk=4, dv=3, unit_keys=False)
    o, S = recurrent_fwd(q, k, v, la, be, S0, "gated_linear")
    o_ref, S_ref = _gated_linear_by_loops(q, k, v, la, S0)
    assert _rel(o, o_ref) < 1e-13
    assert _rel(S, S_ref) < 1e-13


def test_gated_linear_special_cases():
    """alpha = 1 is plain linear attention; alpha -> 0 keeps only the token's
    own write, o_t = (q_t . k_t) v_t; beta is ignored."""
    q, k, v, la, be, S0 = _rand(62, L=9, dk=4, dv=5)
    a, Sa = recurrent_fwd(q, k, v, np.zeros_like(la), be, S0, "gated_linear")
    b, Sb = recurrent_fwd(q, k, v, None, None, S0, "linear")
    assert _rel(a, b) < 1e-15 and _rel(Sa, Sb) < 1e-15
    o0, _ = recurrent_fwd(q, k, v, np.full_like(la, -1e30), be, S0, "gated_linear")
    assert _rel(o0, np.sum(q * k, axis=-1)[..., None] * v) < 1e-14
    c, _ = recurrent_fwd(q, k, v, la, None, S0, "gated_linear")
    d, _ = recurrent_fwd(q, k, v, la, be, S0, "gated_linear")
    assert np.array_equal(c, d)
    with pytest.raises(ValueError):
        recurrent_fwd(q, k, v, None, be, S0, "gated_linear")


def test_gated_linear_scalar_by_hand():
    """dk = dv = 1: s <- alpha s + k v, o = s q, with plain Python floats."""
    rng = np.random.default_rng(63)
    L = 7
    q, k, v = (rng.standard_normal(L) for _ in range(3))
    la = -np.abs(rng.standard_normal(L)) / 2
    s = -0.4
    want = []
    for t in range(L):
        s = float(np.exp(la[t])) * s + k[t] * v[t]
        want.append(s * q[t])
    o, S = recurrent_fwd(q[None, None, :, None], k[None, None, :, None],
                         v[None, None, :, None], la[None, None], None,
                         np.array([[[[-0.4]]]]), "gated_linear")
    assert np.allclose(o[0, 0, :, 0], want, rtol=1e-14, atol=0)
    assert abs(S[0, 0, 0, 0] - s) < 1e-14


# ---------------------------------------------------------------- chunkwise

@pytest.mark.parametrize("mode", oracle.MODES)
@pytest.mark.parametrize("C", [1, 3, 7, 16, 32])
def test_chunkwise_is_exact_for_every_chunk_size(mode, C):
    """[LA-OV "FLASH"; HA-1 "FWP分块并行机制"]: the chunkwise form equals the
    recurrent form for any chunk size (C = 1 is the recurrent form, C = L the
    parallel one), including a ragged last chunk (C = 3, 7 do not divide 32).
    Exact in exact arithmetic; float64 round-off here."""
    q, k, v, la, be, S0 = _rand(100 + C, L=32, dk=6, dv=5)
    o_ref, S_ref = recurrent_fwd(q, k, v, la, be, S0, mode)
    o, S = chunkwise_fwd(q, k, v, la, be, S0, mode, C)
    assert _rel(o, o_ref) < 1e-12
    assert _rel(S, S_ref) < 1e-12


def test_chunkwise_linear_single_chunk_is_parallel_form():
    """C = L with a zero state is exactly the masked parallel form."""
    q, k, v, la, be, _ = _rand(31, L=12, dk=4, dv=6, unit_keys=False)
    o, _ = chunkwise_fwd(q, k, v, la, be, None, "linear", 12)
    assert _rel(o, parallel_masked_linear(q, k, v)) < 1e-13


def test_forward_substitution_matches_library_triangular_solve():
    """T = (I + A)^{-1} for strictly lower A, checked against SciPy's
    triangular solve (a textbook routine, independent of the loop)."""
    rng = np.random.default_rng(17)
    for C in (1, 5, 16, 64):
        A = np.tril(rng.standard_normal((C, C)) * 0.2, k=-1)
        T = forward_substitution_inverse(A)
        ref = scipy.linalg.solve_triangular(np.eye(C) + A, np.eye(C), lower=True,
                                            unit_diagonal=True)
        assert np.max(np.abs(T - ref)) < 1e-12


@pytest.mark.parametrize("mode", ["delta", "gated_delta"])
def test_wy_representation_equals_product_of_factors(mode):
    """[HA-1 "HouseHolder变换和WY表示"]: a product of rank-1 corrections is
    the identity minus a low-rank product.  For one chunk the WY/UT form
    gamma_C I - (diag(gamma_C/gamma) K)^T W must equal the explicit product
    of dk x dk factors alpha_r (I - beta_r k_r k_r^T), latest on the left.
    dk = 9 > n = 6 so the product is a genuine rank-6 correction."""
    rng = np.random.default_rng(23)
    n, dk = 6, 9
    k = rng.standard_normal((n, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    beta = rng.uniform(0.1, 1.0, n)
    la = -rng.uniform(0.0, 0.5, n) if mode == "gated_delta" else None
    P = np.eye(dk)
    for r in range(n):
        a = 1.0 if la is None else np.exp(la[r])
        P = a * (np.eye(dk) - beta[r] * np.outer(k[r], k[r])) @ P
    assert np.max(np.abs(wy_transition(k, la, beta, mode) - P)) < 1e-13
    # and T from the transform solves the unit lower-triangular system
    ut = ut_transform(k, np.zeros((n, 1)), la, beta, mode)
    assert np.max(np.abs((np.eye(n) + ut["A"]) @ ut["T"] - np.eye(n))) < 1e-13


# ---------------------------------------------------------------- carry / decode

@pytest.mark.parametrize("mode", oracle.MODES)
def test_state_carry_and_decode_match_forward(mode):
    """Only the fixed-size state is carried between calls [CS336 "朴素线性注意力"]:
    a forward over L1 tokens followed by one over L2 tokens started from its
    final state equals one forward over L1 + L2; L single decode steps equal
    the forward over the same L tokens [HA-1 "Prefill、Decode与KVCache"]."""
    q, k, v, la, be, S0 = _rand(41, L=20, dk=5, dv=4)
    o_ref, S_ref = recurrent_fwd(q, k, v, la, be, S0, mode)
    o1, S1 = chunkwise_fwd(q[:, :, :8], k[:, :, :8], v[:, :, :8], la[:, :, :8],
                           be[:, :, :8], S0, mode, 4)
    o2, S2 = chunkwise_fwd(q[:, :, 8:], k[:, :, 8:], v[:, :, 8:], la[:, :, 8:],
                           be[:, :, 8:], S1, mode, 5)
    assert _rel(np.concatenate([o1, o2], axis=2), o_ref) < 1e-12
    assert _rel(S2, S_ref) < 1e-12
    tq = np.moveaxis(q, 2, 0)
    od, Sd = decode_steps(S0, tq, np.moveaxis(k, 2, 0), np.moveaxis(v, 2, 0),
                          np.moveaxis(la, 2, 0), np.moveaxis(be, 2, 0), mode)
    assert _rel(np.moveaxis(od, 0, 2), o_ref) < 1e-14
    assert _rel(Sd, S_ref) < 1e-14


@pytest.mark.parametrize("mode", oracle.MODES)
def test_segment_state_is_affine_in_start_state(mode):
    """Every token's update is affine in the state, so a run of tokens maps
    its start state to M S_start + X: X the end state from a zero start, M
    (dk x dk) the end state of the same run with V = 0 from the identity --
    a scalar exp(sum of log alpha) times the identity when nothing is erased.
    Cutting a sequence into segments, computing X and M of each from the
    tokens alone and chaining S_in(p+1) = M_p S_in(p) + X_p gives every
    segment's true start state; running the segments from those reproduces
    the whole forward.  This is the decomposition behind the
    sequence-parallel forward (the chunkwise form holds for any cut of the
    sequence [LA-OV "FLASH"]; the inter-block part is carried by the state
    alone [LA-OV "Lightning Attention"])."""
    dk = dv = 4
    q, k, v, la, be, S0 = _rand(43, B=1, H=2, L=23, dk=dk, dv=dv)
    o_ref, S_ref = recurrent_fwd(q, k, v, la, be, S0, mode)
    cuts = [0, 6, 7, 15, 23]
    eye = np.broadcast_to(np.eye(dk), (1, 2, dk, dk))
    S_in, outs = S0, []
    for a, b in zip(cuts[:-1], cuts[1:]):
        seg = lambda t: t[:, :, a:b]          # noqa: E731
        _, X = recurrent_fwd(seg(q), seg(k), seg(v), seg(la), seg(be),
                             np.zeros_like(S0), mode)
        _, M = recurrent_fwd(seg(q), seg(k), np.zeros((1, 2, b - a, dk)), seg(la), seg(be),
                             eye, mode)
        if mode not in oracle.ERASE_MODES:
            g = la[:, :, a:b].sum(-1) if mode in oracle.GATED_MODES else np.zeros((1, 2))
            assert _rel(M, np.exp(g)[..., None, None] * eye) < 1e-14
        # the true run from S_in: outputs and M S_in + X
        o, S_end = recurrent_fwd(seg(q), seg(k), seg(v), seg(la), seg(be), S_in, mode)
        assert _rel(np.einsum("bhij,bhjc->bhic", M, S_in) + X, S_end) < 1e-13
        outs.append(o)
        S_in = np.einsum("bhij,bhjc->bhic", M, S_in) + X
    assert _rel(np.concatenate(outs, axis=2), o_ref) < 1e-13
    assert _rel(S_in, S_ref) < 1e-13


def test_modes_ignore_unused_gates():
    """linear ignores beta and alpha; delta ignores alpha (gated_linear's
    beta: test_gated_linear_special_cases)."""
    q, k, v, la, be, S0 = _rand(51, L=6)
    a, _ = recurrent_fwd(q, k, v, la, be, S0, "linear")
    b, _ = recurrent_fwd(q, k, v, None, None, S0, "linear")
    assert np.array_equal(a, b)
    c, _ = recurrent_fwd(q, k, v, la, be, S0, "delta")
    d, _ = recurrent_fwd(q, k, v, np.zeros_like(la), be, S0, "gated_delta")
    assert _rel(c, d) < 1e-15
    with pytest.raises(ValueError):
        recurrent_fwd(q, k, v, la, None, S0, "delta")
    with pytest.raises(ValueError):
        recurrent_fwd(q, k, v, la, be, S0, "softmax")


# ---------------------------------------------------------------- fused prologue

def test_gate_activations_closed_forms():
    """sigmoid and softplus against values fixed by their definitions:
    sigmoid(0) = 1/2, sigmoid(log 3) = 3/4, sigmoid(x) + sigmoid(-x) = 1;
    softplus(0) = log 2, softplus(log(e - 1)) = 1, softplus(a) - softplus(-a)
    = a; far from 0 they saturate (0 and 1; 0 and a) without overflow."""
    from oracle.prologue import sigmoid, softplus
    assert sigmoid(0.0) == 0.5
    assert abs(sigmoid(np.log(3.0)) - 0.75) < 1e-15
    x = np.linspace(-30, 30, 121)
    assert np.max(np.abs(sigmoid(x) + sigmoid(-x) - 1.0)) < 1e-15
    assert abs(softplus(0.0) - np.log(2.0)) < 1e-16
    assert abs(softplus(np.log(np.e - 1.0)) - 1.0) < 1e-15
    assert np.max(np.abs(softplus(x) - softplus(-x) - x)) < 1e-13
    assert sigmoid(-800.0) == 0.0 and sigmoid(800.0) == 1.0
    assert softplus(-800.0) == 0.0 and softplus(800.0) == 800.0


def test_l2_normalise_closed_form():
    """|x / sqrt(|x|^2 + eps)|^2 = |x|^2 / (|x|^2 + eps) exactly, per token
    (last axis only); the zero vector stays zero."""
    from oracle.prologue import QK_NORM_EPS, l2_normalise
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 4, 7, 6)) * rng.uniform(0.01, 10.0, (3, 4, 7, 1))
    y = l2_normalise(x)
    n2 = np.sum(x * x, axis=-1)
    assert _rel(np.sum(y * y, axis=-1), n2 / (n2 + QK_NORM_EPS)) < 1e-14
    # the direction is kept: y is a positive multiple of x, token by token
    ratio = y / x
    assert np.max(np.abs(ratio - ratio[..., :1])) < 1e-12 and np.all(ratio > 0)
    assert np.all(l2_normalise(np.zeros((2, 5))) == 0.0)


@pytest.mark.parametrize("mode", oracle.MODES)
def test_prologue_makes_op_scale_invariant(mode):
    """With q and k normalised inside, scaling any token's q or k by a
    positive factor leaves the outputs and the state unchanged (up to the
    eps inside the root): a normalisation over the wrong axis, or by the
    sum instead of the norm, fails this.  The activated gates are a decay in
    (0, 1] and a write strength in (0, 1)."""
    from oracle.prologue import GATES, QK_L2NORM, prepare
    q, k, v, _, _, S0 = _rand(47, B=1, H=2, L=17, dk=6, dv=5, unit_keys=False)
    rng = np.random.default_rng(48)
    a, b = rng.standard_normal((2, 1, 2, 17))
    flags = GATES | QK_L2NORM
    o1, S1 = recurrent_fwd(*_prepared(q, k, v, a, b, mode, flags), S0, mode)
    sq = rng.uniform(0.2, 5.0, (1, 2, 17, 1))
    sk = rng.uniform(0.2, 5.0, (1, 2, 17, 1))
    o2, S2 = recurrent_fwd(*_prepared(q * sq, k * sk, v, a, b, mode, flags), S0, mode)
    # each normalised vector moves by at most about eps / |x|^2 relative
    n2 = min(np.min(np.sum(x * x, -1)) for x in (q, k, q * sq, k * sk))
    tol = 50 * 1e-6 / n2
    assert _rel(o2, o1) < tol and _rel(S2, S1) < tol
    # without the normalisation the same scaling changes the result
    o3, _ = recurrent_fwd(*_prepared(q * sq, k * sk, v, a, b, mode, GATES), S0, mode)
    o4, _ = recurrent_fwd(*_prepared(q, k, v, a, b, mode, GATES), S0, mode)
    assert _rel(o3, o4) > 1e-2
    _, _, la, be = prepare(q, k, a, b, mode, flags, 0.25)
    if mode in oracle.GATED_MODES:
        assert np.all(la <= 0.0) and np.all(la >= -0.25 * (np.abs(a) + 1.0))
    if mode in oracle.ERASE_MODES:
        assert np.all((be > 0.0) & (be < 1.0))


def _prepared(q, k, v, a, b, mode, flags):
    from oracle.prologue import prepare
    qq, kk, la, be = prepare(q, k, a, b, mode, flags, 1.0 / 16.0)
    return qq, kk, v, la, be


# ---------------------------------------------------------------- fused epilogue

def test_dskip_worked_example():
    """o + D v per (head, channel): a hand-computed case with two heads, so a
    D applied per token, per batch or transposed fails."""
    from oracle.epilogue import add_dskip
    o = np.array([[[[1.0, 2.0]], [[0.0, -1.0]]]])       # [B=1, H=2, L=1, dv=2]
    v = np.array([[[[3.0, 4.0]], [[2.0, 5.0]]]])
    D = np.array([[0.5, -1.0], [2.0, 0.25]])            # [H, dv]
    want = np.array([[[[2.5, -2.0]], [[4.0, 0.25]]]])
    assert np.array_equal(add_dskip(o, v, D), want)


def test_out_norm_closed_form():
    """With unit weights the normalised row has mean square m / (m + eps),
    m the row's mean square, and keeps each element's sign and ratio; a
    weight multiplies channel by channel, per head; the norm is taken over
    the value channels only (scaling one token's row leaves the others)."""
    from oracle.epilogue import out_norm
    rng = np.random.default_rng(9)
    o = rng.standard_normal((2, 3, 5, 8)) * rng.uniform(0.01, 10.0, (2, 3, 5, 1))
    eps = 1e-3
    y = out_norm(o, eps=eps)
    m = np.mean(o * o, axis=-1)
    assert _rel(np.mean(y * y, axis=-1), m / (m + eps)) < 1e-14
    assert np.all(np.sign(y) == np.sign(o))
    w = rng.uniform(0.5, 2.0, (3, 8))
    assert _rel(out_norm(o, w, eps), y * w[None, :, None, :]) < 1e-15
    o2 = o.copy()
    o2[1, 2, 3] *= 7.0
    y2 = out_norm(o2, eps=eps)
    mask = np.ones(o.shape[:3], bool)
    mask[1, 2, 3] = False
    assert np.array_equal(y2[mask], y[mask])


# ---------------------------------------------------------------- non-causal form

def test_noncausal_orders_and_causal_last_token():
    """O = Q (S0 + K^T V) equals the other evaluation order (Q K^T) V + Q S0
    [LA-OV "快速预览"]; its state is the causal LINEAR recurrence's final
    state, and its last token's output the causal last output (both see the
    whole sequence) -- while earlier tokens differ (they see the future)."""
    from oracle.noncausal import noncausal_fwd
    q, k, v, _, _, S0 = _rand(53, B=2, H=2, L=11, dk=4, dv=3, unit_keys=False)
    o, S = noncausal_fwd(q, k, v, S0)
    qk = np.einsum("bhtd,bhsd->bhts", q, k)
    assert _rel(o, np.einsum("bhts,bhsv->bhtv", qk, v) + np.einsum("bhtd,bhdv->bhtv", q, S0)) < 1e-13
    o_c, S_c = recurrent_fwd(q, k, v, None, None, S0, "linear")
    assert _rel(S, S_c) < 1e-13
    assert _rel(o[:, :, -1], o_c[:, :, -1]) < 1e-13
    assert _rel(o[:, :, 0], o_c[:, :, 0]) > 1e-3


# ---------------------------------------------------------------- backward

def _loss(q, k, v, la, be, S0, mode, dO, dSf):
    o, S = recurrent_fwd(q, k, v, la, be, S0, mode)
    return float(np.sum(o * dO) + np.sum(S * dSf))


@pytest.mark.parametrize("mode", oracle.MODES)
def test_backward_matches_finite_differences(mode):
    """Every gradient of sum(dO * O) + sum(dS_final * S_final) against
    central finite differences of the forward, element by element, on a
    tiny case (non-unit keys, beta and alpha away from their limits)."""
    from oracle.backward import recurrent_bwd
    q, k, v, la, be, S0 = _rand(61, B=1, H=2, L=6, dk=3, dv=2, unit_keys=False)
    rng = np.random.default_rng(62)
    dO = rng.standard_normal((1, 2, 6, 2))
    dSf = rng.standard_normal((1, 2, 3, 2))
    g = recurrent_bwd(q, k, v, la, be, S0, mode, dO, dSf)
    args = dict(q=q, k=k, v=v, la=la, be=be, S0=S0)
    names = dict(q="dq", k="dk", v="dv", S0="dS0")
    if mode in oracle.GATED_MODES:
        names["la"] = "dlog_alpha"
    if mode in oracle.ERASE_MODES:
        names["be"] = "dbeta"
    h = 1e-6
    for name, gname in names.items():
        x = args[name]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            lp = _loss(**{**args, name: xp}, mode=mode, dO=dO, dSf=dSf)
            lm = _loss(**{**args, name: xm}, mode=mode, dO=dO, dSf=dSf)
            num[idx] = (lp - lm) / (2 * h)
        assert _rel(g[gname], num) < 1e-7, (name, _rel(g[gname], num))
    if mode not in oracle.GATED_MODES:
        assert g["dlog_alpha"] is None
    if mode not in oracle.ERASE_MODES:
        assert g["dbeta"] is None


def test_backward_linear_closed_forms():
    """Causal linear attention O = (Q K^T * M) V + Q S0 has dV = (Q K^T *
    M)^T dO, dQ = (dO V^T * M) K + dO S0^T, dK = (dO V^T * M)^T Q and dS0 =
    Q^T dO (S0 reaches every output through o_t += S0^T q_t)."""
    from oracle.backward import recurrent_bwd
    q, k, v, _, _, S0 = _rand(63, B=2, H=1, L=9, dk=4, dv=3, unit_keys=False)
    dO = np.random.default_rng(64).standard_normal((2, 1, 9, 3))
    g = recurrent_bwd(q, k, v, None, None, S0, "linear", dO)
    M = np.tril(np.ones((9, 9)))
    A = np.einsum("bhtd,bhsd->bhts", q, k) * M
    dA = np.einsum("bhtv,bhsv->bhts", dO, v) * M
    assert _rel(g["dv"], np.einsum("bhts,bhtv->bhsv", A, dO)) < 1e-13
    dq = np.einsum("bhts,bhsd->bhtd", dA, k) + np.einsum("bhtv,bhdv->bhtd", dO, S0)
    assert _rel(g["dq"], dq) < 1e-13
    assert _rel(g["dk"], np.einsum("bhts,bhtd->bhsd", dA, q)) < 1e-13
    assert _rel(g["dS0"], np.einsum("bhtd,bhtv->bhdv", q, dO)) < 1e-13


@pytest.mark.parametrize("mode", oracle.MODES)
@pytest.mark.parametrize("C", [1, 3, 7, 16, 29])
def test_chunkwise_backward_equals_token_backward(mode, C):
    """The chunkwise backward (per-chunk entry states, a reverse chain over
    chunks with T transposed, parallel per-chunk gradients, dA = -dR U^T
    through the triangular inverse, decay gradients summed back through the
    in-chunk cumsum) gives the token backward's gradients for every chunk
    size, ragged last chunk included."""
    from oracle.backward import recurrent_bwd
    q, k, v, la, be, S0 = _rand(71, B=2, H=1, L=29, dk=4, dv=3, unit_keys=True)
    rng = np.random.default_rng(72)
    dO = rng.standard_normal((2, 1, 29, 3))
    dSf = rng.standard_normal((2, 1, 4, 3))
    ref = recurrent_bwd(q, k, v, la, be, S0, mode, dO, dSf)
    got = oracle.chunkwise_bwd(q, k, v, la, be, S0, mode, C, dO, dSf)
    for name in ("dq", "dk", "dv", "dS0", "dlog_alpha", "dbeta"):
        if ref[name] is None:
            assert got[name] is None
            continue
        assert _rel(got[name], ref[name]) < 1e-11, (name, _rel(got[name], ref[name]))


@pytest.mark.parametrize("flags", [1, 2, 3])
@pytest.mark.parametrize("mode", oracle.MODES)
def test_prologue_backward_matches_finite_differences(mode, flags):
    """The gradients of the raw inputs through the fused prologue (q, k
    normalisation, gate activations) composed with the recurrence's
    backward, against central finite differences of the loss taken through
    prepare and the recurrence, element by element, on a tiny case."""
    from oracle.backward import recurrent_bwd
    rng = np.random.default_rng(71 + flags)
    B, H, L, dk, dv = 1, 2, 5, 3, 2
    q = rng.standard_normal((B, H, L, dk))
    k = rng.standard_normal((B, H, L, dk))
    v = rng.standard_normal((B, H, L, dv))
    a = rng.standard_normal((B, H, L)) if flags & 1 else -0.05 + 0.01 * rng.standard_normal((B, H, L))
    b = rng.standard_normal((B, H, L)) if flags & 1 else 0.3 + 0.4 * rng.random((B, H, L))
    S0 = 0.1 * rng.standard_normal((B, H, dk, dv))
    dO = rng.standard_normal((B, H, L, dv))
    dSf = rng.standard_normal((B, H, dk, dv))
    scale = 0.4

    def loss(q, k, a, b):
        qp, kp, la, be = oracle.prepare(q, k, a, b, mode, flags, scale)
        return _loss(qp, kp, v, la, be, S0, mode, dO, dSf)

    qp, kp, la, be = oracle.prepare(q, k, a, b, mode, flags, scale)
    g = recurrent_bwd(qp, kp, v, la, be, S0, mode, dO, dSf)
    dq, dk_, da, db = oracle.prologue_bwd(q, k, a, b, mode, flags, scale, g["dq"], g["dk"],
                                          g["dlog_alpha"], g["dbeta"])
    args = dict(q=q, k=k, a=a, b=b)
    want = dict(q=dq, k=dk_)
    if mode in oracle.GATED_MODES:
        want["a"] = da
    if mode in oracle.ERASE_MODES:
        want["b"] = db
    h = 1e-6
    for name, grad in want.items():
        x = args[name]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            num[idx] = (loss(**{**args, name: xp}) - loss(**{**args, name: xm})) / (2 * h)
        assert _rel(grad, num) < 1e-7, (name, _rel(grad, num))


@pytest.mark.parametrize("mode", oracle.MODES)
def test_checkpointed_token_backward_is_bit_identical(mode):
    """Keeping only every n-th state and recomputing each run of n tokens
    repeats the forward's own steps, so the gradients equal those of the
    backward that keeps every state, bit for bit, whatever n (1, a divisor
    of L, a ragged last run, n > L)."""
    from oracle.backward import recurrent_bwd
    q, k, v, la, be, S0 = _rand(81, B=2, H=1, L=23, dk=4, dv=3, unit_keys=False)
    rng = np.random.default_rng(82)
    dO = rng.standard_normal((2, 1, 23, 3))
    dSf = rng.standard_normal((2, 1, 4, 3))
    ref = recurrent_bwd(q, k, v, la, be, S0, mode, dO, dSf)
    for n in (1, 5, 23, 64):
        got = recurrent_bwd(q, k, v, la, be, S0, mode, dO, dSf, checkpoint=n)
        for name, r in ref.items():
            if r is None:
                assert got[name] is None
            else:
                assert np.array_equal(got[name], r), (n, name)


@pytest.mark.parametrize("mode", oracle.MODES)
@pytest.mark.parametrize("d", [32, 128])
def test_chunkwise_backward_equals_token_backward_at_kernel_chunk(mode, d):
    """The chunkwise backward at the kernels' chunk size C = 64, with a
    state wider than a chunk (d = 128 > C) and narrower (d = 32 < C), over
    three full chunks and a ragged fourth (L = 200), keys not normalised
    (the erase terms then scale with |k|^2), against the token backward."""
    from oracle.backward import recurrent_bwd
    q, k, v, la, be, S0 = _rand(91 + d, B=1, H=1, L=200, dk=d, dv=d, unit_keys=False)
    k *= 1.0 / np.sqrt(d)                     # |k| around 1, not equal to 1
    q *= 1.0 / np.sqrt(d)
    rng = np.random.default_rng(92 + d)
    dO = rng.standard_normal((1, 1, 200, d))
    dSf = 0.1 * rng.standard_normal((1, 1, d, d))
    ref = recurrent_bwd(q, k, v, la, be, S0, mode, dO, dSf)
    got = oracle.chunkwise_bwd(q, k, v, la, be, S0, mode, 64, dO, dSf)
    for name in ("dq", "dk", "dv", "dS0", "dlog_alpha", "dbeta"):
        if ref[name] is None:
            assert got[name] is None
            continue
        assert _rel(got[name], ref[name]) < 1e-10, (name, _rel(got[name], ref[name]))
