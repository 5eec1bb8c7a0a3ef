"""A CPU model of the bf16 chunk kernels' operand roundings.

Not the oracle and not the GPU path: the chunkwise algebra evaluated with
torch float32 matrix products (the MFMA's float accumulation of exact bf16
products), where each float operand that the kernels feed to a bf16 matrix
product is either split into bf16 hi + lo parts or rounded to a single
bf16, as chosen per operand.  With every operand exact (float64) it is the
chunkwise form of the recurrence.  Used to size the kernels' precision
budget against the bf16 tolerance max|err| <= 2e-2 RMS(ref).

The kernels' choice: T = (I + A)^-1 as a single bf16 in the T R product
(R split), the state S as a single bf16 in the chain's K S product and split
everywhere else (Q S), U_new split in the state update and in
(Q K^T * Gamma) U_new, the scores split.
"""
import torch

BF = torch.bfloat16

KERNEL = dict(T="hi", S_chain="hi", S_out="split", U_upd="split", scores="split",
              U_out="split")


def _r16(x):
    return x.to(BF).to(x.dtype)


def _split(x):
    hi = _r16(x)
    return hi, _r16(x - hi)


def _opnd(x, how):
    """An operand as the kernel feeds it: 'split' (hi + lo, summed after the
    products), 'hi' (one bf16) or 'exact'."""
    if how == "exact":
        return [x]
    if how == "hi":
        return [_r16(x)]
    return list(_split(x))


def _mm(a_parts, b_parts):
    """Sum of the part products except lo * lo (below float rounding)."""
    out = None
    for i, a in enumerate(a_parts):
        for j, b in enumerate(b_parts):
            if i and j:
                continue
            p = a @ b
            out = p if out is None else out + p
    return out


def chunk_forward(x, mode, C=64, scheme=None):
    """Forward of one workload's inputs (torch tensors as the workloads
    module makes them).  scheme=None: float64, every operand exact."""
    exact = scheme is None
    dt = torch.float64 if exact else torch.float32
    sch = {k: "exact" for k in KERNEL} if exact else scheme
    q, k, v = (x[n].to(dt) for n in ("q", "k", "v"))
    B, H, L, d = q.shape
    q, k, v = (t.reshape(B * H, L, d) for t in (q, k, v))
    gated = mode in ("gated_delta", "gated_linear")
    erase = mode in ("delta", "gated_delta")
    la = x["log_alpha"].to(dt).reshape(B * H, L) if gated else torch.zeros(B * H, L, dtype=dt)
    be = x["beta"].to(dt).reshape(B * H, L) if erase else torch.ones(B * H, L, dtype=dt)
    S0 = x.get("S0")
    S = S0.to(dt).reshape(B * H, d, d).clone() if S0 is not None else torch.zeros(B * H, d, d, dtype=dt)
    o = torch.empty(B * H, L, d, dtype=dt)
    for c0 in range(0, L, C):
        Q, K, V = q[:, c0:c0 + C], k[:, c0:c0 + C], v[:, c0:c0 + C]
        n = Q.shape[1]
        M = torch.tril(torch.ones(n, n, dtype=dt))
        g = torch.cumsum(la[:, c0:c0 + C], -1)
        b = be[:, c0:c0 + C]
        gam = torch.exp(g)
        Gam = torch.exp((g[:, :, None] - g[:, None, :]).clamp(max=0)) * M
        f = torch.exp(g[:, -1:] - g)
        Aqk = (Q @ K.transpose(1, 2)) * Gam
        if erase:
            I = torch.eye(n, dtype=dt).expand(B * H, n, n)
            A = (b[:, :, None] * (K @ K.transpose(1, 2)) * Gam) * torch.tril(torch.ones(n, n, dtype=dt), -1)
            T = torch.linalg.solve_triangular(I + A, I, upper=False)
            KS = _mm([K], _opnd(S, sch["S_chain"]))
            R = b[:, :, None] * (V - gam[:, :, None] * KS)
            Un = _mm(_opnd(T, sch["T"]), _opnd(R, "split" if not exact else "exact"))
        else:
            Un = V
        QS = _mm([Q], _opnd(S, sch["S_out"]))
        o[:, c0:c0 + n] = gam[:, :, None] * QS + _mm(_opnd(Aqk, sch["scores"]),
                                                      _opnd(Un, sch["U_out"]))
        upd = f[:, :, None] * Un
        S = gam[:, -1:, None] * S + _mm([K.transpose(1, 2)], _opnd(upd, sch["U_upd"]))
    return o.reshape(B, H, L, d), S.reshape(B, H, d, d)


def error_ratio(x, mode, scheme):
    """max|err| / (2e-2 RMS(ref)) of the output and of the final state."""
    o_ref, S_ref = chunk_forward(x, mode)
    o, S = chunk_forward(x, mode, scheme=scheme)
    bo = 2e-2 * float(o_ref.pow(2).mean().sqrt())
    bs = 2e-2 * float(S_ref.pow(2).mean().sqrt())
    return (float((o.double() - o_ref).abs().max()) / bo,
            float((S.double() - S_ref).abs().max()) / bs)
