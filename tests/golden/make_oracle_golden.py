"""Writes tests/golden/oracle_small.json from the float64 oracle only.

The fixture freezes the oracle's outputs on a tiny fixed input for every
mode, so that a later change to the oracle's arithmetic shows up as a failed
comparison and has to be justified.  The values come from the token
recurrence (o_t = S_t^T q_t after the gated-delta update of the
hybrid-attention notes, section "Gated DeltaNet", its special cases, and
the gated linear update of the same section), and -- under "extra" -- from
the oracle's other functions on the same input: the backward (reverse of the
recurrence), the fused prologue and epilogue, and the non-causal form.

Run from the repository root:  python tests/golden/make_oracle_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402
from oracle import recurrent_fwd  # noqa: E402


def tiny_inputs():
    # Values on a coarse dyadic grid so the JSON text round-trips exactly.
    rng = np.random.default_rng(2024)
    B, H, L, dk, dv = 1, 2, 6, 3, 2
    q = rng.integers(-8, 9, size=(B, H, L, dk)) / 8.0
    k = rng.integers(-8, 9, size=(B, H, L, dk)) / 8.0
    v = rng.integers(-8, 9, size=(B, H, L, dv)) / 8.0
    beta = rng.integers(1, 16, size=(B, H, L)) / 16.0
    log_alpha = -rng.integers(0, 8, size=(B, H, L)) / 32.0
    S0 = rng.integers(-4, 5, size=(B, H, dk, dv)) / 4.0
    return dict(q=q, k=k, v=v, beta=beta, log_alpha=log_alpha, S0=S0)


def extra_inputs(x):
    """Upstream gradients, raw gate scores and epilogue parameters on the
    same dyadic grid."""
    rng = np.random.default_rng(2025)
    B, H, L, dk = x["k"].shape
    dv = x["v"].shape[-1]
    return dict(dO=rng.integers(-8, 9, size=(B, H, L, dv)) / 8.0,
                dS=rng.integers(-8, 9, size=(B, H, dk, dv)) / 8.0,
                a=rng.integers(-16, 17, size=(B, H, L)) / 8.0,
                b=rng.integers(-16, 17, size=(B, H, L)) / 8.0,
                D=rng.integers(-8, 9, size=(H, dv)) / 8.0,
                w=rng.integers(4, 12, size=(H, dv)) / 8.0)


def extra_outputs(x):
    e = extra_inputs(x)
    res = {"inputs": {n: a.tolist() for n, a in e.items()}, "modes": {}}
    for mode in ("linear", "delta", "gated_delta", "gated_linear"):
        g = oracle.recurrent_bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["S0"],
                                 mode, e["dO"], e["dS"])
        q, k, la, be = oracle.prepare(x["q"], x["k"], e["a"], e["b"], mode, 3, 1.0 / 16.0)
        o, _ = recurrent_fwd(q, k, x["v"], la, be, x["S0"], mode)
        o = oracle.out_norm(oracle.add_dskip(o, x["v"], e["D"]), e["w"], 1e-6)
        res["modes"][mode] = {"grads": {n: (None if a is None else a.tolist())
                                        for n, a in g.items()},
                              "fused_o": o.tolist()}
    o, S = oracle.noncausal_fwd(x["q"], x["k"], x["v"], x["S0"])
    res["noncausal"] = {"o": o.tolist(), "S": S.tolist()}
    return res


def main():
    x = tiny_inputs()
    out = {"source": "oracle.recurrent_fwd on tiny_inputs() of this script",
           "inputs": {n: a.tolist() for n, a in x.items()}, "modes": {}}
    for mode in ("linear", "delta", "gated_delta", "gated_linear"):
        o, S = recurrent_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"],
                             x["S0"], mode)
        out["modes"][mode] = {"o": o.tolist(), "S_final": S.tolist()}
    out["extra"] = extra_outputs(x)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
