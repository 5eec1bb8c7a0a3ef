"""Golden regression fixture for the oracle, and checks of the input recipe."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import recurrent_fwd
import workloads

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_matches_frozen_golden():
    """tests/golden/oracle_small.json was written by make_oracle_golden.py from
    the oracle alone; any change in the oracle's arithmetic must show here."""
    with open(os.path.join(HERE, "golden", "oracle_small.json")) as f:
        g = json.load(f)
    x = {n: np.array(a) for n, a in g["inputs"].items()}
    for mode, ref in g["modes"].items():
        o, S = recurrent_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"],
                             x["S0"], mode)
        assert np.max(np.abs(o - np.array(ref["o"]))) < 1e-14
        assert np.max(np.abs(S - np.array(ref["S_final"]))) < 1e-14


def test_oracle_extras_match_frozen_golden():
    """The same fixture's "extra" block: the backward, the fused prologue and
    epilogue, and the non-causal form on the frozen input."""
    import oracle
    with open(os.path.join(HERE, "golden", "oracle_small.json")) as f:
        g = json.load(f)
    x = {n: np.array(a) for n, a in g["inputs"].items()}
    e = {n: np.array(a) for n, a in g["extra"]["inputs"].items()}
    close = lambda a, b: np.max(np.abs(np.asarray(a) - np.asarray(b))) < 1e-12   # noqa: E731
    for mode, ref in g["extra"]["modes"].items():
        gr = oracle.recurrent_bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["S0"],
                                  mode, e["dO"], e["dS"])
        for n, a in ref["grads"].items():
            assert (a is None) == (gr[n] is None), (mode, n)
            assert a is None or close(gr[n], a), (mode, n)
        q, k, la, be = oracle.prepare(x["q"], x["k"], e["a"], e["b"], mode, 3, 1.0 / 16.0)
        o, _ = recurrent_fwd(q, k, x["v"], la, be, x["S0"], mode)
        o = oracle.out_norm(oracle.add_dskip(o, x["v"], e["D"]), e["w"], 1e-6)
        assert close(o, ref["fused_o"]), mode
    o, S = oracle.noncausal_fwd(x["q"], x["k"], x["v"], x["S0"])
    assert close(o, g["extra"]["noncausal"]["o"]) and close(S, g["extra"]["noncausal"]["S"])


@pytest.mark.parametrize("wid", [1, 2, 3])
def test_workload_recipe_small_sizes(wid):
    w = workloads.WORKLOADS[wid].scaled(B=1, H=2, L=64)
    x = workloads.make_inputs(w)
    y = workloads.make_inputs(w)
    for n in x:
        assert torch.equal(x[n], y[n]), n          # seeded and deterministic
    assert x["q"].dtype == w.torch_dtype and x["v"].dtype == w.torch_dtype
    assert x["q"].shape == (1, 2, 64, w.dk) and x["v"].shape == (1, 2, 64, w.dv)
    assert x["beta"].dtype == torch.float32 and x["S0"].dtype == torch.float32
    assert (x["beta"] > 0).all() and (x["beta"] < 1).all()
    assert (x["log_alpha"] < 0).all()
    if w.qk_norm:
        n_k = torch.linalg.vector_norm(x["k"].float(), dim=-1)
        assert torch.allclose(n_k, torch.ones_like(n_k), atol=2e-2 if w.dtype == "bf16" else 1e-6)
    else:
        assert abs(x["q"].float().std().item() - w.qkv_scale) < 0.2 * w.qkv_scale


def test_decode_workload_shapes():
    w = workloads.WORKLOADS[5].scaled(B=2, H=3, steps=4)
    x = workloads.make_inputs(w)
    assert x["q"].shape == (4, 2, 3, 128) and x["beta"].shape == (4, 2, 3)
    assert x["S0"].shape == (2, 3, 128, 128)
    assert abs(x["S0"].std().item() - 0.02) < 2e-3
