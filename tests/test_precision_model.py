"""The bf16 kernels' precision budget, on the CPU (no GPU).

tests/_precision_model.py evaluates the chunkwise forward with the kernels'
operand roundings (float32 products of bf16 parts).  Its exact (float64)
evaluation is first tied to the oracle's recurrence; then the kernels'
choice of split and single bf16 operands must keep max|err| within half of
the bf16 tolerance (2e-2 RMS) on long DeltaNet (alpha = 1: nothing decays,
rounding accumulates over the whole sequence) and gated-delta sequences.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from _precision_model import KERNEL, chunk_forward, error_ratio


def _inputs(wid, H=None, L=None, seed=None):
    w0 = workloads.WORKLOADS[wid]
    w = w0.scaled(H=H or w0.H, L=L or w0.L, seed=seed or w0.seed)
    x = workloads.make_inputs(w)
    if w.s0_std == 0:
        x["S0"] = None
    return w, x


def test_exact_model_is_the_recurrence():
    w, x = _inputs(4, H=2, L=200, seed=5)
    x = dict(x)
    o, S = chunk_forward(x, w.mode)
    y = workloads.to_f64(x)
    o_ref, S_ref = oracle.recurrent_fwd(y["q"], y["k"], y["v"], y["log_alpha"], y["beta"],
                                        y["S0"], w.mode)
    assert np.max(np.abs(o.numpy() - o_ref)) < 1e-10 * np.max(np.abs(o_ref))
    assert np.max(np.abs(S.numpy() - S_ref)) < 1e-10 * np.max(np.abs(S_ref))


@pytest.mark.parametrize("wid,H", [(3, None), (4, 8)])
def test_kernel_roundings_within_half_the_bound(wid, H):
    """The DeltaNet workload at full size and a quarter of the long-context
    gated workload's heads at full length: the largest errors sit in the
    tails, so the sample must be large."""
    w, x = _inputs(wid, H=H)
    eo, es = error_ratio(x, w.mode, KERNEL)
    print(f"{w.name}: output {eo:.3f}, final state {es:.3f} of the bound")
    assert eo <= 0.5 and es <= 0.5, (eo, es)
