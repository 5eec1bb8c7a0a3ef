"""GPU parity of the wide kernel: the modes without erase (linear and gated
linear attention, bf16) over enough (batch, head) streams that the library
runs one workgroup per stream and 64 state columns, four waves sharing the
chunk's Q, K and masked scores ("LinearAttention 概述", section FLASH: the
chunk's intra part (Q K^T * M) V and inter part Q S; "混合注意力学习(1):
线性注意力", FWP分块并行机制: the state carried chunk to chunk).  Smaller
batches take the chain kernel, which tests/test_parity_gpu.py covers.

Every output element and final state against the oracle, the bf16 output
against the float one (rounded to nearest even), ragged and packed inputs,
and repeated calls bit for bit (a read of a tile still in flight would not
repeat).
"""
import numpy as np
import pytest
import torch

import chunkwise_gated_delta_la_amd as la
import workloads
from _parity import assert_close, assert_out_pair, f64, log, oracle_fwd, to_cuda
from test_parity_gpu import GATE_SCALE, _fused_call, _fused_oracle, _packed, _packed_oracle, \
    _raw, recipe

pytestmark = pytest.mark.gpu

WIDE_MODES = ["linear", "gated_linear"]


def _streams(d):
    """(B, H) with B * H * d / 64 = 256 workgroups: the smallest grid the
    library gives the wide kernel."""
    return (4, 64) if d == 64 else (2, 64)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode", WIDE_MODES)
def test_wide_forward(mode, d):
    """1 partial chunk, 2 exact chunks, 3 with a ragged tail, 5 chunks; with
    and without S0."""
    B, H = _streams(d)
    for L, s0 in ((40, 0.3), (128, 0.0), (170, 0.3), (320, 0.3)):
        w = recipe(mode, "bf16", B=B, H=H, L=L, d=d, s0_std=s0, seed=L + d)
        log(f"wide {w}")
        x = workloads.make_inputs(w)
        o_ref, S_ref = oracle_fwd(x, mode)
        dev = to_cuda(x)
        S0 = dev["S0"] if s0 > 0 else None
        outs = []
        for dt in (None, torch.float32, torch.float32):
            outs.append(la.chunk_fwd(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"],
                                     S0, mode=mode, out_dtype=dt))
        torch.cuda.synchronize()
        (o16, S16), (o32, S32), (o32b, S32b) = outs
        assert_out_pair("o", o16, o32, o_ref)
        assert_close("S_final", f64(S32), S_ref, "bf16")
        assert torch.equal(S16, S32), "the output dtype must not change the state"
        assert torch.equal(o32, o32b) and torch.equal(S32, S32b), "repeated calls differ"


@pytest.mark.parametrize("mode", WIDE_MODES)
def test_wide_state_in_place(mode):
    """S_final may be S0 itself: each workgroup reads its columns of S0
    before it writes them."""
    B, H = _streams(128)
    w = recipe(mode, "bf16", B=B, H=H, L=200, d=128, s0_std=0.3, seed=91)
    log(f"wide in place {w}")
    x = workloads.make_inputs(w)
    o_ref, S_ref = oracle_fwd(x, mode)
    dev = to_cuda(x)
    S = dev["S0"].clone()
    out, _ = la.chunk_fwd(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], S,
                          mode=mode, S_final=S, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close("o (f32 out)", f64(out), o_ref, "bf16")
    assert_close("S_final (in place)", f64(S), S_ref, "bf16")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode", WIDE_MODES)
def test_wide_varlen_packed(mode, d):
    """A packed batch of 9 sequences (empty ones first, middle and last; one
    token; partial, exact and several chunks) over enough heads for the wide
    kernel; out and S_final start as NaN."""
    lens = [0, 1, 63, 64, 0, 65, 200, 130, 0]
    H = 32
    w, x, S0, cu = _packed(lens, H, d, "bf16", mode, seed=97)
    log(f"wide varlen {mode} d{d} H{H} lens {lens}")
    o_ref, S_ref = _packed_oracle(x, S0, cu, mode)
    dev = {n: t.cuda() for n, t in x.items()}
    T = int(cu[-1])
    out = torch.full((H, T, d), float("nan"), dtype=torch.float32, device="cuda")
    S = torch.full((len(lens), H, d, d), float("nan"), dtype=torch.float32, device="cuda")
    la.chunk_fwd_varlen(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"],
                        S0.cuda(), cu.cuda(), mode=mode, out=out, S_final=S)
    torch.cuda.synchronize()
    assert_close("o (f32 out)", f64(out), o_ref, "bf16")
    assert_close("S_final", f64(S), S_ref, "bf16")
    for s, n in enumerate(lens):
        if n == 0:
            assert torch.equal(S[s].cpu(), S0[s]), f"sequence {s} (empty) changed its state"


def test_wide_gate_activation():
    """Gated linear attention from raw gate scores (the fused prologue's gate
    activation only): the wide kernel reads the activated gates the T-solve
    kernel's prologue writes."""
    B, H = _streams(128)
    w = recipe("gated_linear", "bf16", B=B, H=H, L=64 * 3 + 11, d=128, s0_std=0.3, seed=101)
    log(f"wide gate activation {w}")
    r = _raw(w, 1)
    o_ref, S_ref = _fused_oracle(r, "gated_linear", 1)
    dev = to_cuda(r)
    out, S = _fused_call(dev, "gated_linear", 1)
    out32, S32 = _fused_call(dev, "gated_linear", 1, out_dtype=torch.float32)
    assert_out_pair("o", out, out32, o_ref)
    assert_close("S_final", f64(S), S_ref, "bf16")
    assert torch.equal(S32, S)
