"""la_chunk_fwd_noalloc: the forward with the library's static scratch in
place of a workspace, against la_chunk_fwd (the same kernels) and the
float64 oracle.

Two calls in a row, the second smaller than the first (the scratch keeps
the first call's contents, which the second must not read), in the cases
that use the scratch: the bf16 delta modes (per-chunk T factors) and a
sequence-parallel call (segment states), plus a float call that needs none.
Outputs must equal la_chunk_fwd's bit for bit and meet the oracle's bound.
"""
import pytest
import torch

import chunkwise_gated_delta_la_amd as la
import workloads
from _parity import assert_close, f64, log, oracle_fwd, to_cuda
from test_parity_gpu import recipe

pytestmark = pytest.mark.gpu


def _both(w, x, mode):
    d = to_cuda(x)
    ref_o, ref_S = la.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"],
                                mode=mode)
    out = torch.full_like(ref_o, float("nan"))
    S = torch.full_like(ref_S, float("nan"))
    la.chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"], out, S,
                         mode=mode)
    torch.cuda.synchronize()
    return out, S, ref_o, ref_S


@pytest.mark.parametrize("mode,dtype,big,small", [
    ("gated_delta", "bf16", (2, 4, 64 * 9 + 5, 128), (1, 2, 200, 64)),
    ("delta", "bf16", (1, 3, 1000, 128), (2, 1, 64, 128)),
    ("linear", "bf16", (1, 1, 4096 + 40, 128), (1, 2, 130, 128)),    # segments in the scratch
    ("gated_delta", "f32", (1, 2, 300, 64), (1, 1, 70, 64)),          # no scratch
])
def test_noalloc_matches_workspace_call(mode, dtype, big, small):
    for (B, H, L, d), seed in ((big, 201), (small, 202)):
        w = recipe(mode, dtype, B=B, H=H, L=L, d=d, s0_std=0.2, seed=seed)
        log(f"noalloc {w} P={la.chunk_segments(B, H, L, d, d, mode=mode, dtype=w.torch_dtype)}")
        x = workloads.make_inputs(w)
        out, S, ref_o, ref_S = _both(w, x, mode)
        assert torch.equal(out, ref_o), "output differs from la_chunk_fwd"
        assert torch.equal(S, ref_S), "final state differs from la_chunk_fwd"
        o_ref, S_ref = oracle_fwd(x, mode)
        assert_close("o", f64(out), o_ref, dtype, bf16_out=dtype == "bf16")
        assert_close("S_final", f64(S), S_ref, dtype)


def test_noalloc_rejects_oversize():
    """More scratch than the static array holds: an error, nothing launched."""
    w = recipe("gated_delta", "bf16", B=1, H=1, L=64, d=128)
    d = to_cuda(workloads.make_inputs(w))
    q = d["q"].expand(1, 1, 64, 128)
    big = torch.empty((1, 1, 64 * 21846, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((1, 1, 64 * 21846), dtype=torch.float32, device="cuda")
    out = torch.empty_like(big)
    with pytest.raises(la.LAError, match="LA_ERR_WORKSPACE"):
        la.chunk_fwd_noalloc(big, big, big, g, g, None, out, None, mode="gated_delta")
    del q
