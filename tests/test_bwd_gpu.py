"""GPU parity of the backward (la_chunk_bwd) against the float64 oracle.

The reference is ``oracle.recurrent_bwd`` -- the reverse of the token
recurrence, the plain derivative of the definition, pinned on the CPU by
finite differences -- in every test.  Long sequences run it with
checkpointed states (every 64th state kept, each run of 64 tokens recomputed
before the reverse walk crosses it; bit-identical to keeping every state),
so no reference shares the chunk algebra the kernels use.  It consumes
float64 copies of exactly the tensors handed to the GPU.  Tolerances per gradient as for the forward: float32 inputs
max|err| <= 1e-4 max|ref|; bf16 inputs max|err| <= 2e-2 RMS(ref) (the
gradients are float32, so no output rounding is added).
"""
import numpy as np
import pytest
import torch

import chunkwise_gated_delta_la_amd as la
import oracle
import workloads
from _parity import assert_close, f64, log, to_cuda
from test_parity_gpu import recipe

pytestmark = pytest.mark.gpu

MODES = ("linear", "delta", "gated_delta", "gated_linear")
GATED = ("gated_delta", "gated_linear")
ERASE = ("delta", "gated_delta")


def run_bwd(w, x, gr, mode, with_s0=True, with_dsf=True):
    d = to_cuda(x)
    g = to_cuda(gr)
    res = la.chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                       d["S0"] if with_s0 else None, g["dout"],
                       g["dS_final"] if with_dsf else None, mode=mode)
    torch.cuda.synchronize()
    return res


def reference(x, gr, mode, with_s0=True, with_dsf=True, checkpoint=None):
    y = workloads.to_f64(x)
    gy = workloads.to_f64(gr)
    args = (y["q"], y["k"], y["v"], y["log_alpha"], y["beta"],
            y["S0"] if with_s0 else None, mode)
    dsf = gy["dS_final"] if with_dsf else None
    return oracle.recurrent_bwd(*args, gy["dout"], dsf, checkpoint=checkpoint)


def compare(res, ref, mode, dtype):
    for name in ("dq", "dk", "dv", "dS0"):
        assert_close(name, f64(res[name]), ref[name], dtype)
    if mode in GATED:
        assert_close("dlog_alpha", f64(res["dlog_alpha"]), ref["dlog_alpha"], dtype)
    else:
        assert res["dlog_alpha"] is None
    if mode in ERASE:
        assert_close("dbeta", f64(res["dbeta"]), ref["dbeta"], dtype)
    else:
        assert res["dbeta"] is None


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype", ("f32", "bf16"))
@pytest.mark.parametrize("d,L", [(64, 64), (64, 200), (128, 131), (128, 1)])
def test_chunk_bwd_small(mode, dtype, d, L):
    """Every gradient, every element, against the token backward: one
    chunk, several chunks with a ragged tail, a single token; nonzero S0
    and dS_final."""
    w = recipe(mode, dtype, B=2, H=1, L=L, d=d, s0_std=0.05, seed=31 + L + d)
    log(f"case chunk_bwd {w.name} mode={mode} seed={w.seed}")
    x = workloads.make_inputs(w)
    gr = workloads.make_upstream_grads(w, ds_std=0.1)
    res = run_bwd(w, x, gr, mode)
    ref = reference(x, gr, mode)
    compare(res, ref, mode, dtype)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
@pytest.mark.parametrize("mode", ERASE)
def test_chunk_bwd_nonunit_keys(mode, dtype, d):
    """The delta modes with keys rescaled per token by a factor in
    [0.5, 1.5] (the erase terms scale with |k|^2): every gradient against
    the token backward."""
    from test_parity_gpu import _nonunit_keys
    w = recipe(mode, dtype, B=2, H=1, L=131, d=d, s0_std=0.05, seed=119)
    log(f"case chunk_bwd_nonunit {w.name} seed={w.seed}")
    x = _nonunit_keys(w, workloads.make_inputs(w), 120)
    gr = workloads.make_upstream_grads(w, ds_std=0.1)
    res = run_bwd(w, x, gr, mode)
    ref = reference(x, gr, mode)
    compare(res, ref, mode, dtype)


@pytest.mark.parametrize("mode", MODES)
def test_chunk_bwd_zero_state_and_no_state_gradient(mode):
    """S0 = NULL and dS_final = NULL read as zeros."""
    w = recipe(mode, "bf16", B=1, H=2, L=130, d=64, seed=5)
    log(f"case chunk_bwd_nulls {w.name} seed={w.seed}")
    x = workloads.make_inputs(w)
    gr = workloads.make_upstream_grads(w)
    res = run_bwd(w, x, gr, mode, with_s0=False, with_dsf=False)
    ref = reference(x, gr, mode, with_s0=False, with_dsf=False)
    compare(res, ref, mode, "bf16")


@pytest.mark.parametrize("mode", MODES)
def test_chunk_bwd_long(mode):
    """A long bf16 sequence at d = 128 (64 chunks, a ragged last one)
    against the token backward; the walks carry the state gradient over
    every chunk."""
    w = recipe(mode, "bf16", B=1, H=2, L=4096 - 17, d=128, s0_std=0.02, seed=77)
    log(f"case chunk_bwd_long {w.name} seed={w.seed}")
    x = workloads.make_inputs(w)
    gr = workloads.make_upstream_grads(w, ds_std=0.05)
    res = run_bwd(w, x, gr, mode)
    ref = reference(x, gr, mode, checkpoint=64)
    compare(res, ref, mode, "bf16")


def test_chunk_bwd_state_gradient_chains_over_a_split():
    """The state gradient chains: the backward of two halves, the second
    half's dS0 fed to the first as dS_final, equals the backward of the
    whole (the chunk boundary at 128 lies on a chunk boundary)."""
    mode = "gated_delta"
    w = recipe(mode, "f32", B=1, H=2, L=256, d=64, s0_std=0.05, seed=91)
    log(f"case chunk_bwd_split {w.name} seed={w.seed}")
    x = workloads.make_inputs(w)
    gr = workloads.make_upstream_grads(w, ds_std=0.1)
    whole = run_bwd(w, x, gr, mode)
    d = to_cuda(x)
    g = to_cuda(gr)
    # forward of the first half gives the second half's S0
    _, S_mid = la.chunk_fwd(d["q"][:, :, :128].contiguous(), d["k"][:, :, :128].contiguous(),
                            d["v"][:, :, :128].contiguous(),
                            d["log_alpha"][:, :, :128].contiguous(),
                            d["beta"][:, :, :128].contiguous(), d["S0"], mode=mode)
    half = lambda t, s: t[:, :, s].contiguous()     # noqa: E731
    second = la.chunk_bwd(*(half(d[n], slice(128, 256)) for n in ("q", "k", "v", "log_alpha",
                                                                   "beta")),
                          S_mid, half(g["dout"], slice(128, 256)), g["dS_final"], mode=mode)
    first = la.chunk_bwd(*(half(d[n], slice(0, 128)) for n in ("q", "k", "v", "log_alpha",
                                                                "beta")),
                         d["S0"], half(g["dout"], slice(0, 128)), second["dS0"], mode=mode)
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv", "dlog_alpha", "dbeta"):
        got = torch.cat([first[name], second[name]], dim=2)
        ref = f64(whole[name])
        err = float(np.max(np.abs(f64(got) - ref)))
        log(f"  {name}: split vs whole max|err| {err:.3e}")
        assert err <= 1e-4 * float(np.max(np.abs(ref)))
    assert_close("dS0", f64(first["dS0"]), f64(whole["dS0"]), "f32")


def test_chunk_bwd_full_size_sampled():
    """The long-context workload at full size (B=1, H=32, L=65536, d=128,
    bf16), launched as the bench launches it; the float64 token backward
    (checkpointed) recomputes two sampled heads over the whole sequence
    (heads do not interact)."""
    w = workloads.WORKLOADS[4]
    log(f"case chunk_bwd_full {w.name} seed={w.seed}")
    x = workloads.make_inputs(w)
    gr = workloads.make_upstream_grads(w, ds_std=0.02)
    res = run_bwd(w, x, gr, w.mode)
    hs = [0, w.H - 1]
    sub = lambda d: {k: t[:, hs].contiguous() for k, t in d.items()}   # noqa: E731
    ref = reference(sub(x), sub(gr), w.mode, checkpoint=64)
    got = {k: (t[:, hs] if t is not None else None) for k, t in res.items()}
    compare(got, ref, w.mode, "bf16")


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("bf16", 128)])
@pytest.mark.parametrize("mode", MODES)
def test_chunk_bwd_varlen_packed(mode, dtype, d):
    """A packed batch of 9 sequences (empty first, middle and last; a single
    token; partial, exact and several chunks): every gradient against the
    token backward run per sequence; each sequence's packed gradients are
    bit-equal to the fixed-length backward on it; empty sequences pass
    dS_final to dS0.  Outputs start as NaN: every element must be written."""
    from test_parity_gpu import _packed
    lens = [0, 1, 63, 64, 0, 65, 200, 130, 0]
    H = 3
    w, x, S0, cu = _packed(lens, H, d, dtype, mode, seed=83)
    log(f"case chunk_bwd_varlen {mode} {dtype} d{d} H{H} lens {lens}")
    T = int(cu[-1])
    N = len(lens)
    gen = torch.Generator("cpu").manual_seed(84)
    dout = torch.randn((H, T, d), generator=gen).to(w.torch_dtype)
    dSf = torch.randn((N, H, d, d), generator=gen) * 0.1
    dev = {n: t.cuda() for n, t in x.items()}
    res = la.chunk_bwd_varlen(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"],
                              S0.cuda(), dout.cuda(), cu.cuda(), dSf.cuda(), mode=mode)
    torch.cuda.synchronize()
    y = {n: t.to(torch.float64).numpy() for n, t in x.items()}
    s0, go, gsf = (t.to(torch.float64).numpy() for t in (S0, dout, dSf))
    for s in range(N):
        a, b = int(cu[s]), int(cu[s + 1])
        if a == b:
            assert torch.equal(res["dS0"][s].cpu(), dSf[s]), f"sequence {s} (empty)"
            continue
        sl = lambda t: t[None, :, a:b]   # noqa: E731  -> [1, H, len, ...]
        ref = oracle.recurrent_bwd(sl(y["q"]), sl(y["k"]), sl(y["v"]), sl(y["log_alpha"]),
                                   sl(y["beta"]), s0[s][None], mode, sl(go), gsf[s][None])
        got = {n: (None if t is None else (t[s][None] if n == "dS0" else t[None, :, a:b]))
               for n, t in res.items()}
        log(f"  sequence {s} ({b - a} tokens)")
        compare(got, ref, mode, dtype)
    # packed == fixed length, bit for bit
    for s in (3, 6):
        a, b = int(cu[s]), int(cu[s + 1])
        one = la.chunk_bwd(*(dev[n][None, :, a:b].contiguous() for n in ("q", "k", "v")),
                           dev["log_alpha"][None, :, a:b].contiguous(),
                           dev["beta"][None, :, a:b].contiguous(), S0[s][None].cuda(),
                           dout[None, :, a:b].contiguous().cuda(), dSf[s][None].cuda(),
                           mode=mode)
        torch.cuda.synchronize()
        for n in ("dq", "dk", "dv", "dlog_alpha", "dbeta"):
            if one[n] is not None:
                assert torch.equal(one[n][0], res[n][:, a:b]), f"sequence {s}: {n} differs"
        assert torch.equal(one["dS0"][0], res["dS0"][s]), f"sequence {s}: dS0 differs"


@pytest.mark.parametrize("mode", MODES)
def test_chunk_bwd_deterministic(mode):
    """Two calls on the same inputs give bit-identical gradients (every sum
    in the kernels has a fixed order: no atomics)."""
    w = recipe(mode, "bf16", B=1, H=4, L=2048 + 37, d=128, s0_std=0.02, seed=101)
    log(f"case chunk_bwd_deterministic {w.name} seed={w.seed}")
    x = workloads.make_inputs(w)
    gr = workloads.make_upstream_grads(w, ds_std=0.05)
    a = run_bwd(w, x, gr, mode)
    b = run_bwd(w, x, gr, mode)
    for n in a:
        if a[n] is not None:
            assert torch.equal(a[n], b[n]), f"{n} differs between two calls"


def _fused_bwd_case(w, mode, flags, scale, checkpoint=None, heads=None):
    """la_chunk_bwd_fused on the raw inputs of `w` against the oracle's
    backward through prepare and the recurrence: (result, reference); with
    `heads`, the oracle recomputes those heads only and the result is cut
    to them (heads do not interact)."""
    r = workloads.make_raw_inputs(w)
    q, k, a, b = r["q"], r["k"], r["a_raw"], r["b_raw"]
    if not flags & 2:      # the op takes q, k as given: hand it normalised ones
        q = (q.float() / torch.linalg.vector_norm(q.float(), dim=-1, keepdim=True)).to(q.dtype)
        k = (k.float() / torch.linalg.vector_norm(k.float(), dim=-1, keepdim=True)).to(k.dtype)
    if not flags & 1:      # the op takes the gates as given
        a = -scale * torch.nn.functional.softplus(a)
        b = torch.sigmoid(b)
    gr = workloads.make_upstream_grads(w, ds_std=0.1)
    x = dict(q=q, k=k, v=r["v"], log_alpha=a, beta=b, S0=r["S0"])
    dev = to_cuda(x)
    g = to_cuda(gr)
    res = la.chunk_bwd(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], dev["S0"],
                       g["dout"], g["dS_final"], mode=mode, qk_l2norm=bool(flags & 2),
                       gate_act=bool(flags & 1), gate_scale=scale)
    torch.cuda.synchronize()
    if heads is not None:
        x = {n: t[:, heads].contiguous() for n, t in x.items()}
        gr = {n: t[:, heads].contiguous() for n, t in gr.items()}
        res = {n: (t[:, heads] if t is not None else None) for n, t in res.items()}
    y = workloads.to_f64(x)
    gy = workloads.to_f64(gr)
    qp, kp, lp, bp = oracle.prepare(y["q"], y["k"], y["log_alpha"], y["beta"], mode, flags,
                                    scale)
    ref = oracle.recurrent_bwd(qp, kp, y["v"], lp, bp, y["S0"], mode, gy["dout"],
                               gy["dS_final"], checkpoint=checkpoint)
    dq, dk_, da, db = oracle.prologue_bwd(y["q"], y["k"], y["log_alpha"], y["beta"], mode, flags,
                                          scale, ref["dq"], ref["dk"], ref["dlog_alpha"],
                                          ref["dbeta"])
    return res, dict(ref, dq=dq, dk=dk_, dlog_alpha=da, dbeta=db)


@pytest.mark.parametrize("mode", MODES)
def test_chunk_bwd_fused_prologue_long(mode):
    """The fused backward over a long bf16 sequence at d = 128 (64 chunks, a
    ragged last one), both prologue steps on: the walks take the k norms
    inside their decay tables and the chunk's total decay from a slot of
    its own at every step, the other kernels the q and k norms as row
    factors; every gradient against the oracle's token backward through
    prepare."""
    w = recipe(mode, "bf16", B=1, H=2, L=4096 - 17, d=128, s0_std=0.05, seed=131)
    log(f"case chunk_bwd_fused_long {mode} seed={w.seed}")
    res, ref = _fused_bwd_case(w, mode, 3, 1.0 / 16.0, checkpoint=64)
    compare(res, ref, mode, "bf16")


def test_chunk_bwd_fused_full_size_sampled():
    """The fused backward on the long-context workload at full size (B=1,
    H=32, L=65536, d=128, bf16; raw q, k and gate scores, both prologue
    steps), launched as the bench launches it; the float64 token backward
    (checkpointed) through prepare recomputes two sampled heads."""
    w = workloads.WORKLOADS[4]
    log(f"case chunk_bwd_fused_full {w.name} seed={w.seed}")
    res, ref = _fused_bwd_case(w, w.mode, 3, 1.0 / 16.0, checkpoint=64, heads=[0, w.H - 1])
    compare(res, ref, w.mode, "bf16")


@pytest.mark.parametrize("flags", [1, 2, 3])
@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
@pytest.mark.parametrize("mode", MODES)
def test_chunk_bwd_fused_prologue(mode, dtype, d, flags):
    """The gradients of the fused forward's raw inputs (unnormalised q, k
    with flag 2; raw gate scores with flag 1) against the oracle's backward
    through prepare and the recurrence, every element."""
    w = recipe(mode, dtype, B=2, H=1, L=131, d=d, s0_std=0.05, seed=111 + flags)
    log(f"case chunk_bwd_fused {mode} {dtype} d{d} flags={flags} seed={w.seed}")
    res, ref = _fused_bwd_case(w, mode, flags, 1.0 / 16.0)
    compare(res, ref, mode, dtype)
