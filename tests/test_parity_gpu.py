"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Every case prints its name, shapes and seed before touching the GPU.  Small
cases compare every element; the full-size workloads run exactly as the
bench launches them and compare sampled (batch, head) slices, which the
oracle computes independently (heads do not interact).
"""
import math

import numpy as np
import pytest
import torch

import chunkwise_gated_delta_la_amd as la
import oracle
import workloads
from _parity import (assert_close, assert_out_pair, f64, log, oracle_decode, oracle_fwd,
                     to_cuda)
from workloads import WORKLOADS, Workload

pytestmark = pytest.mark.gpu

MODES = ("linear", "delta", "gated_delta", "gated_linear")


def recipe(mode, dtype, B, H, L, d, s0_std=0.0, seed=7):
    """The workloads' recipe for `mode` at reduced sizes (the modes without
    erase take the linear-attention recipe: raw scaled q, k)."""
    lin = mode in ("linear", "gated_linear")
    return Workload(f"{mode}_{dtype}_b{B}h{H}l{L}d{d}", mode, dtype, B=B, H=H, L=L, dk=d,
                    dv=d, C=64, qk_norm=not lin,
                    qkv_scale=1.0 / math.sqrt(d) if lin else 1.0, s0_std=s0_std, seed=seed)


def run_chunk(w, x, mode=None, S_final=True, out_dtype=None):
    mode = mode or w.mode
    d = to_cuda(x)
    s0 = d["S0"] if w.s0_std > 0 else None
    out, S = la.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], s0, mode=mode,
                          C=w.C, return_state=S_final, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, S


def check_fwd(w, x, o_ref, S_ref, mode=None, sel=None):
    """Run the forward with the workload's output dtype and, for bf16
    inputs, also with a float32 output; compare both with the oracle."""
    sel = sel or (lambda t: t)
    bf16 = w.dtype == "bf16"
    out, S = run_chunk(w, x, mode)
    assert_close("o", f64(sel(out)), o_ref, w.dtype, bf16_out=bf16)
    assert_close("S_final", f64(sel(S)), S_ref, w.dtype)
    if bf16:
        out32, S32 = run_chunk(w, x, mode, out_dtype=torch.float32)
        assert_close("o (f32 out)", f64(sel(out32)), o_ref, w.dtype)
        assert torch.equal(S32, S), "the output dtype must not change the state"
        # the bf16 output is the float output rounded to nearest even
        assert torch.equal(out32.to(torch.bfloat16), out), "bf16 out != rne(f32 out)"


# ------------------------------------------------------------------ decode

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_decode_small(mode, dtype, dk, dv):
    w = WORKLOADS[5].scaled(mode=mode, dtype=dtype, B=3, H=5, dk=dk, dv=dv, steps=4, seed=11)
    log(f"decode small {w}")
    x = workloads.make_inputs(w)
    d = to_cuda(x)
    S = d["S0"].clone()
    outs = [la.decode_step(d["q"][n], d["k"][n], d["v"][n], d["log_alpha"][n],
                           d["beta"][n], S, mode=mode) for n in range(w.steps)]
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_decode(x, mode)
    assert_close("o", np.stack([f64(o) for o in outs]), o_ref, dtype, bf16_out=dtype == "bf16")
    assert_close("S", f64(S), S_ref, dtype)
    if dtype == "bf16":
        S2 = d["S0"].clone()
        outs = [la.decode_step(d["q"][n], d["k"][n], d["v"][n], d["log_alpha"][n],
                               d["beta"][n], S2, mode=mode, out_dtype=torch.float32)
                for n in range(w.steps)]
        torch.cuda.synchronize()
        assert_close("o (f32 out)", np.stack([f64(o) for o in outs]), o_ref, dtype)
        assert torch.equal(S2, S)


def test_decode_full_size_sampled():
    """B=256, H=32, d=128, 128 steps in place, as the bench runs it; the
    oracle follows 12 sampled (b, h) states through all 128 steps."""
    w = WORKLOADS[5]
    log(f"decode full {w}")
    x = workloads.make_inputs(w)
    d = to_cuda(x)
    S = d["S0"].clone()
    outs = torch.empty((w.steps, w.B, w.H, w.dv), dtype=w.torch_dtype, device="cuda")
    for n in range(w.steps):
        la.decode_step(d["q"][n], d["k"][n], d["v"][n], d["log_alpha"][n], d["beta"][n], S,
                       mode=w.mode, out=outs[n])
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    heads = [(0, 0), (w.B - 1, w.H - 1)] + [(int(b), int(h)) for b, h in
                                            zip(rng.integers(0, w.B, 10), rng.integers(0, w.H, 10))]
    # the same 128 steps with a float32 output
    S32 = d["S0"].clone()
    outs32 = torch.empty((w.steps, w.B, w.H, w.dv), dtype=torch.float32, device="cuda")
    for n in range(w.steps):
        la.decode_step(d["q"][n], d["k"][n], d["v"][n], d["log_alpha"][n], d["beta"][n], S32,
                       mode=w.mode, out=outs32[n])
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_decode(x, w.mode, heads)
    bs = [b for b, _ in heads]
    hs = [h for _, h in heads]
    assert_out_pair("o[sampled]", outs[:, bs, hs], outs32[:, bs, hs], o_ref, w.dtype)
    assert_close("S[sampled]", f64(S[bs, hs]), S_ref, w.dtype)
    assert torch.equal(S32, S), "the output dtype must not change the state"


# ------------------------------------------------------------------ chunk forward

@pytest.mark.parametrize("s0", [0.0, 0.3])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", MODES)
def test_chunk_small(mode, dtype, d, s0):
    """B=2, H=3, L=320 (5 chunks): every output and state element."""
    w = recipe(mode, dtype, B=2, H=3, L=320, d=d, s0_std=s0)
    log(f"chunk small {w}")
    x = workloads.make_inputs(w)
    o_ref, S_ref = oracle_fwd(x, mode)
    check_fwd(w, x, o_ref, S_ref)


@pytest.mark.parametrize("mode", ["linear", "gated_linear"])
@pytest.mark.parametrize("d", [64, 128])
def test_no_erase_repeat_bit_identical(mode, d):
    """Ten calls on the same inputs agree bit for bit (a read of a tile still
    being written by the DMA would not), and the first matches the oracle;
    lengths with 1, 2, 3 and 5 chunks and a ragged tail.  (Batches this
    small run the chain kernel; tests/test_wide_gpu.py repeats the check on
    the wide kernel.)"""
    for L in (40, 128, 170, 320):
        w = recipe(mode, "bf16", B=2, H=3, L=L, d=d, s0_std=0.3 if L != 128 else 0.0, seed=L)
        log(f"wide repeat {w}")
        x = workloads.make_inputs(w)
        dev = to_cuda(x)
        s0 = dev["S0"] if w.s0_std > 0 else None
        outs = []
        for _ in range(10):
            o, S = la.chunk_fwd(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], s0,
                                mode=mode, C=w.C, return_state=True, out_dtype=torch.float32)
            outs.append((o.clone(), S.clone()))
        torch.cuda.synchronize()
        for o, S in outs[1:]:
            assert torch.equal(o, outs[0][0]) and torch.equal(S, outs[0][1]), \
                f"{w}: repeated calls differ"
        o_ref, S_ref = oracle_fwd(x, mode)
        assert_close("o (f32 out)", f64(outs[0][0]), o_ref, "bf16")
        assert_close("S_final", f64(outs[0][1]), S_ref, "bf16")


@pytest.mark.parametrize("mode", MODES)
def test_chunk_single_chunk_single_head(mode):
    w = recipe(mode, "bf16", B=1, H=1, L=64, d=128, s0_std=0.5, seed=3)
    log(f"chunk one chunk {w}")
    x = workloads.make_inputs(w)
    o_ref, S_ref = oracle_fwd(x, mode)
    check_fwd(w, x, o_ref, S_ref)


@pytest.mark.parametrize("L", [128, 192, 256])
@pytest.mark.parametrize("mode", MODES)
def test_chunk_short_sequences(mode, L):
    """2, 3 and 4 chunks: the load pipeline runs two chunks ahead, so these
    are the lengths where its prologue and drain overlap."""
    w = recipe(mode, "bf16", B=1, H=2, L=L, d=64, s0_std=0.3, seed=11)
    log(f"chunk short {w}")
    x = workloads.make_inputs(w)
    o_ref, S_ref = oracle_fwd(x, mode)
    check_fwd(w, x, o_ref, S_ref)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("bf16", 128), ("f32", 128)])
@pytest.mark.parametrize("mode", MODES)
def test_chunk_ragged_lengths(mode, dtype, d):
    """L not a multiple of C: one partial chunk (L = 1, 37), a full chunk
    and a partial one (L = 69), and a partial chunk after the load pipeline
    has reached its steady state (L = 389).  The output buffer is one row
    longer than the call's out and pre-filled with NaN: the row past the end
    must stay untouched, every row before it written."""
    for L in (1, 37, 69, 389):
        w = recipe(mode, dtype, B=1, H=3, L=L, d=d, s0_std=0.3, seed=41 + L)
        log(f"chunk ragged {w}")
        x = workloads.make_inputs(w)
        o_ref, S_ref = oracle_fwd(x, mode)
        check_fwd(w, x, o_ref, S_ref)
        dev = to_cuda(x)
        big = torch.full((w.B * w.H * w.L * w.dv + w.dv,), float("nan"), dtype=w.torch_dtype,
                         device="cuda")
        out = big[: w.B * w.H * w.L * w.dv].view(w.B, w.H, w.L, w.dv)
        la.chunk_fwd(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], dev["S0"],
                     mode=mode, out=out)
        torch.cuda.synchronize()
        assert torch.isnan(big[w.B * w.H * w.L * w.dv:]).all(), "a store went past the end"
        assert_close("o (guarded)", f64(out), o_ref, dtype, bf16_out=dtype == "bf16")


def _packed(lens, H, d, dtype, mode, seed):
    """A packed batch of sequences of the given lengths: the workloads'
    recipe drawn as one [1, H, T, d] sequence and cut at the offsets, plus
    one initial state per sequence."""
    T = int(sum(lens))
    w = recipe(mode, dtype, B=1, H=H, L=max(T, 1), d=d, s0_std=0.3, seed=seed)
    x = workloads.make_inputs(w)
    gen = torch.Generator("cpu")
    gen.manual_seed(seed + 1)
    S0 = torch.randn((len(lens), H, d, d), generator=gen, dtype=torch.float32) * 0.3
    x = {n: t[0, :, :T].contiguous() for n, t in x.items() if n != "S0"}
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    return w, x, S0, cu


def _packed_oracle(x, S0, cu, mode):
    """The oracle run on each sequence on its own."""
    y = {n: t.to(torch.float64).numpy() for n, t in x.items()}
    s0 = S0.to(torch.float64).numpy()
    H, T, dv = y["v"].shape
    o = np.zeros((H, T, dv))
    S = np.empty_like(s0)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if a == b:
            S[s] = s0[s]
            continue
        sl = lambda t: t[None, :, a:b]   # noqa: E731  -> [1, H, len, ...]
        os_, Ss = oracle.recurrent_fwd(sl(y["q"]), sl(y["k"]), sl(y["v"]), sl(y["log_alpha"]),
                                       sl(y["beta"]), s0[s][None], mode)
        o[:, a:b] = os_[0]
        S[s] = Ss[0]
    return o, S


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("bf16", 128)])
@pytest.mark.parametrize("mode", MODES)
def test_chunk_varlen_packed(mode, dtype, d):
    """A packed batch of 9 sequences: empty ones (first, middle, last), a
    single token, partial and exact chunks, and several chunks; every token
    and every final state against the oracle run per sequence.  out and
    S_final start as NaN: all of out and every state must be written."""
    lens = [0, 1, 63, 64, 0, 65, 200, 130, 0]
    H = 3
    w, x, S0, cu = _packed(lens, H, d, dtype, mode, seed=61)
    log(f"chunk varlen {mode} {dtype} d{d} H{H} lens {lens}")
    o_ref, S_ref = _packed_oracle(x, S0, cu, mode)
    dev = {n: t.cuda() for n, t in x.items()}
    T = int(cu[-1])
    out = torch.full((H, T, d), float("nan"), dtype=w.torch_dtype, device="cuda")
    S = torch.full((len(lens), H, d, d), float("nan"), dtype=torch.float32, device="cuda")
    la.chunk_fwd_varlen(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"],
                        S0.cuda(), cu.cuda(), mode=mode, out=out, S_final=S)
    torch.cuda.synchronize()
    if dtype == "bf16":
        out32 = torch.full((H, T, d), float("nan"), dtype=torch.float32, device="cuda")
        _, S32 = la.chunk_fwd_varlen(dev["q"], dev["k"], dev["v"], dev["log_alpha"],
                                     dev["beta"], S0.cuda(), cu.cuda(), mode=mode, out=out32)
        torch.cuda.synchronize()
        assert_out_pair("o", out, out32, o_ref, dtype)
        assert torch.equal(S32, S), "the output dtype must not change the state"
    else:
        assert_close("o", f64(out), o_ref, dtype)
    assert_close("S_final", f64(S), S_ref, dtype)
    # empty sequences pass their state through unchanged
    for s, n in enumerate(lens):
        if n == 0:
            assert torch.equal(S[s].cpu(), S0[s]), f"sequence {s} (empty) changed its state"
    # and the packed call equals the fixed-length call on each sequence
    for s in (2, 6):
        a, b = int(cu[s]), int(cu[s + 1])
        o1, S1 = la.chunk_fwd(*(dev[n][None, :, a:b].contiguous() for n in ("q", "k", "v")),
                              dev["log_alpha"][None, :, a:b].contiguous(),
                              dev["beta"][None, :, a:b].contiguous(), S0[s][None].cuda(),
                              mode=mode)
        torch.cuda.synchronize()
        assert torch.equal(o1[0], out[:, a:b]) and torch.equal(S1[0], S[s]), (
            f"sequence {s}: packed and fixed-length calls differ")


def _nonunit_keys(w, x, seed):
    """Keys rescaled per token by a factor drawn uniform in [0.5, 1.5]: the
    recurrence is defined for any |k|, and larger keys grow the entries of
    A = strict_lower(diag(beta) K K^T * Gamma) that the T solve inverts
    (beta |k|^2 up to 2.25: the erase can overshoot)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    lead = x["k"].shape[:-1]
    scale = 0.5 + torch.rand(lead + (1,), generator=gen)
    return dict(x, k=(x["k"].float() * scale).to(x["k"].dtype))


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("bf16", 128), ("f32", 128)])
@pytest.mark.parametrize("mode", ("delta", "gated_delta"))
def test_chunk_nonunit_keys(mode, dtype, d):
    """The delta modes with |k| in [0.5, 1.5] over 5 full chunks and a
    partial one, with S0: every element of the forward against the oracle
    (bf16: float and bf16 outputs); the sequence-parallel forward (P = 3);
    and 12 decode steps."""
    w = recipe(mode, dtype, B=2, H=2, L=64 * 5 + 13, d=d, s0_std=0.3, seed=113)
    log(f"chunk non-unit keys {w}")
    x = _nonunit_keys(w, workloads.make_inputs(w), 114)
    o_ref, S_ref = oracle_fwd(x, mode)
    check_fwd(w, x, o_ref, S_ref)
    dev = to_cuda(x)
    if dtype == "bf16":
        out, S = _seg_call(dev, mode, 3, dev["S0"])
        out32, _ = _seg_call(dev, mode, 3, dev["S0"], out_dtype=torch.float32)
        assert_out_pair("o P=3", out, out32, o_ref)
        assert_close("S_final P=3", f64(S), S_ref, "bf16")
    steps = 12
    col = lambda t, n: t[:, :, n].contiguous()       # noqa: E731
    Sd = dev["S0"].clone()
    outs = [la.decode_step(col(dev["q"], n), col(dev["k"], n), col(dev["v"], n),
                           col(dev["log_alpha"], n), col(dev["beta"], n), Sd, mode=mode,
                           out_dtype=torch.float32) for n in range(steps)]
    torch.cuda.synchronize()
    y = workloads.to_f64(x)
    mv = lambda t: np.moveaxis(t, 2, 0)[:steps]      # noqa: E731
    o_d, S_d = oracle.decode_steps(y["S0"], mv(y["q"]), mv(y["k"]), mv(y["v"]),
                                   mv(y["log_alpha"]), mv(y["beta"]), mode)
    assert_close("decode o", np.stack([f64(o) for o in outs]), o_d, dtype)
    assert_close("decode S", f64(Sd), S_d, dtype)


# ------------------------------------------------------------------ sequence-parallel

def _seg_call(d, mode, P, S0=None, S_final=None, out_dtype=None):
    out, S = la.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], S0, mode=mode,
                          segments=P, S_final=S_final, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, S


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode", MODES)
def test_chunk_segmented(mode, d):
    """Each sequence cut into P parallel segments (state pass, scan, output
    pass) over 9 full chunks and a partial one: P = 2 (no transition), 3,
    7 and 10 (one chunk per segment, the partial one last), every element
    against the oracle; the bf16 output is the float one rounded; the
    in-place state update (S_final is S0) works as in the whole walk."""
    w = recipe(mode, "bf16", B=2, H=1, L=64 * 9 + 23, d=d, s0_std=0.3, seed=53)
    x = workloads.make_inputs(w)
    o_ref, S_ref = oracle_fwd(x, mode)
    dev = to_cuda(x)
    for P in (2, 3, 7, 10):
        log(f"chunk segmented P={P} {w}")
        out, S = _seg_call(dev, mode, P, dev["S0"])
        out32, S32 = _seg_call(dev, mode, P, dev["S0"], out_dtype=torch.float32)
        assert_out_pair(f"o P={P}", out, out32, o_ref)
        assert_close(f"S_final P={P}", f64(S), S_ref, "bf16")
        assert torch.equal(S32, S), "the output dtype must not change the state"
    S_io = dev["S0"].clone()
    _seg_call(dev, mode, 7, S_io, S_final=S_io)
    assert_close("S in place P=7", f64(S_io), S_ref, "bf16")


@pytest.mark.parametrize("mode", MODES)
def test_chunk_segmented_zero_state_and_single(mode):
    """No S0 (the scan starts from zeros), and P = 1 through the segmented
    entry point is the whole-sequence walk, bit for bit."""
    w = recipe(mode, "bf16", B=1, H=3, L=64 * 6, d=128, s0_std=0.0, seed=59)
    log(f"chunk segmented zero state {w}")
    x = workloads.make_inputs(w)
    o_ref, S_ref = oracle_fwd(x, mode)
    dev = to_cuda(x)
    out, S = _seg_call(dev, mode, 4)
    out32, _ = _seg_call(dev, mode, 4, out_dtype=torch.float32)
    assert_out_pair("o P=4", out, out32, o_ref)
    assert_close("S_final P=4", f64(S), S_ref, "bf16")
    a_o, a_S = _seg_call(dev, mode, 1)
    b_o, b_S = la.chunk_fwd(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], None,
                            mode=mode)
    torch.cuda.synchronize()
    assert torch.equal(a_o, b_o) and torch.equal(a_S, b_S)


@pytest.mark.parametrize("mode", MODES)
def test_chunk_auto_segments(mode):
    """One long sequence: la_chunk_fwd cuts it by itself (the plan says
    P > 1), every element against the oracle."""
    w = recipe(mode, "bf16", B=1, H=1, L=4096 + 40, d=128, s0_std=0.2, seed=61)
    P = la.chunk_segments(w.B, w.H, w.L, w.dk, w.dv, mode=mode)
    log(f"chunk auto segments P={P} {w}")
    assert P > 1
    x = workloads.make_inputs(w)
    o_ref, S_ref = oracle_fwd(x, mode)
    check_fwd(w, x, o_ref, S_ref)


def test_chunk_shard_sampled():
    """One GPU's share of workload 4 over 8 GPUs (B=1 H=4 L=65536 d=128) as
    the bench runs it: sequence-parallel by the plan; the oracle recomputes
    2 heads over the whole sequence."""
    w = workloads.WORKLOAD4_SHARD8
    P = la.chunk_segments(w.B, w.H, w.L, w.dk, w.dv, mode=w.mode)
    log(f"chunk shard P={P} {w}")
    assert P > 1
    x = workloads.make_inputs(w)
    heads = [(0, 0), (0, w.H - 1)]
    o_ref, S_ref = oracle_fwd(x, w.mode, heads)
    check_fwd(w, x, o_ref, S_ref, sel=lambda t: t[[0, 0], [0, w.H - 1]])


# ------------------------------------------------------------------ fused prologue

PRO = {"gates": 1, "norm": 2, "both": 3}
GATE_SCALE = 1.0 / 16.0


def _raw(w, flags):
    """Raw inputs and the gates to pass: q, k not normalised when the
    prologue normalises them (else the recipe's prepared q, k, as a caller
    without that step passes them), raw gate scores next to the activated
    values (float32, computed here in front of the op)."""
    r = workloads.make_raw_inputs(w)
    if not flags & 2:
        x = workloads.make_inputs(w)
        r["q"], r["k"] = x["q"], x["k"]
    r["log_alpha"] = -torch.nn.functional.softplus(r["a_raw"]) * GATE_SCALE
    r["beta"] = torch.sigmoid(r["b_raw"])
    return r


def _fused_oracle(r, mode, flags, heads=None):
    """The oracle's prologue (oracle.prepare) on the raw float64 inputs,
    then its recurrence; gates not activated by the prologue are the float32
    values the device received."""
    y = {key: t.to(torch.float64).numpy() for key, t in r.items()}
    a = y["a_raw"] if flags & 1 else y["log_alpha"]
    b = y["b_raw"] if flags & 1 else y["beta"]
    q, k, la, be = oracle.prepare(y["q"], y["k"], a, b, mode, flags, GATE_SCALE)
    v, S0 = y["v"], y["S0"]
    if heads is not None:
        bs, hs = [b_ for b_, _ in heads], [h for _, h in heads]
        sel = lambda t: t[bs, hs][None]       # noqa: E731
        o, S = oracle.recurrent_fwd(sel(q), sel(k), sel(v), sel(la), sel(be), sel(S0), mode)
        return o[0], S[0]
    return oracle.recurrent_fwd(q, k, v, la, be, S0, mode)


def _fused_call(d, mode, flags, out_dtype=None):
    a = d["a_raw"] if flags & 1 else d["log_alpha"]
    b = d["b_raw"] if flags & 1 else d["beta"]
    out, S = la.chunk_fwd(d["q"], d["k"], d["v"], a, b, d["S0"], mode=mode,
                          qk_l2norm=bool(flags & 2), gate_act=bool(flags & 1),
                          gate_scale=GATE_SCALE, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, S


@pytest.mark.parametrize("flags", ["gates", "norm", "both"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode", MODES)
def test_chunk_fused_prologue(mode, d, flags):
    """Raw q, k (N(0, 1), not normalised) and raw gate scores: the T-solve
    kernel activates the gates and folds the inverse norms of q and k into
    the decay tables; every element against the oracle's prologue and
    recurrence, over 5 full chunks and a partial one, with S0.  The bf16
    output is the float one rounded."""
    f = PRO[flags]
    w = recipe(mode, "bf16", B=2, H=2, L=64 * 5 + 13, d=d, s0_std=0.3, seed=67)
    log(f"chunk fused prologue {flags} {w}")
    r = _raw(w, f)
    o_ref, S_ref = _fused_oracle(r, mode, f)
    dev = to_cuda(r)
    out, S = _fused_call(dev, mode, f)
    out32, S32 = _fused_call(dev, mode, f, out_dtype=torch.float32)
    assert_out_pair("o", out, out32, o_ref)
    assert_close("S_final", f64(S), S_ref, "bf16")
    assert torch.equal(S32, S)


@pytest.mark.parametrize("mode", MODES)
def test_chunk_fused_prologue_segmented(mode):
    """The fused prologue on one long sequence, which the plan runs
    sequence-parallel (state pass, scan and output pass with the folded
    tables)."""
    w = recipe(mode, "bf16", B=1, H=1, L=4096 + 40, d=128, s0_std=0.2, seed=71)
    P = la.chunk_segments(w.B, w.H, w.L, w.dk, w.dv, mode=mode)
    log(f"chunk fused prologue segmented P={P} {w}")
    assert P > 1
    r = _raw(w, 3)
    o_ref, S_ref = _fused_oracle(r, mode, 3)
    dev = to_cuda(r)
    out, S = _fused_call(dev, mode, 3)
    out32, _ = _fused_call(dev, mode, 3, out_dtype=torch.float32)
    assert_out_pair("o", out, out32, o_ref)
    assert_close("S_final", f64(S), S_ref, "bf16")


def test_chunk_fused_no_flags_is_plain_forward():
    """flags = 0 is la_chunk_fwd, bit for bit."""
    w = recipe("gated_delta", "bf16", B=1, H=2, L=300, d=128, s0_std=0.2, seed=73)
    log(f"chunk fused flags 0 {w}")
    dev = to_cuda(_raw(w, 0))
    a = _fused_call(dev, "gated_delta", 0)
    b = la.chunk_fwd(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], dev["S0"],
                     mode="gated_delta")
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_chunk_fused_shard_sampled():
    """One GPU's share of workload 4 from raw inputs with the whole prologue
    fused, as a model layer would call it; 2 heads against the oracle."""
    w = workloads.WORKLOAD4_SHARD8
    log(f"chunk fused shard {w}")
    r = _raw(w, 3)
    heads = [(0, 0), (0, w.H - 1)]
    o_ref, S_ref = _fused_oracle(r, w.mode, 3, heads)
    dev = to_cuda(r)
    out, S = _fused_call(dev, w.mode, 3)
    sel = lambda t: t[[0, 0], [0, w.H - 1]]   # noqa: E731
    out32 = _fused_call(dev, w.mode, 3, out_dtype=torch.float32)[0]
    assert_out_pair("o", sel(out), sel(out32), o_ref)
    assert_close("S_final", f64(sel(S)), S_ref, "bf16")


@pytest.mark.parametrize("mode", MODES)
def test_fused_extreme_inputs(mode):
    """Raw gate scores of +-40 (softplus and sigmoid must not overflow: alpha
    -> 0, beta -> 0 or 1), an all-zero q row and an all-zero k row (the eps
    inside the norm keeps them zero), and a zero-valued token (its output
    row may be all zero: the output norm's eps keeps it finite) -- forward
    and decode against the oracle, every value finite."""
    w = recipe(mode, "bf16", B=1, H=2, L=64 * 2 + 9, d=128, s0_std=0.3, seed=107)
    log(f"fused extreme inputs {w}")
    r = _raw(w, 3)
    r["a_raw"][0, 0, 5:9] = torch.tensor([40.0, -40.0, 40.0, -40.0])
    r["b_raw"][0, 0, 5:9] = torch.tensor([-40.0, 40.0, 40.0, -40.0])
    r["q"][0, 1, 3] = 0
    r["k"][0, 1, 7] = 0
    r["v"][0, 1, 0] = 0
    r["q"][0, 1, 0] = 0
    D, nw = _epi_params(w, 108)
    o_ref, S_ref = _fused_oracle(r, mode, 3)
    o_ref = _epi_oracle(o_ref, r["v"].double().numpy(), D, nw, True, True, 1e-6)
    dev = to_cuda(r)
    out, S = la.chunk_fwd(dev["q"], dev["k"], dev["v"], dev["a_raw"], dev["b_raw"], dev["S0"],
                          mode=mode, qk_l2norm=True, gate_act=True, gate_scale=GATE_SCALE,
                          dskip=D.cuda(), out_norm=True, norm_weight=nw.cuda())
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(S).all()
    assert_close("o", f64(out), o_ref, "bf16", bf16_out=True)
    assert_close("S_final", f64(S), S_ref, "bf16")
    # float output at the plain bound (the output norm of a bf16 output reads
    # its rounded values, so the two outputs differ by more than one rounding)
    out32, _ = la.chunk_fwd(dev["q"], dev["k"], dev["v"], dev["a_raw"], dev["b_raw"], dev["S0"],
                            mode=mode, qk_l2norm=True, gate_act=True, gate_scale=GATE_SCALE,
                            dskip=D.cuda(), out_norm=True, norm_weight=nw.cuda(),
                            out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close("o (f32 out)", f64(out32), o_ref, "bf16")
    # the same tokens one by one through the fused decode step
    y = {key: t.to(torch.float64).numpy() for key, t in r.items()}
    q, k, lg, be = oracle.prepare(y["q"], y["k"], y["a_raw"], y["b_raw"], mode, 3, GATE_SCALE)
    steps = 12
    mv = lambda t: np.moveaxis(t, 2, 0)[:steps]      # noqa: E731
    o_d, S_d = oracle.decode_steps(y["S0"], mv(q), mv(k), mv(y["v"]), mv(lg), mv(be), mode)
    o_d = np.moveaxis(_epi_oracle(np.moveaxis(o_d, 0, 2), y["v"][:, :, :steps], D, nw, True,
                                  True, 1e-6), 2, 0)
    Sg = dev["S0"].clone()
    col = lambda t, n: t[:, :, n].contiguous()       # noqa: E731
    outs = [la.decode_step(col(dev["q"], n), col(dev["k"], n), col(dev["v"], n),
                           col(dev["a_raw"], n), col(dev["b_raw"], n), Sg, mode=mode,
                           qk_l2norm=True, gate_act=True, gate_scale=GATE_SCALE, dskip=D.cuda(),
                           out_norm=True, norm_weight=nw.cuda()) for n in range(steps)]
    torch.cuda.synchronize()
    od = np.stack([f64(o) for o in outs])
    assert np.all(np.isfinite(od)) and torch.isfinite(Sg).all()
    assert_close("decode o", od, o_d, "bf16", bf16_out=True)
    assert_close("decode S", f64(Sg), S_d, "bf16")
    Sg32 = dev["S0"].clone()
    outs32 = [la.decode_step(col(dev["q"], n), col(dev["k"], n), col(dev["v"], n),
                             col(dev["a_raw"], n), col(dev["b_raw"], n), Sg32, mode=mode,
                             qk_l2norm=True, gate_act=True, gate_scale=GATE_SCALE,
                             dskip=D.cuda(), out_norm=True, norm_weight=nw.cuda(),
                             out_dtype=torch.float32) for n in range(steps)]
    torch.cuda.synchronize()
    assert_out_pair("decode o", torch.stack(outs), torch.stack(outs32), o_d)
    assert torch.equal(Sg32, Sg)


@pytest.mark.parametrize("flags", ["gates", "norm", "both"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", MODES)
def test_decode_fused_prologue(mode, dtype, flags):
    """Decode steps from raw inputs: 12 steps of B=3 H=2 d=128 against the
    oracle's prologue and decode."""
    f = PRO[flags]
    w = Workload(f"decode_{mode}_{dtype}", mode, dtype, B=3, H=2, L=1, dk=128, dv=128, C=1,
                 qk_norm=True, qkv_scale=1.0, s0_std=0.3, steps=12, seed=79)
    log(f"decode fused prologue {flags} {w}")
    r = _raw(w, f)
    y = {key: t.to(torch.float64).numpy() for key, t in r.items()}
    a = y["a_raw"] if f & 1 else y["log_alpha"]
    b = y["b_raw"] if f & 1 else y["beta"]
    q, k, lg, be = oracle.prepare(y["q"], y["k"], a, b, mode, f, GATE_SCALE)
    o_ref, S_ref = oracle.decode_steps(y["S0"], q, k, y["v"], lg, be, mode)
    d = to_cuda(r)
    S = d["S0"].clone()
    ga = d["a_raw"] if f & 1 else d["log_alpha"]
    gb = d["b_raw"] if f & 1 else d["beta"]
    outs = [la.decode_step(d["q"][n], d["k"][n], d["v"][n], ga[n], gb[n], S, mode=mode,
                           qk_l2norm=bool(f & 2), gate_act=bool(f & 1), gate_scale=GATE_SCALE)
            for n in range(w.steps)]
    torch.cuda.synchronize()
    assert_close("o", np.stack([f64(o) for o in outs]), o_ref, dtype, bf16_out=dtype == "bf16")
    assert_close("S", f64(S), S_ref, dtype)


def _epi_params(w, seed):
    gen = torch.Generator("cpu").manual_seed(seed)
    D = torch.randn((w.H, w.dv), generator=gen) * 0.5
    nw = 1.0 + 0.1 * torch.randn((w.H, w.dv), generator=gen)
    return D, nw


def _epi_oracle(o, v, D, nw, dskip, norm, eps):
    if dskip:
        o = oracle.add_dskip(o, v, D.double().numpy())
    if norm:
        o = oracle.out_norm(o, nw.double().numpy(), eps)
    return o


@pytest.mark.parametrize("steps", ["dskip", "norm", "all"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode", MODES)
def test_chunk_fused_epilogue(mode, d, steps):
    """The residual D v added by the output waves and the output norm (its
    own pass over out), alone and after the whole prologue; every element
    against the oracle's prologue, recurrence and epilogue, over 5 full
    chunks and a partial one."""
    dskip, norm = steps in ("dskip", "all"), steps in ("norm", "all")
    f = 3 if steps == "all" else 0
    w = recipe(mode, "bf16", B=2, H=2, L=64 * 5 + 13, d=d, s0_std=0.3, seed=83)
    log(f"chunk fused epilogue {steps} {w}")
    r = _raw(w, f)
    D, nw = _epi_params(w, 84)
    o_ref, S_ref = _fused_oracle(r, mode, f)
    o_ref = _epi_oracle(o_ref, r["v"].double().numpy(), D, nw, dskip, norm, 1e-5)
    dev = to_cuda(r)
    a = dev["a_raw"] if f & 1 else dev["log_alpha"]
    b = dev["b_raw"] if f & 1 else dev["beta"]
    for odt in (None, torch.float32):
        out, S = la.chunk_fwd(dev["q"], dev["k"], dev["v"], a, b, dev["S0"], mode=mode,
                              qk_l2norm=bool(f & 2), gate_act=bool(f & 1), gate_scale=GATE_SCALE,
                              dskip=D.cuda() if dskip else None, out_norm=norm,
                              norm_weight=nw.cuda() if norm else None, norm_eps=1e-5,
                              out_dtype=odt)
        torch.cuda.synchronize()
        assert_close(f"o ({odt})", f64(out), o_ref, "bf16", bf16_out=odt is None)
        assert_close("S_final", f64(S), S_ref, "bf16")


def test_chunk_fused_all_segmented():
    """Every fused step on one long gated-delta sequence, which the plan
    runs sequence-parallel."""
    mode = "gated_delta"
    w = recipe(mode, "bf16", B=1, H=1, L=4096 + 40, d=128, s0_std=0.2, seed=89)
    P = la.chunk_segments(w.B, w.H, w.L, w.dk, w.dv, mode=mode)
    log(f"chunk fused all segmented P={P} {w}")
    assert P > 1
    r = _raw(w, 3)
    D, nw = _epi_params(w, 90)
    o_ref, S_ref = _fused_oracle(r, mode, 3)
    o_ref = _epi_oracle(o_ref, r["v"].double().numpy(), D, nw, True, True, 1e-6)
    dev = to_cuda(r)
    out, S = la.chunk_fwd(dev["q"], dev["k"], dev["v"], dev["a_raw"], dev["b_raw"], dev["S0"],
                          mode=mode, qk_l2norm=True, gate_act=True, gate_scale=GATE_SCALE,
                          dskip=D.cuda(), out_norm=True, norm_weight=nw.cuda())
    torch.cuda.synchronize()
    assert_close("o", f64(out), o_ref, "bf16", bf16_out=True)
    assert_close("S_final", f64(S), S_ref, "bf16")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", MODES)
def test_decode_fused_epilogue(mode, dtype):
    """Decode steps with every fused step (the norm over dv reduced inside
    the kernel): 12 steps of B=3 H=2 d=128 against the oracle."""
    w = Workload(f"decode_{mode}_{dtype}", mode, dtype, B=3, H=2, L=1, dk=128, dv=128, C=1,
                 qk_norm=True, qkv_scale=1.0, s0_std=0.3, steps=12, seed=97)
    log(f"decode fused epilogue {w}")
    r = _raw(w, 3)
    D, nw = _epi_params(w, 98)
    y = {key: t.to(torch.float64).numpy() for key, t in r.items()}
    q, k, lg, be = oracle.prepare(y["q"], y["k"], y["a_raw"], y["b_raw"], mode, 3, GATE_SCALE)
    o_ref, S_ref = oracle.decode_steps(y["S0"], q, k, y["v"], lg, be, mode)
    # [N, B, H, dv] -> [B, H, N, dv] for the epilogue, and back
    o_ref = np.moveaxis(_epi_oracle(np.moveaxis(o_ref, 0, 2), np.moveaxis(y["v"], 0, 2), D, nw,
                                    True, True, 1e-6), 2, 0)
    d = to_cuda(r)
    S = d["S0"].clone()
    outs = [la.decode_step(d["q"][n], d["k"][n], d["v"][n], d["a_raw"][n], d["b_raw"][n], S,
                           mode=mode, qk_l2norm=True, gate_act=True, gate_scale=GATE_SCALE,
                           dskip=D.cuda(), out_norm=True, norm_weight=nw.cuda())
            for n in range(w.steps)]
    torch.cuda.synchronize()
    assert_close("o", np.stack([f64(o) for o in outs]), o_ref, dtype, bf16_out=dtype == "bf16")
    assert_close("S", f64(S), S_ref, dtype)


# ------------------------------------------------------------------ non-causal form

def _nc_oracle(x, heads=None):
    y = workloads.to_f64(x)
    if heads is not None:
        bs, hs = [b for b, _ in heads], [h for _, h in heads]
        sel = lambda t: t[bs, hs][None]      # noqa: E731
        o, S = oracle.noncausal_fwd(sel(y["q"]), sel(y["k"]), sel(y["v"]), sel(y["S0"]))
        return o[0], S[0]
    return oracle.noncausal_fwd(y["q"], y["k"], y["v"], y["S0"])


@pytest.mark.parametrize("L", [1, 64 * 5 + 13])
@pytest.mark.parametrize("d", [64, 128])
def test_noncausal_small(d, L):
    """O = Q (S0 + K^T V): every element against the oracle, bf16 and float
    outputs, with S0, one token and a ragged length; S_final == S0 in place."""
    w = recipe("linear", "bf16", B=2, H=3, L=L, d=d, s0_std=0.3, seed=101)
    log(f"noncausal small {w}")
    x = workloads.make_inputs(w)
    o_ref, S_ref = _nc_oracle(x)
    dev = to_cuda(x)
    out, S = la.noncausal_fwd(dev["q"], dev["k"], dev["v"], dev["S0"])
    out32, S32 = la.noncausal_fwd(dev["q"], dev["k"], dev["v"], dev["S0"],
                                  out_dtype=torch.float32)
    S_io = dev["S0"].clone()
    la.noncausal_fwd(dev["q"], dev["k"], dev["v"], S_io, S_final=S_io)
    torch.cuda.synchronize()
    assert_close("o", f64(out), o_ref, "bf16", bf16_out=True)
    assert_close("o (f32 out)", f64(out32), o_ref, "bf16")
    assert_close("S", f64(S), S_ref, "bf16")
    assert torch.equal(S32, S) and torch.equal(out32.to(torch.bfloat16), out)
    assert_close("S in place", f64(S_io), S_ref, "bf16")


def test_noncausal_long_few_heads():
    """One long sequence per head (the sum pass cut into parallel segments)
    and the linear workload's shape, sampled heads against the oracle."""
    w = recipe("linear", "bf16", B=1, H=2, L=20000, d=128, s0_std=0.1, seed=103)
    log(f"noncausal long {w}")
    x = workloads.make_inputs(w)
    o_ref, S_ref = _nc_oracle(x)
    dev = to_cuda(x)
    out, S = la.noncausal_fwd(dev["q"], dev["k"], dev["v"], dev["S0"])
    torch.cuda.synchronize()
    assert_close("o", f64(out), o_ref, "bf16", bf16_out=True)
    assert_close("S", f64(S), S_ref, "bf16")
    w = WORKLOADS[2]
    log(f"noncausal full {w}")
    x = workloads.make_inputs(w)
    heads = [(0, 0), (w.B - 1, w.H - 1)]
    o_ref, S_ref = _nc_oracle(x, heads)
    dev = to_cuda(x)
    out, S = la.noncausal_fwd(dev["q"], dev["k"], dev["v"], None)
    torch.cuda.synchronize()
    sel = lambda t: t[[0, w.B - 1], [0, w.H - 1]]   # noqa: E731
    assert_close("o", f64(sel(out)), o_ref, "bf16", bf16_out=True)
    assert_close("S", f64(sel(S)), S_ref, "bf16")


def test_chunk_workload1_full():
    """Gated delta, float32, B=1 H=2 L=256 d=64: all elements, rel 1e-4."""
    w = WORKLOADS[1]
    log(f"chunk full {w}")
    x = workloads.make_inputs(w)
    o_ref, S_ref = oracle_fwd(x, w.mode)
    check_fwd(w, x, o_ref, S_ref)


@pytest.mark.parametrize("wid", [2, 3, 4])
def test_chunk_full_size_sampled(wid):
    """Workloads 2-4 at full size, launched as the bench launches them; the
    oracle recomputes 2 sampled heads over the whole sequence."""
    w = WORKLOADS[wid]
    log(f"chunk full {w}")
    x = workloads.make_inputs(w)
    heads = [(0, 0), (w.B - 1, w.H - 1)]
    bs = [b for b, _ in heads]
    hs = [h for _, h in heads]
    o_ref, S_ref = oracle_fwd(x, w.mode, heads)
    check_fwd(w, x, o_ref, S_ref, sel=lambda t: t[bs, hs])


# ------------------------------------------------------------------ properties

@pytest.mark.parametrize("mode", MODES)
def test_state_carry_and_in_place(mode):
    """fwd(L1) then fwd(L2, S0 = S_final) equals fwd(L1 + L2); the second
    call updates its state in place (S_final is S0)."""
    w = recipe(mode, "bf16", B=2, H=2, L=448, d=128, s0_std=0.2, seed=17)
    log(f"carry {w}")
    x = workloads.make_inputs(w)
    d = to_cuda(x)
    o_ref, S_ref = oracle_fwd(x, mode)
    L1 = 192
    part = lambda t, a, b: t[:, :, a:b].contiguous()   # noqa: E731
    S = d["S0"].clone()
    o1, _ = la.chunk_fwd(part(d["q"], 0, L1), part(d["k"], 0, L1), part(d["v"], 0, L1),
                         part(d["log_alpha"], 0, L1), part(d["beta"], 0, L1), S, mode=mode,
                         S_final=S)
    o2, _ = la.chunk_fwd(part(d["q"], L1, w.L), part(d["k"], L1, w.L), part(d["v"], L1, w.L),
                         part(d["log_alpha"], L1, w.L), part(d["beta"], L1, w.L), S,
                         mode=mode, S_final=S)
    S32 = d["S0"].clone()
    o1f, _ = la.chunk_fwd(part(d["q"], 0, L1), part(d["k"], 0, L1), part(d["v"], 0, L1),
                          part(d["log_alpha"], 0, L1), part(d["beta"], 0, L1), S32, mode=mode,
                          S_final=S32, out_dtype=torch.float32)
    o2f, _ = la.chunk_fwd(part(d["q"], L1, w.L), part(d["k"], L1, w.L), part(d["v"], L1, w.L),
                          part(d["log_alpha"], L1, w.L), part(d["beta"], L1, w.L), S32,
                          mode=mode, S_final=S32, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_out_pair("o", torch.cat([o1, o2], dim=2), torch.cat([o1f, o2f], dim=2), o_ref)
    assert_close("S_final", f64(S), S_ref, "bf16")
    assert torch.equal(S32, S)


@pytest.mark.parametrize("mode", MODES)
def test_decode_steps_match_chunk_forward(mode):
    """L decode steps and one chunkwise forward over the same L tokens reach
    the same outputs and state (train with the chunk form, infer with the
    recurrent one)."""
    w = recipe(mode, "f32", B=2, H=2, L=128, d=64, s0_std=0.3, seed=23)
    log(f"decode vs chunk {w}")
    x = workloads.make_inputs(w)
    d = to_cuda(x)
    out, S_chunk = la.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"],
                                mode=mode)
    S = d["S0"].clone()
    outs = [la.decode_step(d["q"][:, :, t].contiguous(), d["k"][:, :, t].contiguous(),
                           d["v"][:, :, t].contiguous(), d["log_alpha"][:, :, t].contiguous(),
                           d["beta"][:, :, t].contiguous(), S, mode=mode)
            for t in range(w.L)]
    torch.cuda.synchronize()
    o_dec = np.stack([f64(o) for o in outs], axis=2)
    assert_close("decode vs chunk o", o_dec, f64(out), "f32")
    assert_close("decode vs chunk S", f64(S), f64(S_chunk), "f32")


def test_deterministic():
    """No atomics and a fixed reduction order: repeated calls are bitwise equal."""
    w = recipe("gated_delta", "bf16", B=2, H=4, L=256, d=128, s0_std=0.1, seed=29)
    log(f"determinism {w}")
    x = workloads.make_inputs(w)
    a_o, a_S = run_chunk(w, x)
    b_o, b_S = run_chunk(w, x)
    assert torch.equal(a_o, b_o) and torch.equal(a_S, b_S)


def test_gate_edge_cases():
    """beta = 0: nothing is written or erased, o_t = gamma_t S0^T q_t.
    alpha -> 0 (log_alpha = -1e4): history is dropped, o_t = beta_t (q_t . k_t) v_t."""
    w = recipe("gated_delta", "f32", B=1, H=2, L=192, d=64, s0_std=0.5, seed=31)
    log(f"gate edges {w}")
    x = workloads.make_inputs(w)
    x0 = dict(x, beta=torch.zeros_like(x["beta"]))
    out, S = run_chunk(w, x0)
    o_ref, S_ref = oracle_fwd(x0, "gated_delta")
    assert_close("beta=0 o", f64(out), o_ref, "f32")
    assert_close("beta=0 S", f64(S), S_ref, "f32")
    x1 = dict(x, log_alpha=torch.full_like(x["log_alpha"], -1e4))
    out, S = run_chunk(w, x1)
    o_ref, S_ref = oracle_fwd(x1, "gated_delta")
    assert_close("alpha->0 o", f64(out), o_ref, "f32")
    assert_close("alpha->0 S", f64(S), S_ref, "f32")


def test_errors_surface_as_exceptions():
    """A library error code comes back as an exception naming it: an empty
    sequence (L = 0) is a shape error, a head size outside the built set an
    unsupported one; nothing is launched."""
    w = recipe("delta", "bf16", B=1, H=1, L=64, d=128)
    x = to_cuda(workloads.make_inputs(w))
    e = {n: t[:, :, :0] for n, t in x.items() if n != "S0"}
    with pytest.raises(la.LAError, match="LA_ERR_SHAPE"):
        la.chunk_fwd(e["q"], e["k"], e["v"], e["log_alpha"], e["beta"], None, mode="delta")
    n = {n: t[..., :96].contiguous() for n, t in x.items() if n in ("q", "k", "v")}
    with pytest.raises(la.LAError, match="LA_ERR_UNSUPPORTED"):
        la.chunk_fwd(n["q"], n["k"], n["v"], x["log_alpha"], x["beta"], None, mode="delta")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", MODES)
def test_outputs_fully_written(mode, dtype, d):
    """out and S_final are pre-filled with NaN: every element must be
    written by the kernel (a skipped row or column tile stays NaN).  B * H
    = 8 exercises the head-to-XCD block numbering.  The workspace is passed
    explicitly, pre-filled with NaN."""
    w = recipe(mode, dtype, B=2, H=4, L=192, d=d, s0_std=0.2, seed=37)
    log(f"outputs fully written {w}")
    x = workloads.make_inputs(w)
    o_ref, S_ref = oracle_fwd(x, mode)
    dev = to_cuda(x)
    out = torch.full((w.B, w.H, w.L, w.dv), float("nan"), dtype=w.torch_dtype, device="cuda")
    S = torch.full((w.B, w.H, w.dk, w.dv), float("nan"), dtype=torch.float32, device="cuda")
    # the workspace too starts as all-ones bytes (NaN in bf16 and float):
    # nothing may be read from it before the call writes it
    nws = la.chunk_workspace_bytes(w.B, w.H, w.L, w.dk, w.dv, mode=mode,
                                   dtype=w.torch_dtype)
    ws = torch.full((max(nws, 1),), 255, dtype=torch.uint8, device="cuda")
    la.chunk_fwd(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], dev["S0"],
                 mode=mode, out=out, S_final=S, workspace=ws)
    torch.cuda.synchronize()
    assert_close("o", f64(out), o_ref, dtype, bf16_out=dtype == "bf16")
    assert_close("S_final", f64(S), S_ref, dtype)
