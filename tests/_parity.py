"""Shared helpers of the GPU parity tests: tolerances and oracle runs.

Tolerances (written into every comparison):

* float32 inputs: max |err| / max |ref| <= 1e-4, for the outputs and,
  separately, the final states;
* bfloat16 inputs (float32 accumulation and state): max |err| <= 2e-2 *
  RMS(ref), for the outputs and, separately, the final states;
* bfloat16 outputs additionally carry their own rounding: an exact result
  rounded to bfloat16 is off by up to half an ulp, at most 2^-8 |ref|, which
  on the full-size workloads alone exceeds 2e-2 * RMS(ref) (the largest
  outputs are 6-9 RMS).  A bf16 output therefore passes when every element
  satisfies |err| <= 2e-2 * RMS(ref) * (1 + 2^-8) + 2^-8 |ref|; the same
  kernels with a float32 output are held to the plain bound.

The oracle always consumes float64 copies of exactly the tensors handed to
the GPU (after bfloat16 rounding).
"""
import sys

import numpy as np
import torch

import oracle
import workloads

F32_REL = 1e-4
BF16_RMS = 2e-2


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bound(ref, dtype):
    ref = np.asarray(ref, dtype=np.float64)
    if dtype == "f32":
        return F32_REL * float(np.max(np.abs(ref)))
    return BF16_RMS * float(np.sqrt(np.mean(ref * ref)))


BF16_HALF_ULP = 2.0 ** -8


def assert_close(name, got, ref, dtype, bf16_out=False):
    """Compare against the oracle under the tolerance of `dtype` (the input
    dtype); `bf16_out` adds the output's own rounding per element."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    diff = np.abs(got - ref)
    err = float(np.max(diff))
    b = bound(ref, dtype)
    if not bf16_out:
        log(f"  {name}: max|err| {err:.3e}  bound {b:.3e}  ({err / b if b else 0:.3f} of bound)")
        assert err <= b, f"{name}: max|err| {err:.3e} exceeds bound {b:.3e}"
        return err / b if b else 0.0
    excess = float(np.max(diff - BF16_HALF_ULP * np.abs(ref)))
    bb = b * (1.0 + BF16_HALF_ULP)
    log(f"  {name} (bf16 out): max|err| {err:.3e} ({err / b:.3f} of plain bound); "
        f"beyond output rounding {excess:.3e} ({excess / bb:.3f} of bound)")
    assert excess <= bb, (f"{name}: error beyond the bf16 output rounding {excess:.3e} "
                          f"exceeds {bb:.3e}")
    return excess / bb


def to_cuda(x):
    return {k: t.cuda() for k, t in x.items()}


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def oracle_fwd(x, mode, heads=None):
    """Oracle forward on all heads, or on a list of (b, h) pairs."""
    y = workloads.to_f64(x)
    s0 = y["S0"]
    if heads is None:
        return oracle.recurrent_fwd(y["q"], y["k"], y["v"], y["log_alpha"], y["beta"],
                                    s0, mode)
    bs = [b for b, _ in heads]
    hs = [h for _, h in heads]
    sel = lambda a: a[bs, hs][None]          # noqa: E731  -> [1, n, ...]
    o, S = oracle.recurrent_fwd(sel(y["q"]), sel(y["k"]), sel(y["v"]),
                                sel(y["log_alpha"]), sel(y["beta"]), sel(s0), mode)
    return o[0], S[0]


def oracle_decode(x, mode, heads=None):
    """Oracle decode run over all steps, on all or on sampled (b, h) pairs."""
    y = workloads.to_f64(x)
    if heads is None:
        return oracle.decode_steps(y["S0"], y["q"], y["k"], y["v"], y["log_alpha"],
                                   y["beta"], mode)
    bs = [b for b, _ in heads]
    hs = [h for _, h in heads]
    o, S = oracle.decode_steps(y["S0"][bs, hs][None], y["q"][:, bs, hs][:, None],
                               y["k"][:, bs, hs][:, None], y["v"][:, bs, hs][:, None],
                               y["log_alpha"][:, bs, hs][:, None],
                               y["beta"][:, bs, hs][:, None], mode)
    return o[:, 0], S[0]


def assert_out_pair(name, out_bf16, out_f32, ref, dtype="bf16", rounded=True):
    """The same call with a bfloat16 and a float32 output: the float output
    is held to the plain bound of `dtype` and, when `rounded`, the bf16
    output must be exactly the float one rounded to nearest even -- the
    pairing that justifies the bf16 output's looser per-element bound (the
    bf16 output is also checked under that bound)."""
    import torch
    assert_close(f"{name} (f32 out)", f64(out_f32), ref, dtype)
    assert_close(name, f64(out_bf16), ref, dtype, bf16_out=True)
    if rounded:
        assert torch.equal(out_f32.to(torch.bfloat16), out_bf16), (
            f"{name}: bf16 out != rne(f32 out)")
