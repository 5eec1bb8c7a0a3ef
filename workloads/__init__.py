"""Seeded synthetic workloads shared by the tests, the bench and the smoke check.

This module only draws random numbers and prepares the op's inputs (the
normalisation and gate activations that sit in front of the op); it holds
none of the method's arithmetic, and it imports neither the oracle nor the
GPU library.  Both sides of every parity check receive the very tensors made
here (the oracle as float64 copies of the device-dtype values).

Recipe (all draws on the CPU in float32 from ``torch.Generator`` seeded with
``1000 + id`` for a named workload, in the fixed order q, k, v, beta_raw,
alpha_raw, S0):

* q, k, v ~ N(0, 1), times ``qkv_scale``; q and k L2-normalised per
  (batch, head, token) when ``qk_norm`` (the delta rule needs unit keys for
  exact replacement; the pages' gated form assumes them);
* beta = sigmoid(beta_raw), beta_raw ~ N(0, 1) -- a write strength in (0, 1)
  produced by an activation, as for the delta rule's learning-rate network
  in the hybrid-attention notes (section on Fast Weight Programmers);
* log_alpha = -softplus(alpha_raw) / 16, alpha_raw ~ N(0, 1) -- so
  alpha = exp(log_alpha) in (0, 1), mean about 0.95;
* S0 ~ N(0, s0_std) with standard deviation ``s0_std`` (zero state when 0);
* q, k, v are then cast to the device dtype (round to nearest even); gates
  and states stay float32.

Decode workloads draw q, k, v as ``[steps, B, H, d]`` and the gates as
``[steps, B, H]``.
"""

import math
from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    mode: str            # "linear" | "delta" | "gated_delta" | "gated_linear"
    dtype: str           # "f32" | "bf16": dtype of q, k, v and the output
    B: int
    H: int
    L: int               # sequence length (forward) -- 1 for decode
    dk: int
    dv: int
    C: int               # chunk size (forward); unused for decode
    qk_norm: bool
    qkv_scale: float
    s0_std: float
    steps: int = 0       # > 0 marks a decode workload: this many steps
    seed: int = 0

    @property
    def is_decode(self):
        return self.steps > 0

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def scaled(self, **kw):
        """The same recipe at other sizes (for reduced parity cases)."""
        return replace(self, **kw)


# The five workloads of the method's forward and decode paths.
WORKLOADS = {
    1: Workload("gated_delta_f32_b1h2l256d64", "gated_delta", "f32",
                B=1, H=2, L=256, dk=64, dv=64, C=64, qk_norm=True,
                qkv_scale=1.0, s0_std=0.0, seed=1001),
    2: Workload("linear_bf16_b8h16l4096d128", "linear", "bf16",
                B=8, H=16, L=4096, dk=128, dv=128, C=64, qk_norm=False,
                qkv_scale=1.0 / math.sqrt(128.0), s0_std=0.0, seed=1002),
    3: Workload("delta_bf16_b4h16l8192d128", "delta", "bf16",
                B=4, H=16, L=8192, dk=128, dv=128, C=64, qk_norm=True,
                qkv_scale=1.0, s0_std=0.0, seed=1003),
    4: Workload("gated_delta_bf16_b1h32l65536d128", "gated_delta", "bf16",
                B=1, H=32, L=65536, dk=128, dv=128, C=64, qk_norm=True,
                qkv_scale=1.0, s0_std=0.02, seed=1004),
    5: Workload("decode_gated_delta_b256h32d128x128", "gated_delta", "bf16",
                B=256, H=32, L=1, dk=128, dv=128, C=1, qk_norm=True,
                qkv_scale=1.0, s0_std=0.02, steps=128, seed=1005),
}


def head_shard(w, n):
    """One GPU's share of forward workload ``w`` when its heads are split
    over ``n`` GPUs: the same recipe with H / n heads (its own seed)."""
    if n < 1 or w.H % n:
        raise ValueError(f"{w.name}: {w.H} heads do not split over {n} GPUs")
    if n == 1:
        return w
    return replace(w, name=w.name.replace(f"h{w.H}", f"h{w.H // n}"), H=w.H // n,
                   seed=w.seed + 2)


# One GPU's share of workload 4 when its 32 heads are split over 8 GPUs:
# few (b, h) sequences, each long -- the shape the sequence-parallel forward
# is for.
WORKLOAD4_SHARD8 = head_shard(WORKLOADS[4], 8)


def _normal(gen, shape):
    return torch.randn(shape, generator=gen, dtype=torch.float32)


def _l2norm(x):
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


def make_raw_inputs(w: Workload, seed=None):
    """The draws of ``make_inputs`` before the preparation in front of the
    op: q, k, v times ``qkv_scale`` (q and k not normalised) in the device
    dtype, the raw gate scores ``a_raw`` (alpha) and ``b_raw`` (beta)
    float32, and S0 -- the inputs of the fused entry points."""
    gen = torch.Generator("cpu")
    gen.manual_seed(w.seed if seed is None else seed)
    lead = (w.steps, w.B, w.H) if w.is_decode else (w.B, w.H, w.L)
    q = _normal(gen, lead + (w.dk,)) * w.qkv_scale
    k = _normal(gen, lead + (w.dk,)) * w.qkv_scale
    v = _normal(gen, lead + (w.dv,)) * w.qkv_scale
    beta_raw = _normal(gen, lead)
    alpha_raw = _normal(gen, lead)
    if w.s0_std > 0:
        S0 = _normal(gen, (w.B, w.H, w.dk, w.dv)) * w.s0_std
    else:
        S0 = torch.zeros((w.B, w.H, w.dk, w.dv), dtype=torch.float32)
    dt = w.torch_dtype
    return dict(q=q.to(dt).contiguous(), k=k.to(dt).contiguous(), v=v.to(dt).contiguous(),
                a_raw=alpha_raw.contiguous(), b_raw=beta_raw.contiguous(), S0=S0.contiguous())


def make_inputs(w: Workload, seed=None):
    """Draw the inputs of workload ``w`` on the CPU.

    Returns a dict of CPU tensors: ``q, k, v`` in the device dtype,
    ``log_alpha, beta`` float32, ``S0`` float32 (zeros when ``s0_std == 0``).
    Forward shapes: q, k ``[B, H, L, dk]``, v ``[B, H, L, dv]``, gates
    ``[B, H, L]``.  Decode shapes: q, k ``[steps, B, H, dk]``, v
    ``[steps, B, H, dv]``, gates ``[steps, B, H]``.  S0 is always
    ``[B, H, dk, dv]``.
    """
    gen = torch.Generator("cpu")
    gen.manual_seed(w.seed if seed is None else seed)
    if w.is_decode:
        lead = (w.steps, w.B, w.H)
    else:
        lead = (w.B, w.H, w.L)
    q = _normal(gen, lead + (w.dk,)) * w.qkv_scale
    k = _normal(gen, lead + (w.dk,)) * w.qkv_scale
    v = _normal(gen, lead + (w.dv,)) * w.qkv_scale
    beta_raw = _normal(gen, lead)
    alpha_raw = _normal(gen, lead)
    if w.s0_std > 0:
        S0 = _normal(gen, (w.B, w.H, w.dk, w.dv)) * w.s0_std
    else:
        S0 = torch.zeros((w.B, w.H, w.dk, w.dv), dtype=torch.float32)
    if w.qk_norm:
        q = _l2norm(q)
        k = _l2norm(k)
    beta = torch.sigmoid(beta_raw)
    log_alpha = -torch.nn.functional.softplus(alpha_raw) / 16.0
    dt = w.torch_dtype
    return dict(q=q.to(dt).contiguous(), k=k.to(dt).contiguous(),
                v=v.to(dt).contiguous(), log_alpha=log_alpha.contiguous(),
                beta=beta.contiguous(), S0=S0.contiguous())


def to_f64(inputs):
    """float64 NumPy copies of exactly the values handed to the device."""
    return {key: t.to(torch.float64).numpy() for key, t in inputs.items()}


def make_upstream_grads(w: Workload, seed=None, ds_std=1.0):
    """Upstream gradients for a backward of workload ``w``: ``dout`` drawn
    N(0, 1) in the device dtype with the output's shape ``[B, H, L, dv]``,
    and ``dS_final`` N(0, ds_std^2) float32 ``[B, H, dk, dv]`` (zeros when
    ds_std == 0).  Seeded on its own (default: the workload's seed + 7919),
    so the forward inputs are unchanged."""
    gen = torch.Generator("cpu")
    gen.manual_seed((w.seed + 7919) if seed is None else seed)
    dout = _normal(gen, (w.B, w.H, w.L, w.dv))
    dS = _normal(gen, (w.B, w.H, w.dk, w.dv)) * ds_std if ds_std > 0 else \
        torch.zeros((w.B, w.H, w.dk, w.dv), dtype=torch.float32)
    return dict(dout=dout.to(w.torch_dtype).contiguous(), dS_final=dS.contiguous())
