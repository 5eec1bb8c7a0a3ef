#!/usr/bin/env python3
"""Benchmark of the chunkwise gated-delta forward and the decode step on one GPU.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

One JSON line on stdout.  A "step" is one call of the chunkwise forward
(la_chunk_fwd) over the long-context gated-delta workload
(B=1, H=32, L=65536, d=128, C=64, bf16 q/k/v/out, float32 gates and state,
nonzero initial state); ``value`` is its throughput in tokens/s with the
inputs already resident in HBM.  The same line carries the decode half of
the metric (128 in-place decode steps over B=256, H=32, d=128 float32
states: state GB/s and fraction of HBM peak), the per-kernel HIP-event
timings, the roofline of the forward's dominant kernel and the float64 CPU
oracle timed on a bounded sample of the same forward workload.

Inputs are seeded synthetic tensors from ``workloads`` (the recipe is in
that module's docstring); two copies of the forward inputs alternate so
consecutive steps do not hit the 256 MB last-level cache.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("chunkwise gated-delta fwd tokens/s (% MFMA peak); "
          "decode state GB/s (% HBM)")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK = 2.5e15        # MI355X dense bf16 MFMA, flop/s
FP32_MFMA_PEAK = 157.3e12      # MI355X dense fp32 matrix, flop/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "chunkwise_gated_delta_la_amd", "csrc")
# Source files each kernel is built from: a traffic measurement is used
# only while these are unchanged.
KERNEL_SOURCES = {
    "la_chunk": ["la_chunk.hip", "la_chunk_pipe.hip", "la_device.hpp", "la_index.hpp",
                 "la_kernels.hpp"],
    "la_tsolve": ["la_chunk_pipe.hip", "la_device.hpp", "la_index.hpp", "la_kernels.hpp"],
    "la_decode": ["la_decode.hip", "la_device.hpp", "la_kernels.hpp"],
}
for _k in ("la_bwd_prep", "la_bwd_states", "la_bwd_rev", "la_bwd_grads"):
    KERNEL_SOURCES[_k] = ["la_bwd.hip", "la_bwd.hpp", "la_device.hpp", "la_kernels.hpp"]
# rocprofv3 kernel names -> library kernel names (chunk_kernel: float
# inputs, chunk_pipe_kernel: bf16 inputs)
KERNEL_SYMBOLS = {"chunk_kernel": "la_chunk", "chunk_pipe_kernel": "la_chunk",
                  "t_solve_kernel": "la_tsolve", "decode_kernel": "la_decode",
                  "bwd_prep_kernel": "la_bwd_prep", "bwd_states_kernel": "la_bwd_states",
                  "bwd_rev_kernel": "la_bwd_rev",
                  "bwd_grads_kernel": "la_bwd_grads"}
T_BYTES_PER_CHUNK = 6 * 1024   # T operand fragments of one (b, h, chunk)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ work model
# Per (token, head) of the forward, d = dk = dv, chunk C, element size e:
#   algorithmic work of the method (dense-block chunkwise):
#     gated/delta: 10 C d + 6 d^2 flop;  linear: 4 C d + 4 d^2
#   la_chunk (the chain kernel) moves q, k, v in and o out (4 d e), plus
#            beta (delta modes) and log_alpha (gated) at 4 B each, plus,
#            for bf16 inputs in the delta modes, the chunk's T factor
#            (6 KiB per chunk: 96 B per token); per (b, h): S0 in (when
#            given) and S_final out at dk dv 4 B
#   la_tsolve (bf16 delta modes) reads k and the gates and writes T
# Per (b, h) state of one decode step: S in and out (2 dk dv 4 B), q, k, v,
# o (2 dk e + 2 dv e), two float gates.

ERASE_MODES = ("delta", "gated_delta")           # beta and the T factor
GATE_BYTES = {"linear": 0, "delta": 4, "gated_delta": 8, "gated_linear": 4}


def fwd_flops_per_token_head(w, exact=False):
    """Dense-block chunkwise flops per (token, head): the C x C products
    (Q K^T, its product with the values, and in the delta modes K K^T, W and
    U) counted in full; `exact` counts their causal triangle only (half)."""
    d, C = w.dk, w.C
    f = 1 if exact else 2
    if w.mode not in ERASE_MODES:
        return f * C * d + 4 * d * d
    return 5 * f * C * d + 6 * d * d


def op_bytes(w):
    """Algorithmic HBM bytes of one forward call: q, k, v read and o written
    once, the gates the mode reads, S0 (when given) read and S_final
    written once per (b, h).  No intermediate of the design (the T records)
    is counted."""
    return (fwd_min_bytes_per_token_head(w) * w.B * w.H * w.L
            + kernel_bytes_per_head("la_chunk", w) * w.B * w.H)


def t_bytes_per_token_head(w):
    """Bytes of the T factor per (token, head): written by la_tsolve, read
    by la_chunk (bf16 inputs in the delta modes only)."""
    return T_BYTES_PER_CHUNK // w.C if (w.dtype == "bf16" and w.mode in ERASE_MODES) else 0


def kernel_bytes_per_token_head(name, w, P=1):
    """Algorithmic HBM bytes per (token, head) of a forward kernel: the
    chain kernel reads q, k, v, the gates the mode uses and T once and
    writes o once (initial and final states are added per head); the T
    solve reads k and the gates and writes T.  With P > 1 segments the
    state pass reads k, v, the gates and T of the first P - 1 segments and,
    in the delta modes, k, the gates and T again for the P - 2 transitions;
    the scan touches states only."""
    e = 2 if w.dtype == "bf16" else 4
    gates = GATE_BYTES[w.mode]
    t = t_bytes_per_token_head(w)
    if name == "la_chunk":
        return fwd_min_bytes_per_token_head(w) + t
    if name == "la_tsolve":
        return w.dk * e + gates + t
    if name == "la_chunk_state":
        s_part = (w.dk + w.dv) * e + gates + t
        m_part = (w.dk * e + gates + t) if w.mode in ERASE_MODES else 0
        return ((P - 1) * s_part + max(P - 2, 0) * m_part) / P
    if name == "la_seg_scan":
        return 0
    raise KeyError(name)


def kernel_bytes_per_head(name, w, P=1):
    """Per-head state bytes of a forward call.  Whole walk: S0 read (if
    given), S_final written by the chain kernel.  P > 1 segments: the state
    pass reads S0 and writes X (P - 1) and M (P - 2, delta modes); the scan
    reads S0, X and M and writes S_in (P); the output pass reads S_in and
    writes S_final."""
    st = w.dk * w.dv * 4
    erase = w.mode in ERASE_MODES
    s0 = 1 if w.s0_std > 0 else 0
    if name == "la_tsolve":
        return 0
    if name == "la_chunk":
        return (s0 + 1) * st if P == 1 else (P + 1) * st
    if name == "la_chunk_state":
        return (s0 + (P - 1) + (P - 2 if erase else 0)) * st
    if name == "la_seg_scan":
        return (s0 + (P - 1) + (P - 2 if erase else 0) + P) * st
    raise KeyError(name)


def decode_bytes_per_head(w):
    e = 2 if w.dtype == "bf16" else 4
    return 2 * w.dk * w.dv * 4 + 2 * w.dk * e + 2 * w.dv * e + 8


def fwd_min_bytes_per_token_head(w):
    """q, k, v, o and the gates the mode reads: what the op must move."""
    e = 2 if w.dtype == "bf16" else 4
    gates = GATE_BYTES[w.mode]
    return (2 * w.dk + 2 * w.dv) * e + gates


# ------------------------------------------------------------------ HBM traffic

def source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the rocprofv3
    FETCH_SIZE / WRITE_SIZE runs recorded in profiles/traffic.json, scaled
    by the copy-kernel calibration; None when absent or when the kernel's
    sources have changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    ent = rec.get("kernels", {}).get(kernel)
    if not ent or ent.get("workload") != workload or ent.get("source_hash") != source_hash(kernel):
        return None
    return ent["hbm_bytes_per_launch"]


def calibrate_copy(mib, reps=5):
    """A plain device-to-device copy of `mib` MiB, `reps` times: the
    reference kernel whose FETCH_SIZE / WRITE_SIZE counters calibrate the
    traffic figures (it reads and writes exactly `mib` MiB per launch)."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.empty(n, dtype=torch.float32, device="cuda").normal_()
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": n * 4, "reps": reps}), flush=True)


def _read_pmc(csv_dir, counter):
    """{kernel: [per-dispatch counter value]} from rocprofv3 counter CSVs."""
    import csv
    import glob
    out = {}
    for path in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != counter:
                    continue
                name = row["Kernel_Name"]
                out.setdefault(name, []).append(float(row["Counter_Value"]))
    return out


def ingest_pmc(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, workload, command):
    """Turn four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE of the
    bench and of the copy calibration) into profiles/traffic.json."""
    def copy_factor(d, counter):
        vals = [v for k, vs in _read_pmc(d, counter).items() if "copy" in k.lower() for v in vs]
        if not vals:
            raise SystemExit(f"no copy kernel in {d}")
        kib = sorted(vals)[len(vals) // 2]          # median dispatch
        return kib * 1024.0, (1 << 30)              # counted bytes, true bytes
    cf, tf = copy_factor(cal_fetch_dir, "FETCH_SIZE")
    cw, tw = copy_factor(cal_write_dir, "WRITE_SIZE")
    sf, sw = tf / cf, tw / cw
    fetch, write = _read_pmc(fetch_dir, "FETCH_SIZE"), _read_pmc(write_dir, "WRITE_SIZE")
    kernels = {}
    for sym, lib_name in KERNEL_SYMBOLS.items():
        fv = [v for k, vs in fetch.items() if sym in k for v in vs]
        wv = [v for k, vs in write.items() if sym in k for v in vs]
        if not fv or not wv or lib_name not in workload:
            continue
        f_b = sorted(fv)[len(fv) // 2] * 1024.0 * sf
        w_b = sorted(wv)[len(wv) // 2] * 1024.0 * sw
        kernels[lib_name] = {
            "workload": workload[lib_name], "source_hash": source_hash(lib_name),
            "fetch_bytes_per_launch": round(f_b), "write_bytes_per_launch": round(w_b),
            "hbm_bytes_per_launch": round(f_b + w_b), "dispatches": len(fv),
            "command": command}
    # kernels not in these runs keep their earlier records
    try:
        with open(TRAFFIC_FILE) as fh:
            old = json.load(fh).get("kernels", {})
    except (OSError, ValueError):
        old = {}
    old.update(kernels)
    rec = {"calibration": {"copy_bytes": 1 << 30, "fetch_scale": sf, "write_scale": sw},
           "kernels": old}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))


# ------------------------------------------------------------------ legs

def bench_forward(w, steps, warmup, x=None):
    import torch

    import chunkwise_gated_delta_la_amd as la
    import workloads

    if x is None:
        log(f"[bench] forward workload {w.name}: generating inputs")
        x = workloads.make_inputs(w)
    copies = []
    for _ in range(2):
        copies.append({k: t.cuda() for k, t in x.items()})
    out = torch.empty((w.B, w.H, w.L, w.dv), dtype=w.torch_dtype, device="cuda")
    S_final = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    ws_bytes = la.chunk_workspace_bytes(w.B, w.H, w.L, w.dk, w.dv, mode=w.mode, C=w.C,
                                        dtype=w.torch_dtype)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def step(i):
        d = copies[i % 2]
        la.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                     d["S0"] if w.s0_std > 0 else None, mode=w.mode, C=w.C,
                     out=out, S_final=S_final, workspace=ws)

    log(f"[bench] forward: {warmup} warmup steps")
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] forward: {steps} timed steps")
    with la.kernel_timer() as kt:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    sec = (t1 - t0) / steps
    token_heads = w.B * w.H * w.L
    P = la.chunk_segments(w.B, w.H, w.L, w.dk, w.dv, mode=w.mode, C=w.C, dtype=w.torch_dtype)
    kernels = _kernel_table(kt.stats, w, token_heads, w.B * w.H, P)
    dom = max(kernels, key=lambda k: kernels[k]["avg_ms"])
    flops = fwd_flops_per_token_head(w) * token_heads
    flops_exact = fwd_flops_per_token_head(w, exact=True) * token_heads
    min_bytes = op_bytes(w)
    dom_s = kernels[dom]["avg_ms"] * 1e-3
    if w.dtype == "f32":
        # float32 matrix work, arithmetic intensity above the fp32 ridge
        ach = flops / dom_s / 1e12
        roofline = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 3),
                    "peak": FP32_MFMA_PEAK / 1e12, "unit": "TFLOP/s",
                    "frac": round(ach * 1e12 / FP32_MFMA_PEAK, 5), "traffic": None,
                    "algorithmic_flops": flops}
    else:
        # the op's own bytes over the chain kernel's time; the T records the
        # design keeps between its two kernels are reported beside them
        ach = min_bytes / dom_s / 1e9
        roofline = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic(dom, w.name), "algorithmic_bytes": min_bytes,
                    "bytes_basis": "q, k, v, o, gates, S0, S_final once each",
                    "t_record_bytes": t_bytes_per_token_head(w) * token_heads}
    peak = FP32_MFMA_PEAK if w.dtype == "f32" else BF16_MFMA_PEAK
    res = {
        "value": w.B * w.L / sec,
        "ms_per_step": sec * 1e3,
        "segments": P,
        "mfma_frac_of_bf16_peak": flops / sec / BF16_MFMA_PEAK,
        "mfma_frac": flops / sec / peak,
        "mfma_frac_exact": flops_exact / sec / peak,
        "mfma_peak": peak,
        "hbm_frac_of_min_bytes": min_bytes / sec / (HBM_PEAK_GBS * 1e9),
        "kernels": kernels,
        "roofline": roofline,
    }
    del copies
    torch.cuda.empty_cache()
    return x, res


def _kernel_table(stats, w, token_heads, heads, P=1):
    kernels = {}
    for name, (n, ms) in stats.items():
        avg_ms = ms / max(n, 1)
        by = round(kernel_bytes_per_token_head(name, w, P) * token_heads
                   + kernel_bytes_per_head(name, w, P) * heads)
        kernels[name] = {"launches": n, "avg_ms": round(avg_ms, 5),
                         "algorithmic_bytes": by,
                         "achieved_GBs": round(by / (avg_ms * 1e-3) / 1e9, 1),
                         "hbm_frac": round(by / (avg_ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4)}
    return kernels


def bench_config(w, steps, warmup, cpu=None):
    """One of the forward configurations at its own sizes: tokens/s, the
    fraction of the MFMA peak of its dtype (dense-block and triangle-exact
    flop counts), the fraction of HBM peak of its algorithmic bytes, the
    dominant kernel's roofline, and the CPU oracle measured beside it."""
    _, res = bench_forward(w, steps, warmup)
    return {"workload": w.name, "mode": w.mode, "dtype": w.dtype,
            "tokens_per_s": round(res["value"], 1),
            "ms_per_step": round(res["ms_per_step"], 5),
            "mfma_peak_flops": res["mfma_peak"],
            "mfma_frac": round(res["mfma_frac"], 5),
            "mfma_frac_exact": round(res["mfma_frac_exact"], 5),
            "hbm_frac_of_min_bytes": round(res["hbm_frac_of_min_bytes"], 4),
            "roofline": res["roofline"], "kernels": res["kernels"], "cpu_baseline": cpu}


def bench_mode(w, steps, warmup):
    """Another mode at a forward workload's sizes (extra measurement)."""
    _, res = bench_forward(w, steps, warmup)
    return {"workload": w.name, "mode": w.mode, "tokens_per_s": round(res["value"], 1),
            "ms_per_step": round(res["ms_per_step"], 4),
            "mfma_frac_of_bf16_peak": round(res["mfma_frac_of_bf16_peak"], 4),
            "hbm_frac_of_min_bytes": round(res["hbm_frac_of_min_bytes"], 4),
            "kernels": res["kernels"]}


def bench_segments(w, steps, warmup):
    """Few long sequences (one GPU's share of a head-sharded workload): the
    whole-sequence walk (segments = 1) against the sequence-parallel
    forward with la_chunk_fwd's own segment plan, tokens/s of each."""
    import torch

    import chunkwise_gated_delta_la_amd as la
    import workloads

    P = la.chunk_segments(w.B, w.H, w.L, w.dk, w.dv, mode=w.mode, C=w.C, dtype=w.torch_dtype)
    log(f"[bench] segments {w.name} (plan P={P}): generating inputs")
    x = workloads.make_inputs(w)
    copies = [{k: t.cuda() for k, t in x.items()} for _ in range(2)]
    out = torch.empty((w.B, w.H, w.L, w.dv), dtype=w.torch_dtype, device="cuda")
    S_final = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    res = {"workload": w.name, "mode": w.mode, "segments": P}
    for label, seg in (("whole", 1), ("segmented", P)):
        nws = la.chunk_workspace_bytes(w.B, w.H, w.L, w.dk, w.dv, mode=w.mode, C=w.C,
                                       dtype=w.torch_dtype, segments=seg)
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")

        def step(i):
            d = copies[i % 2]
            la.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                         d["S0"] if w.s0_std > 0 else None, mode=w.mode, C=w.C, out=out,
                         S_final=S_final, workspace=ws, segments=seg)

        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        with la.kernel_timer() as kt:
            t0 = time.perf_counter()
            for i in range(steps):
                step(i)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
        sec = (t1 - t0) / steps
        res[label] = {"P": seg, "tokens_per_s": round(w.B * w.L / sec, 1),
                      "ms_per_step": round(sec * 1e3, 4),
                      "kernels": {k: {"launches": n, "avg_ms": round(ms / max(n, 1), 5)}
                                  for k, (n, ms) in kt.stats.items()}}
        del ws
    res["speedup"] = round(res["segmented"]["tokens_per_s"] / res["whole"]["tokens_per_s"], 3)
    del copies, out
    torch.cuda.empty_cache()
    return res


def segment_sweep(base, steps, warmup, heads=(1, 2, 4, 8, 16),
                  counts=(1, 2, 3, 4, 6, 8, 12, 16, 24, 32)):
    """ms per forward of the sequence-parallel path at explicit segment
    counts against la_chunk_fwd's own plan, for a few head counts of one
    long-sequence workload (the evidence the plan's cost model is fitted
    to).  One JSON object: {H: {"plan": P, "ms": {P: ms}}}."""
    import torch

    import chunkwise_gated_delta_la_amd as la
    import workloads

    res = {}
    for H in heads:
        w = base.scaled(H=H, name=f"{base.name}_h{H}")
        nc = -(-w.L // w.C)
        plan = la.chunk_segments(w.B, w.H, w.L, w.dk, w.dv, mode=w.mode, C=w.C,
                                 dtype=w.torch_dtype)
        log(f"[bench] segment sweep H={H} (plan P={plan})")
        x = {k: t.cuda() for k, t in workloads.make_inputs(w).items()}
        out = torch.empty((w.B, w.H, w.L, w.dv), dtype=w.torch_dtype, device="cuda")
        S_final = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
        ms = {}
        for P in sorted({c for c in counts if c <= nc} | {plan}):
            def step():
                la.chunk_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"],
                             x["S0"] if w.s0_std > 0 else None, mode=w.mode, C=w.C, out=out,
                             S_final=S_final, segments=P)
            ms[P] = round(_timed(step, steps, warmup)[0], 4)
        res[H] = {"plan": plan, "ms": ms}
        del x, out, S_final
        torch.cuda.empty_cache()
    return res


def _timed(step, steps, warmup):
    """ms per call of step() (host clock around synchronised runs) and the
    library's per-kernel HIP-event times over the same calls."""
    import torch

    import chunkwise_gated_delta_la_amd as la
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    with la.kernel_timer() as kt:
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    kernels = {k: {"launches": n, "avg_ms": round(ms / max(n, 1), 5)}
               for k, (n, ms) in kt.stats.items()}
    return (t1 - t0) / steps * 1e3, kernels


def bench_fused(w, steps, warmup):
    """The forward from raw inputs with every step in front of and behind
    the op fused (q, k normalisation, gate activations, residual D v, output
    norm), against the same steps as separate torch operations around
    la_chunk_fwd (context: what the fusion saves)."""
    import torch

    import chunkwise_gated_delta_la_amd as la
    import workloads

    log(f"[bench] fused steps {w.name}: generating inputs")
    r = {k: t.cuda() for k, t in workloads.make_raw_inputs(w).items()}
    gen = torch.Generator("cpu").manual_seed(w.seed + 11)
    D = (torch.randn((w.H, w.dv), generator=gen) * 0.5).cuda()
    nw = (1.0 + 0.1 * torch.randn((w.H, w.dv), generator=gen)).cuda()
    out = torch.empty((w.B, w.H, w.L, w.dv), dtype=w.torch_dtype, device="cuda")
    S_final = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    scale = 1.0 / 16.0
    nws = la.chunk_workspace_bytes(w.B, w.H, w.L, w.dk, w.dv, mode=w.mode, dtype=w.torch_dtype,
                                   qk_l2norm=True, gate_act=True)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")

    def fused():
        la.chunk_fwd(r["q"], r["k"], r["v"], r["a_raw"], r["b_raw"], r["S0"], mode=w.mode,
                     out=out, S_final=S_final, workspace=ws, qk_l2norm=True, gate_act=True,
                     gate_scale=scale, dskip=D, out_norm=True, norm_weight=nw, norm_eps=1e-6)

    def unfused():
        qf, kf = r["q"].float(), r["k"].float()
        qn = (qf * torch.rsqrt((qf * qf).sum(-1, keepdim=True) + 1e-6)).to(w.torch_dtype)
        kn = (kf * torch.rsqrt((kf * kf).sum(-1, keepdim=True) + 1e-6)).to(w.torch_dtype)
        lg = -scale * torch.nn.functional.softplus(r["a_raw"])
        be = torch.sigmoid(r["b_raw"])
        o, _ = la.chunk_fwd(qn, kn, r["v"], lg, be, r["S0"], mode=w.mode, S_final=S_final,
                            out_dtype=torch.float32)
        o = o + D[None, :, None, :] * r["v"].float()
        o = o * torch.rsqrt((o * o).mean(-1, keepdim=True) + 1e-6) * nw[None, :, None, :]
        out.copy_(o)

    f_ms, f_k = _timed(fused, steps, warmup)
    u_ms, _ = _timed(unfused, steps, warmup)
    del ws
    torch.cuda.empty_cache()
    return {"workload": w.name, "steps_fused": "qk_l2norm, gate_act, dskip, out_norm",
            "ms_per_step": round(f_ms, 4), "tokens_per_s": round(w.B * w.L / f_ms * 1e3, 1),
            "kernels": f_k, "torch_composed_ms_per_step": round(u_ms, 4)}


def bench_noncausal(w, steps, warmup):
    """The bidirectional form O = Q (S0 + K^T V) at a forward workload's
    sizes: tokens/s and the fraction of HBM peak of its algorithmic bytes
    (q, k, v read and o written once, states per head)."""
    import torch

    import chunkwise_gated_delta_la_amd as la
    import workloads

    log(f"[bench] non-causal {w.name}: generating inputs")
    x = {k: t.cuda() for k, t in workloads.make_inputs(w).items()}
    out = torch.empty((w.B, w.H, w.L, w.dv), dtype=torch.bfloat16, device="cuda")
    S = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    s0 = x["S0"] if w.s0_std > 0 else None
    ms, kernels = _timed(lambda: la.noncausal_fwd(x["q"], x["k"], x["v"], s0, out=out,
                                                 S_final=S), steps, warmup)
    by = w.B * w.H * (w.L * (w.dk * 2 + w.dv * 2 * 2) + (2 if s0 is not None else 1) * w.dk
                      * w.dv * 4)
    del x, out
    torch.cuda.empty_cache()
    return {"workload": "noncausal_" + w.name, "ms_per_step": round(ms, 4),
            "tokens_per_s": round(w.B * w.L / ms * 1e3, 1), "algorithmic_bytes": by,
            "hbm_frac": round(by / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4), "kernels": kernels}


def bwd_flops_per_token_head(w):
    """Dense chunkwise backward flops per token-head as built (the forward
    walk recomputes U and the states): 12 C x C x d products per chunk in
    the delta modes (scores twice, K K^T twice, T R, P^T dO, T^T dU, dO U^T,
    dR U^T, E K, E^T Q, G K; 7 without erase) and 8 C x d x d (K S, K^T U,
    Q^T dO, K dS', K^T dR, dO S^T, dR S^T, U dS'^T; 5 without erase), plus
    the T solve, C^3 / 3 per chunk."""
    erase = w.mode in ("delta", "gated_delta")
    d, C = w.dk, w.C
    n_ccd = 12 if erase else 7
    n_cdd = 8 if erase else 5
    return n_ccd * 2 * C * d + n_cdd * 2 * d * d + (C * C / 3 if erase else 0)


def bench_backward(w, steps, warmup, cpu_tokens=0):
    """la_chunk_bwd at a forward workload's sizes (upstream gradients drawn
    N(0, 1), dS_final N(0, 0.02^2)): tokens/s, the per-kernel HIP-event
    times, the fraction of bf16 MFMA peak of the dense backward flops and of
    HBM peak of the minimal bytes (q, k, v, dO read and dq, dk, dv written
    as float32 once, gates and their gradients, states per head)."""
    import torch

    import chunkwise_gated_delta_la_amd as la
    import workloads

    log(f"[bench] backward {w.name}: generating inputs")
    xc = workloads.make_inputs(w)
    grc = workloads.make_upstream_grads(w, ds_std=0.02)
    x = {k: t.cuda() for k, t in xc.items()}
    gr = {k: t.cuda() for k, t in grc.items()}
    nws = la.chunk_bwd_workspace_bytes(w.B, w.H, w.L, w.dk, w.dv, mode=w.mode,
                                       dtype=w.torch_dtype)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    s0 = x["S0"] if w.s0_std > 0 else None
    ms, kernels = _timed(lambda: la.chunk_bwd(x["q"], x["k"], x["v"], x["log_alpha"],
                                              x["beta"], s0, gr["dout"], gr["dS_final"],
                                              mode=w.mode, workspace=ws), steps, warmup)
    th = w.B * w.H * w.L
    esz = 2 if w.dtype == "bf16" else 4
    by = th * (4 * w.dk * esz + 3 * w.dk * 4 + 4 * 4) + w.B * w.H * 3 * w.dk * w.dv * 4
    fl = th * bwd_flops_per_token_head(w)
    for name, k in kernels.items():
        kb = bwd_kernel_bytes(name, w)
        if kb:
            k["algorithmic_bytes"] = kb
            k["achieved_GBs"] = round(kb / (k["avg_ms"] * 1e-3) / 1e9, 1)
            k["hbm_frac"] = round(k["achieved_GBs"] / HBM_PEAK_GBS, 4)
    dom = max(kernels, key=lambda n: kernels[n]["avg_ms"] if n != "la_bwd_rev" and
              n != "la_bwd_states" else 0.0)
    roof = {"kernel": dom, "bound": "hbm", "achieved": kernels[dom].get("achieved_GBs"),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": kernels[dom].get("hbm_frac"),
            "traffic": measured_traffic(dom, "backward_" + w.name),
            "algorithmic_bytes": kernels[dom].get("algorithmic_bytes"),
            "note": "largest of the parallel kernels; the walks (la_bwd_states, la_bwd_rev) "
                    "are bound by their serial chunk chain"}
    del ws
    torch.cuda.empty_cache()
    cpu = None
    if cpu_tokens > 0:
        cpu = bwd_cpu_baseline(w, xc, grc, cpu_tokens)
    del x, gr
    torch.cuda.empty_cache()
    return {"workload": "backward_" + w.name, "mode": w.mode, "ms_per_step": round(ms, 4),
            "tokens_per_s": round(w.B * w.L / ms * 1e3, 1),
            "flops_per_token_head": bwd_flops_per_token_head(w),
            "mfma_frac_of_bf16_peak": round(fl / (ms * 1e-3) / BF16_MFMA_PEAK, 4),
            "min_bytes": by, "hbm_frac_of_min_bytes": round(by / (ms * 1e-3) /
                                                             (HBM_PEAK_GBS * 1e9), 4),
            "workspace_bytes": nws, "roofline": roof, "kernels": kernels, "cpu_baseline": cpu}


def bwd_kernel_bytes(name, w):
    """Algorithmic bytes per launch of each backward kernel: its own inputs
    and outputs read or written once (workspace arrays as the kernels hold
    them: float32, or bf16 hi + lo planes of the same size)."""
    erase = w.mode in ("delta", "gated_delta")
    d, C = w.dk, w.C
    nc = -(-w.L // C)
    bh = w.B * w.H
    tok = bh * w.L                 # real tokens
    ptok = bh * nc * C             # padded rows of the workspace arrays
    esz = 2 if w.dtype == "bf16" else 4
    cc = bh * nc * C * C * 4       # one C x C float record per chunk-head
    st = bh * nc * d * d * 4       # one state per chunk-head
    S = bh * d * d * 4             # one state per head
    return {
        # T^T once, for both walks
        "la_bwd_prep": tok * (3 * d * esz + 8) + ptok * 4 + (cc if erase else 0)
                       + ptok * d * 4 + st,
        "la_bwd_states": tok * (2 * d * esz + 8) + ptok * 4 + (cc if erase else 0) + S + st
                         + (ptok * d * 4 if erase else 0),
        "la_bwd_rev": tok * (d * esz + 4 + d * 4) + ptok * 4 + (cc if erase else 0)
                      + ptok * d * 4 + 2 * st + 2 * S + (ptok * d * 4 if erase else 0),
        "la_bwd_grads": tok * (4 * d * esz + 4 + 2 * d * 4 + 8) + ptok * 4 + 2 * st
                        + (2 * ptok * d * 4 if erase else 0),
    }.get(name)


def bwd_cpu_baseline(w, x, gr, tokens):
    """The float64 chunkwise backward oracle, as it stands, on the first
    `tokens` tokens of every head, BLAS limited to one thread."""
    import oracle
    import workloads
    from threadpoolctl import threadpool_limits

    sub = {k: (t[:, :, :tokens] if k != "S0" else t) for k, t in x.items()}
    y = workloads.to_f64(sub)
    g = workloads.to_f64({"dout": gr["dout"][:, :, :tokens], "dS_final": gr["dS_final"]})
    log(f"[bench] cpu baseline (backward): oracle on {tokens} tokens x {w.B * w.H} heads")
    with threadpool_limits(1):
        t0 = time.perf_counter()
        oracle.chunkwise_bwd(y["q"], y["k"], y["v"], y["log_alpha"], y["beta"],
                             y["S0"] if w.s0_std > 0 else None, w.mode, w.C, g["dout"],
                             g["dS_final"])
        sec = time.perf_counter() - t0
    return {"value": w.B * tokens / sec, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {tokens} of {w.L} tokens of all {w.B}x{w.H} (batch, head) "
                      f"sequences of {w.name}, float64 chunkwise backward, {sec:.1f} s"}


def varlen_lengths(n, total, seed):
    """Seeded length mix of a packed batch: n lengths summing to `total`,
    log-uniform between 1 and 16 K tokens (short prompts next to long
    documents), rescaled to the total."""
    import numpy as np
    rng = np.random.default_rng(seed)
    raw = np.exp(rng.uniform(0.0, np.log(16384.0), n))
    lens = np.maximum(1, np.floor(raw / raw.sum() * total)).astype(np.int64)
    lens[-1] += total - int(lens.sum())
    return [int(v) for v in lens]


def bench_varlen(base, n_seq, total, steps, warmup):
    """Packed batch of n_seq sequences (total tokens) with the recipe of
    `base` (mode, dtype, heads, d): la_chunk_fwd_varlen tokens/s."""
    import torch

    import chunkwise_gated_delta_la_amd as la
    import workloads

    lens = varlen_lengths(n_seq, total, seed=base.seed + 7)
    w = base.scaled(name=f"varlen_{base.mode}_{base.dtype}_n{n_seq}h{base.H}t{total}d{base.dk}",
                    B=1, L=total, s0_std=0.0)
    log(f"[bench] packed batch {w.name}: generating inputs")
    x = workloads.make_inputs(w)
    d = {k: t[0].contiguous().cuda() for k, t in x.items() if k != "S0"}
    cu = torch.tensor([0] + list(__import__("itertools").accumulate(lens)), dtype=torch.int32,
                      device="cuda")
    out = torch.empty((w.H, total, w.dv), dtype=w.torch_dtype, device="cuda")
    S_final = torch.empty((n_seq, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    nws = la.chunk_varlen_workspace_bytes(n_seq, w.H, total, w.dk, w.dv, mode=w.mode,
                                          dtype=w.torch_dtype)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")

    def step():
        la.chunk_fwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], None, cu,
                            mode=w.mode, out=out, S_final=S_final, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    with la.kernel_timer() as kt:
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    sec = (t1 - t0) / steps
    token_heads = w.H * total
    res = {"workload": w.name, "mode": w.mode, "sequences": n_seq, "tokens": total,
           "length_min": min(lens), "length_max": max(lens),
           "tokens_per_s": round(total / sec, 1), "ms_per_step": round(sec * 1e3, 4),
           "kernels": _kernel_table(kt.stats, w, token_heads, n_seq * w.H)}
    del d, out, ws
    torch.cuda.empty_cache()
    return res


def bench_bwd_fused(w, steps, warmup):
    """la_chunk_bwd_fused (q, k normalisation and the gate activations inside)
    at a forward workload's sizes, from the raw inputs: tokens/s and the
    per-kernel times (the prologue and its gradients are two extra kernels)."""
    import torch

    import chunkwise_gated_delta_la_amd as la
    import workloads

    log(f"[bench] fused backward {w.name}: generating inputs")
    r = {k: t.cuda() for k, t in workloads.make_raw_inputs(w).items()}
    gr = {k: t.cuda() for k, t in workloads.make_upstream_grads(w, ds_std=0.02).items()}
    nws = la.chunk_bwd_workspace_bytes(w.B, w.H, w.L, w.dk, w.dv, mode=w.mode,
                                       dtype=w.torch_dtype, qk_l2norm=True, gate_act=True)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    ms, kernels = _timed(lambda: la.chunk_bwd(r["q"], r["k"], r["v"], r["a_raw"], r["b_raw"],
                                              r["S0"], gr["dout"], gr["dS_final"], mode=w.mode,
                                              workspace=ws, qk_l2norm=True, gate_act=True),
                         steps, warmup)
    del r, gr, ws
    torch.cuda.empty_cache()
    return {"workload": "backward_fused_" + w.name, "mode": w.mode,
            "steps_fused": "qk_l2norm, gate_act", "ms_per_step": round(ms, 4),
            "tokens_per_s": round(w.B * w.L / ms * 1e3, 1), "kernels": kernels}

def bench_bwd_varlen(base, n_seq, total, steps, warmup):
    """la_chunk_bwd_varlen over the packed batch of bench_varlen (same length
    mix, upstream gradients N(0, 1)): tokens/s and per-kernel times."""
    import torch

    import chunkwise_gated_delta_la_amd as la
    import workloads

    lens = varlen_lengths(n_seq, total, seed=base.seed + 7)
    w = base.scaled(name=f"varlen_{base.mode}_{base.dtype}_n{n_seq}h{base.H}t{total}d{base.dk}",
                    B=1, L=total, s0_std=0.0)
    log(f"[bench] packed backward {w.name}: generating inputs")
    x = workloads.make_inputs(w)
    d = {k: t[0].contiguous().cuda() for k, t in x.items() if k != "S0"}
    gr = workloads.make_upstream_grads(w, ds_std=0.0)
    dout = gr["dout"][0].contiguous().cuda()
    cu = torch.tensor([0] + list(__import__("itertools").accumulate(lens)), dtype=torch.int32,
                      device="cuda")
    nws = la.chunk_bwd_varlen_workspace_bytes(n_seq, w.H, total, w.dk, w.dv, mode=w.mode,
                                              dtype=w.torch_dtype)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    ms, kernels = _timed(lambda: la.chunk_bwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"],
                                                     d["beta"], None, dout, cu, mode=w.mode,
                                                     workspace=ws), steps, warmup)
    del d, dout, ws
    torch.cuda.empty_cache()
    return {"workload": "backward_" + w.name, "mode": w.mode, "sequences": n_seq,
            "tokens": total, "length_min": min(lens), "length_max": max(lens),
            "tokens_per_s": round(total / ms * 1e3, 1), "ms_per_step": round(ms, 4),
            "kernels": kernels}

def bench_decode(w, warmup=1):
    import torch

    import chunkwise_gated_delta_la_amd as la
    import workloads

    log(f"[bench] decode workload {w.name}: generating inputs")
    x = workloads.make_inputs(w)
    d = {k: t.cuda() for k, t in x.items()}
    S = d["S0"].clone()
    outs = torch.empty((w.steps, w.B, w.H, w.dv), dtype=w.torch_dtype, device="cuda")

    def run():
        for n in range(w.steps):
            la.decode_step(d["q"][n], d["k"][n], d["v"][n], d["log_alpha"][n], d["beta"][n],
                           S, mode=w.mode, out=outs[n])

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    log(f"[bench] decode: {w.steps} timed steps")
    with la.kernel_timer() as kt:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    n, ms = kt.stats["la_decode"]
    avg_ms = ms / n
    by = decode_bytes_per_head(w) * w.B * w.H
    gbs = by / (avg_ms * 1e-3) / 1e9
    wall = (t1 - t0) / w.steps
    return {
        "workload": w.name, "steps": w.steps,
        "tokens_per_s": w.B / wall,
        "ms_per_step_wall": wall * 1e3,
        "kernel_avg_ms": round(avg_ms, 5),
        "state_GBs": round(gbs, 1),
        "roofline": {"kernel": "la_decode", "bound": "hbm", "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("la_decode", w.name),
                     "algorithmic_bytes": by},
    }


_POOL_INPUTS = {}


def cpu_workers():
    """Worker processes for the oracle baseline: the CPUs this process may
    run on, bounded by a cgroup CPU quota when one is set, and by
    LA_BENCH_CPU_WORKERS (default 16, one GPU's share of a shared host)."""
    n = len(os.sched_getaffinity(0))
    try:
        quota, period = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if quota != "max":
            n = min(n, max(1, -(-int(quota) // int(period))))
    except (OSError, ValueError):
        pass
    return max(1, min(n, int(os.environ.get("LA_BENCH_CPU_WORKERS", "16"))))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_task(task):
    """One worker's share: the oracle on a slice of (batch, head) pairs."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    key, heads, tokens = task
    w, x = _POOL_INPUTS[key]
    bs = [b for b, _ in heads]
    hs = [h for _, h in heads]
    with threadpool_limits(1):
        if w.is_decode:            # decode: [steps, B, H, ...]
            sel = lambda t: t[:tokens, bs, hs][:, None].to("cpu").double().numpy()   # noqa: E731
            oracle.decode_steps(x["S0"][bs, hs][None].double().numpy(), sel(x["q"]),
                                sel(x["k"]), sel(x["v"]), sel(x["log_alpha"]), sel(x["beta"]),
                                w.mode)
        else:
            sel = lambda t: t[bs, hs][None, :, :tokens].double().numpy()   # noqa: E731
            s0 = x["S0"][bs, hs][None].double().numpy() if w.s0_std > 0 else None
            oracle.recurrent_fwd(sel(x["q"]), sel(x["k"]), sel(x["v"]), sel(x["log_alpha"]),
                                 sel(x["beta"]), s0, w.mode)
    return len(heads) * tokens


def cpu_baseline(w, x, tokens):
    """The float64 oracle, as it stands, on the first `tokens` tokens (decode:
    steps) of every (batch, head) sequence of workload `w`, split over a
    pool of worker processes (one BLAS thread each).  Must run before this
    process touches the GPU (the pool forks)."""
    import multiprocessing as mp

    n = cpu_workers()
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)]
    per = -(-len(pairs) // n)
    tasks = [(w.name, pairs[i:i + per], tokens) for i in range(0, len(pairs), per)]
    _POOL_INPUTS[w.name] = (w, x)
    log(f"[bench] cpu baseline {w.name}: oracle on {tokens} tokens x {len(pairs)} heads, "
        f"{len(tasks)} tasks on {n} workers")
    with mp.get_context("fork").Pool(min(n, len(tasks))) as pool:
        t0 = time.perf_counter()
        done = sum(pool.map(_oracle_task, tasks, chunksize=1))
        sec = time.perf_counter() - t0
    del _POOL_INPUTS[w.name]
    unit_tokens = done / w.H          # (b, token) pairs: tokens/s counts B * L
    what = "steps" if w.is_decode else "tokens"
    full = w.steps if w.is_decode else w.L
    return {"value": round(unit_tokens / sec, 1), "unit": "tokens/s", "cores": min(n, len(tasks)),
            "kind": "oracle", "cpu_model": cpu_model(), "host_logical_cpus": os.cpu_count(),
            "sample": f"first {tokens} of {full} {what} of all {w.B}x{w.H} (batch, head) "
                      f"sequences of {w.name}, float64 token recurrence, "
                      f"{min(n, len(tasks))} worker processes, {sec:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=4,
                    help="forward workload id in workloads.WORKLOADS (default 4)")
    ap.add_argument("--shard", type=int, default=1, metavar="N",
                    help="time one GPU's share of the forward workload when its heads are "
                         "split over N GPUs (H / N heads on this GPU)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the extra measurements (other configurations, modes, packed "
                         "batch, fused steps, backward)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the legs of the other forward configurations (1-3)")
    ap.add_argument("--only-backward", action="store_true",
                    help="only time la_chunk_bwd at the forward workload's sizes and print "
                         "that measurement (for profiling runs)")
    ap.add_argument("--bwd-cpu-tokens", type=int, default=32768,
                    help="tokens per head of the backward's CPU oracle sample (0 = skip)")
    ap.add_argument("--cpu-tokens", type=int, default=16384,
                    help="tokens per head of the CPU oracle sample (0 = skip)")
    ap.add_argument("--segment-sweep", action="store_true",
                    help="only time the forward at explicit segment counts against the "
                         "plan, for 1-16 heads of the workload's sequence")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain MIB-MiB device copy (traffic calibration)")
    ap.add_argument("--ingest-pmc", nargs=5, metavar=("FETCH", "WRITE", "CAL_FETCH",
                                                      "CAL_WRITE", "COMMAND"),
                    help="write profiles/traffic.json from rocprofv3 --pmc CSV folders")
    args = ap.parse_args()
    if args.ingest_pmc:
        import workloads
        wname = workloads.WORKLOADS[args.workload].name
        if args.only_backward:
            wl = {k: "backward_" + wname for k in KERNEL_SOURCES if k.startswith("la_bwd")}
        else:
            wl = {"la_chunk": wname, "la_tsolve": wname, "la_decode": workloads.WORKLOADS[5].name}
        ingest_pmc(*args.ingest_pmc[:4], wl, args.ingest_pmc[4])
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not "
              "supported (the forward shards over (batch, head) or over the sequence, "
              "see the design notes, but no multi-GPU path is built).", file=sys.stderr)
        sys.exit(2)

    import workloads

    w = workloads.head_shard(workloads.WORKLOADS[args.workload], args.shard)
    configs = () if (args.no_extra or args.no_configs or args.only_backward or
                     args.calibrate_copy) else (1, 2, 3)
    # The CPU oracle baselines run first: their worker pool forks, which
    # must happen before this process touches the GPU.
    x = cpu = None
    cpu_cfg = {}
    if not (args.only_backward or args.calibrate_copy or args.segment_sweep):
        x = workloads.make_inputs(w)
        if args.cpu_tokens > 0:
            cpu = cpu_baseline(w, x, min(args.cpu_tokens, w.L))
            for i in configs:
                wi = workloads.WORKLOADS[i]
                cpu_cfg[i] = cpu_baseline(wi, workloads.make_inputs(wi), wi.L)
            if not args.no_decode:
                wd = workloads.WORKLOADS[5]
                cpu_cfg[5] = cpu_baseline(wd, workloads.make_inputs(wd), 16)

    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.segment_sweep:
        print(json.dumps({"segment_sweep": {
            "workload": workloads.WORKLOADS[args.workload].name,
            "sweep": segment_sweep(workloads.WORKLOADS[args.workload], 5, 2)}}), flush=True)
        return
    if args.only_backward:
        print(json.dumps({"backward": bench_backward(w, args.steps, args.warmup,
                                                     args.bwd_cpu_tokens)}), flush=True)
        return
    _, fwd = bench_forward(w, args.steps, args.warmup, x)
    dec = None
    if not args.no_decode:
        dec = bench_decode(workloads.WORKLOADS[5])
        dec["cpu_baseline"] = cpu_cfg.get(5)
    cfg = {f"config{i}": bench_config(workloads.WORKLOADS[i], args.steps, 1, cpu_cfg.get(i))
           for i in configs}
    extra = None
    if not args.no_extra:
        extra = {
            "gated_linear": bench_mode(w.scaled(name=w.name.replace(w.mode, "gated_linear"),
                                                mode="gated_linear"), args.steps, 1),
            "varlen": bench_varlen(w, 64, w.L, args.steps, 1),
            "segments": bench_segments(workloads.WORKLOAD4_SHARD8, args.steps, 1),
            "fused": bench_fused(w, args.steps, 1),
            "noncausal": bench_noncausal(workloads.WORKLOADS[2], args.steps, 1),
            "backward": bench_backward(w, args.steps, 1, args.bwd_cpu_tokens),
            "backward_varlen": bench_bwd_varlen(w, 64, w.L, args.steps, 1),
            "backward_fused": bench_bwd_fused(w, args.steps, 1),
        }
    line = {
        "metric": METRIC,
        "value": fwd["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": fwd["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "mode": w.mode, "B": w.B, "H": w.H, "L": w.L,
                   "dk": w.dk, "dv": w.dv, "C": w.C, "inputs": w.dtype + " q/k/v/out, "
                   "float32 gates and state", "segments": fwd["segments"],
                   "head_shard_of": args.shard},
        "mfma_frac_of_bf16_peak": round(fwd["mfma_frac_of_bf16_peak"], 4),
        "mfma_frac_exact": round(fwd["mfma_frac_exact"], 4),
        "hbm_frac_of_min_bytes": round(fwd["hbm_frac_of_min_bytes"], 4),
        "roofline": fwd["roofline"],
        "kernels": fwd["kernels"],
        "decode": dec,
        "configs": cfg,
        "extra": extra,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
