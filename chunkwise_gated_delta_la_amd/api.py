"""Tensor-level entry points with the same names as the C ABI calls.

Argument marshalling only: shapes, dtypes, devices and contiguity are
checked here so that errors name the offending tensor; the library checks
them again and does all the work.
"""
import ctypes

import torch

from . import _lib

MODES = {"linear": 0, "delta": 1, "gated_delta": 2, "gated_linear": 3}
_DECAY = (2, 3)      # modes that read log_alpha
_ERASE = (1, 2)      # modes that read beta
_DTYPES = {torch.float32: 0, torch.bfloat16: 1}


def _dtype_code(in_dtype, out_dtype):
    if in_dtype == torch.float32 and out_dtype == torch.float32:
        return 0
    if in_dtype == torch.bfloat16 and out_dtype == torch.bfloat16:
        return 1
    if in_dtype == torch.bfloat16 and out_dtype == torch.float32:
        return 2
    raise TypeError(f"unsupported (input, output) dtypes ({in_dtype}, {out_dtype})")


def version():
    return _lib.get().la_version().decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, shape, dtype, device):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _mode(mode):
    if mode not in MODES:
        raise ValueError(f"mode must be one of {sorted(MODES)}, got {mode!r}")
    return MODES[mode]


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


PRO_GATES, PRO_QK_L2NORM, EPI_DSKIP, EPI_OUT_NORM = 1, 2, 4, 8     # la_fused_flag_t


def _fused_opts(qk_l2norm=False, gate_act=False, gate_scale=1.0 / 16.0, dskip=None,
                out_norm=False, norm_weight=None, norm_eps=1e-6):
    """la_fused_opts_t for these steps, or None when none is asked for."""
    flags = ((PRO_QK_L2NORM if qk_l2norm else 0) | (PRO_GATES if gate_act else 0)
             | (EPI_DSKIP if dskip is not None else 0) | (EPI_OUT_NORM if out_norm else 0))
    if not flags:
        return None
    return _lib.FusedOpts(flags, float(gate_scale), _ptr(dskip).value if dskip is not None
                          else None, _ptr(norm_weight).value if norm_weight is not None
                          else None, float(norm_eps))


def chunk_workspace_bytes(B, H, L, dk, dv, *, mode="gated_delta", C=64,
                          dtype=torch.bfloat16, out_dtype=None, segments=None,
                          qk_l2norm=False, gate_act=False, fused=None):
    """Workspace bytes ``la_chunk_fwd`` needs for these sizes
    (``la_chunk_workspace_bytes``), or ``la_chunk_fwd_segmented`` with
    ``segments`` segments (``la_chunk_segmented_workspace_bytes``), or
    ``la_chunk_fwd_fused`` with its prologue (``la_chunk_fused_workspace_bytes``)."""
    code = _dtype_code(dtype, out_dtype or dtype)
    n = ctypes.c_size_t(0)
    lib = _lib.get()
    opts = fused if fused is not None else _fused_opts(qk_l2norm, gate_act)
    if opts is not None:
        if segments is not None:
            raise ValueError("the fused forward runs with the automatic segment plan")
        rc = lib.la_chunk_fused_workspace_bytes(B, H, L, dk, dv, C, _mode(mode), code,
                                                ctypes.byref(opts), ctypes.byref(n))
    elif segments is None:
        rc = lib.la_chunk_workspace_bytes(B, H, L, dk, dv, C, _mode(mode), code, ctypes.byref(n))
    else:
        rc = lib.la_chunk_segmented_workspace_bytes(B, H, L, dk, dv, C, _mode(mode), code,
                                                    int(segments), ctypes.byref(n))
    _lib.check(rc)
    return n.value


def chunk_segments(B, H, L, dk, dv, *, mode="gated_delta", C=64, dtype=torch.bfloat16,
                   out_dtype=None):
    """Segments per sequence ``la_chunk_fwd`` runs in parallel for these
    sizes (``la_chunk_segments``; 1 = the whole-sequence walk)."""
    code = _dtype_code(dtype, out_dtype or dtype)
    n = ctypes.c_int(0)
    _lib.check(_lib.get().la_chunk_segments(B, H, L, dk, dv, C, _mode(mode), code,
                                            ctypes.byref(n)))
    return n.value


def chunk_fwd(q, k, v, log_alpha=None, beta=None, S0=None, *, mode="gated_delta",
              C=64, out=None, S_final=None, return_state=True, out_dtype=None,
              workspace=None, segments=None, qk_l2norm=False, gate_act=False,
              gate_scale=1.0 / 16.0, dskip=None, out_norm=False, norm_weight=None,
              norm_eps=1e-6):
    """Chunkwise forward (``la_chunk_fwd``; ``la_chunk_fwd_segmented`` when
    ``segments`` is given: each sequence cut into that many segments run in
    parallel; ``la_chunk_fwd_fused`` when a fused step is asked for:
    ``qk_l2norm`` -- q and k normalised inside; ``gate_act`` -- log_alpha
    and beta are raw scores a, b, used as -gate_scale softplus(a) and
    sigmoid(b); ``dskip`` -- a float32 ``[H, dv]`` tensor D, o += D v;
    ``out_norm`` -- o / sqrt(mean(o^2) + norm_eps) * norm_weight ``[H, dv]``
    (ones when None)).

    q, k ``[B, H, L, dk]``, v ``[B, H, L, dv]`` (float32 or bfloat16, on the
    GPU); log_alpha, beta ``[B, H, L]`` float32; S0 ``[B, H, dk, dv]`` float32
    or None.  Returns ``(out, S_final)`` (S_final None if not requested).
    ``S_final`` may be the same tensor as ``S0`` for an in-place update.
    ``out_dtype`` (default: the input dtype) may be float32 for bf16 inputs.
    ``workspace`` is an optional uint8 device tensor of at least
    ``chunk_workspace_bytes(...)`` bytes; without one, a buffer of that size
    is taken from torch's allocator for the call.
    """
    m = _mode(mode)
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, L, d]")
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dt not in _DTYPES:
        raise TypeError(f"q must be float32 or bfloat16, got {dt}")
    _need(k, "k", (B, H, L, dk), dt, dev)
    _need(v, "v", (B, H, L, dv), dt, dev)
    _need(q, "q", (B, H, L, dk), dt, dev)
    _need(log_alpha if m in _DECAY else None, "log_alpha", (B, H, L), torch.float32, dev)
    _need(beta if m in _ERASE else None, "beta", (B, H, L), torch.float32, dev)
    _need(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    odt = out_dtype or (out.dtype if out is not None else dt)
    code = _dtype_code(dt, odt)
    if out is None:
        out = torch.empty((B, H, L, dv), dtype=odt, device=dev)
    _need(out, "out", (B, H, L, dv), odt, dev)
    if S_final is None and return_state:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    _need(S_final, "S_final", (B, H, dk, dv), torch.float32, dev)
    lib = _lib.get()
    for t, name in ((dskip, "dskip"), (norm_weight, "norm_weight")):
        _need(t, name, (H, dv), torch.float32, dev)
    opts = _fused_opts(qk_l2norm, gate_act, gate_scale, dskip, out_norm, norm_weight, norm_eps)
    need = chunk_workspace_bytes(B, H, L, dk, dv, mode=mode, C=C, dtype=dt, out_dtype=odt,
                                 segments=segments, fused=opts)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        if workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    ws_bytes = 0 if workspace is None else workspace.numel()
    with torch.cuda.device(dev):
        la, be = _ptr(log_alpha if m in _DECAY else None), _ptr(beta if m in _ERASE else None)
        if opts is not None:
            rc = lib.la_chunk_fwd_fused(_ptr(q), _ptr(k), _ptr(v), la, be, _ptr(S0), _ptr(out),
                                        _ptr(S_final), B, H, L, dk, dv, C, m, code,
                                        ctypes.byref(opts), _ptr(workspace), ws_bytes,
                                        _stream(dev))
        elif segments is None:
            rc = lib.la_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), la, be, _ptr(S0), _ptr(out),
                                  _ptr(S_final), B, H, L, dk, dv, C, m, code, _ptr(workspace),
                                  ws_bytes, _stream(dev))
        else:
            rc = lib.la_chunk_fwd_segmented(_ptr(q), _ptr(k), _ptr(v), la, be, _ptr(S0),
                                            _ptr(out), _ptr(S_final), B, H, L, dk, dv, C, m,
                                            code, int(segments), _ptr(workspace), ws_bytes,
                                            _stream(dev))
    _lib.check(rc)
    return out, S_final


NOALLOC_SCRATCH_BYTES = 128 << 20      # LA_NOALLOC_SCRATCH_BYTES


def chunk_fwd_noalloc(q, k, v, log_alpha, beta, S0, out, S_final=None, *,
                      mode="gated_delta", C=64):
    """``la_chunk_fwd_noalloc``: the chunkwise forward with the library's
    static per-GPU scratch in place of a workspace, for callers that must not
    allocate.  The caller passes every tensor, ``out`` and ``S_final`` (or
    None) included; nothing is allocated here or in the library.  Calls that
    overlap in time on one GPU race on the shared scratch.  Shapes and dtypes
    as ``chunk_fwd``; the output dtype is ``out``'s."""
    m = _mode(mode)
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, L, d]")
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dt not in _DTYPES:
        raise TypeError(f"q must be float32 or bfloat16, got {dt}")
    if out is None:
        raise ValueError("out is required (this entry point allocates nothing)")
    _need(k, "k", (B, H, L, dk), dt, dev)
    _need(v, "v", (B, H, L, dv), dt, dev)
    _need(log_alpha if m in _DECAY else None, "log_alpha", (B, H, L), torch.float32, dev)
    _need(beta if m in _ERASE else None, "beta", (B, H, L), torch.float32, dev)
    _need(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    code = _dtype_code(dt, out.dtype)
    _need(out, "out", (B, H, L, dv), out.dtype, dev)
    _need(S_final, "S_final", (B, H, dk, dv), torch.float32, dev)
    lib = _lib.get()
    with torch.cuda.device(dev):
        la, be = _ptr(log_alpha if m in _DECAY else None), _ptr(beta if m in _ERASE else None)
        rc = lib.la_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), la, be, _ptr(S0), _ptr(out),
                                      _ptr(S_final), B, H, L, dk, dv, C, m, code, _stream(dev))
    _lib.check(rc)
    return out, S_final


def noncausal_fwd(q, k, v, S0=None, *, out=None, S_final=None, return_state=True,
                  out_dtype=None, workspace=None):
    """Bidirectional linear attention (``la_noncausal_fwd``): S = S0 + K^T V
    over the whole sequence and o_t = S^T q_t for every token.  q, k, v
    ``[B, H, L, d]`` bfloat16; S0 ``[B, H, d, d]`` float32 or None.  Returns
    ``(out, S_final)``."""
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, L, d]")
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dt != torch.bfloat16:
        raise TypeError(f"noncausal_fwd takes bfloat16 q, k, v, got {dt}")
    _need(k, "k", (B, H, L, dk), dt, dev)
    _need(v, "v", (B, H, L, dv), dt, dev)
    _need(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    odt = out_dtype or (out.dtype if out is not None else dt)
    code = _dtype_code(dt, odt)
    if out is None:
        out = torch.empty((B, H, L, dv), dtype=odt, device=dev)
    _need(out, "out", (B, H, L, dv), odt, dev)
    if S_final is None and return_state:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    _need(S_final, "S_final", (B, H, dk, dv), torch.float32, dev)
    lib = _lib.get()
    n = ctypes.c_size_t(0)
    _lib.check(lib.la_noncausal_workspace_bytes(B, H, L, dk, dv, code, ctypes.byref(n)))
    if workspace is None:
        workspace = torch.empty(max(n.value, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        rc = lib.la_noncausal_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(S0), _ptr(out), _ptr(S_final),
                                  B, H, L, dk, dv, code, _ptr(workspace), workspace.numel(),
                                  _stream(dev))
    _lib.check(rc)
    return out, S_final


def chunk_varlen_workspace_bytes(N, H, T, dk, dv, *, mode="gated_delta", C=64,
                                 dtype=torch.bfloat16, out_dtype=None):
    """Workspace bytes ``la_chunk_fwd_varlen`` needs for these sizes
    (``la_chunk_varlen_workspace_bytes``)."""
    code = _dtype_code(dtype, out_dtype or dtype)
    n = ctypes.c_size_t(0)
    _lib.check(_lib.get().la_chunk_varlen_workspace_bytes(N, H, T, dk, dv, C, _mode(mode), code,
                                                          ctypes.byref(n)))
    return n.value


def chunk_fwd_varlen(q, k, v, log_alpha, beta, S0, cu_seqlens, *, mode="gated_delta", C=64,
                     out=None, S_final=None, return_state=True, out_dtype=None,
                     workspace=None):
    """Chunkwise forward over a packed batch (``la_chunk_fwd_varlen``).

    q, k ``[H, T, dk]``, v ``[H, T, dv]``: the tokens of N sequences back to
    back per head; log_alpha, beta ``[H, T]`` float32; cu_seqlens ``[N + 1]``
    int32 on the GPU (sequence s is tokens cu_seqlens[s] .. cu_seqlens[s+1]-1);
    S0 ``[N, H, dk, dv]`` float32 or None.  Returns ``(out [H, T, dv],
    S_final [N, H, dk, dv])``.
    """
    m = _mode(mode)
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [H, T, d]")
    H, T, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dt not in _DTYPES:
        raise TypeError(f"q must be float32 or bfloat16, got {dt}")
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be [N + 1] with N >= 1")
    N = cu_seqlens.numel() - 1
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    _need(k, "k", (H, T, dk), dt, dev)
    _need(v, "v", (H, T, dv), dt, dev)
    _need(log_alpha if m in _DECAY else None, "log_alpha", (H, T), torch.float32, dev)
    _need(beta if m in _ERASE else None, "beta", (H, T), torch.float32, dev)
    _need(S0, "S0", (N, H, dk, dv), torch.float32, dev)
    odt = out_dtype or (out.dtype if out is not None else dt)
    code = _dtype_code(dt, odt)
    if out is None:
        out = torch.empty((H, T, dv), dtype=odt, device=dev)
    _need(out, "out", (H, T, dv), odt, dev)
    if S_final is None and return_state:
        S_final = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    _need(S_final, "S_final", (N, H, dk, dv), torch.float32, dev)
    need = chunk_varlen_workspace_bytes(N, H, T, dk, dv, mode=mode, C=C, dtype=dt,
                                        out_dtype=odt)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        if workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    ws_bytes = 0 if workspace is None else workspace.numel()
    lib = _lib.get()
    with torch.cuda.device(dev):
        rc = lib.la_chunk_fwd_varlen(_ptr(q), _ptr(k), _ptr(v),
                                     _ptr(log_alpha if m in _DECAY else None),
                                     _ptr(beta if m in _ERASE else None), _ptr(S0),
                                     _ptr(out), _ptr(S_final), _ptr(cu_seqlens), N, H, T, dk, dv,
                                     C, m, code, _ptr(workspace), ws_bytes, _stream(dev))
    _lib.check(rc)
    return out, S_final


def decode_step(q, k, v, log_alpha, beta, S, *, mode="gated_delta", out=None,
                out_dtype=None, qk_l2norm=False, gate_act=False, gate_scale=1.0 / 16.0,
                dskip=None, out_norm=False, norm_weight=None, norm_eps=1e-6):
    """One recurrent decode step (``la_decode_step``), updating ``S`` in place.

    q, k ``[B, H, dk]``, v ``[B, H, dv]`` (float32 or bfloat16); log_alpha,
    beta ``[B, H]`` float32; S ``[B, H, dk, dv]`` float32.  Returns ``out``
    ``[B, H, dv]``.  The fused steps (``qk_l2norm``, ``gate_act``,
    ``gate_scale``, ``dskip``, ``out_norm``, ``norm_weight``, ``norm_eps``)
    as in ``chunk_fwd`` (``la_decode_step_fused``).
    """
    m = _mode(mode)
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [B, H, d]")
    B, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dt not in _DTYPES:
        raise TypeError(f"q must be float32 or bfloat16, got {dt}")
    _need(k, "k", (B, H, dk), dt, dev)
    _need(v, "v", (B, H, dv), dt, dev)
    _need(log_alpha if m in _DECAY else None, "log_alpha", (B, H), torch.float32, dev)
    _need(beta if m in _ERASE else None, "beta", (B, H), torch.float32, dev)
    _need(S, "S", (B, H, dk, dv), torch.float32, dev)
    odt = out_dtype or (out.dtype if out is not None else dt)
    code = _dtype_code(dt, odt)
    if out is None:
        out = torch.empty((B, H, dv), dtype=odt, device=dev)
    _need(out, "out", (B, H, dv), odt, dev)
    lib = _lib.get()
    for t, name in ((dskip, "dskip"), (norm_weight, "norm_weight")):
        _need(t, name, (H, dv), torch.float32, dev)
    opts = _fused_opts(qk_l2norm, gate_act, gate_scale, dskip, out_norm, norm_weight, norm_eps)
    la, be = _ptr(log_alpha if m in _DECAY else None), _ptr(beta if m in _ERASE else None)
    with torch.cuda.device(dev):
        if opts is not None:
            rc = lib.la_decode_step_fused(_ptr(q), _ptr(k), _ptr(v), la, be, _ptr(S), _ptr(out),
                                          B, H, dk, dv, m, code, ctypes.byref(opts),
                                          _stream(dev))
        else:
            rc = lib.la_decode_step(_ptr(q), _ptr(k), _ptr(v), la, be, _ptr(S), _ptr(out),
                                    B, H, dk, dv, m, code, _stream(dev))
    _lib.check(rc)
    return out


class kernel_timer:
    """Context manager timing the library's kernel launches with HIP events
    (``la_profile_begin`` / ``la_profile_end``).  On exit, ``stats`` maps a
    kernel name to ``(launches, total_ms)``; leaving the block waits for
    the recorded events."""

    def __enter__(self):
        _lib.check(_lib.get().la_profile_begin())
        self.stats = {}
        return self

    def __exit__(self, *exc):
        lib = _lib.get()
        buf = (_lib.KernelTime * 16)()
        n = ctypes.c_int(0)
        rc = lib.la_profile_end(buf, 16, ctypes.byref(n))
        for i in range(min(n.value, 16)):
            self.stats[buf[i].name.decode()] = (buf[i].launches, buf[i].total_ms)
        if exc[0] is None:
            _lib.check(rc)
        return False


def chunk_bwd_workspace_bytes(B, H, L, dk, dv, *, mode="gated_delta", C=64,
                              dtype=torch.bfloat16, qk_l2norm=False, gate_act=False,
                              fused=None):
    """Workspace bytes ``la_chunk_bwd`` needs for these sizes
    (``la_chunk_bwd_workspace_bytes``), or ``la_chunk_bwd_fused`` with its
    prologue (``la_chunk_bwd_fused_workspace_bytes``)."""
    code = _dtype_code(dtype, dtype)
    n = ctypes.c_size_t(0)
    opts = fused if fused is not None else _fused_opts(qk_l2norm, gate_act)
    if opts is not None:
        _lib.check(_lib.get().la_chunk_bwd_fused_workspace_bytes(
            B, H, L, dk, dv, C, _mode(mode), code, ctypes.byref(opts), ctypes.byref(n)))
    else:
        _lib.check(_lib.get().la_chunk_bwd_workspace_bytes(B, H, L, dk, dv, C, _mode(mode),
                                                           code, ctypes.byref(n)))
    return n.value


def chunk_bwd(q, k, v, log_alpha, beta, S0, dout, dS_final=None, *, mode="gated_delta",
              C=64, workspace=None, want_dS0=True, qk_l2norm=False, gate_act=False,
              gate_scale=1.0 / 16.0):
    """Gradients of ``chunk_fwd`` (``la_chunk_bwd``) for upstream gradients
    ``dout [B, H, L, dv]`` (the inputs' dtype) and ``dS_final [B, H, dk, dv]``
    float32 (or None: zero).  With ``qk_l2norm`` / ``gate_act`` the
    gradients of the fused forward's raw inputs (``la_chunk_bwd_fused``):
    q, k unnormalised, log_alpha and beta the raw scores a and b.

    Returns a dict of float32 tensors ``dq, dk, dv [B, H, L, d]``,
    ``dlog_alpha, dbeta [B, H, L]`` (the gradients of the gate arguments
    passed -- the raw scores with ``gate_act``; None where the mode does not
    read the gate) and ``dS0 [B, H, dk, dv]`` (None unless ``want_dS0``).
    ``workspace`` is an optional uint8 device tensor of at least
    ``chunk_bwd_workspace_bytes(...)`` bytes.
    """
    m = _mode(mode)
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, L, d]")
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dt not in _DTYPES:
        raise TypeError(f"q must be float32 or bfloat16, got {dt}")
    _need(k, "k", (B, H, L, dk), dt, dev)
    _need(v, "v", (B, H, L, dv), dt, dev)
    _need(dout, "dout", (B, H, L, dv), dt, dev)
    _need(log_alpha if m in _DECAY else None, "log_alpha", (B, H, L), torch.float32, dev)
    _need(beta if m in _ERASE else None, "beta", (B, H, L), torch.float32, dev)
    _need(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    _need(dS_final, "dS_final", (B, H, dk, dv), torch.float32, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    res = {"dq": torch.empty((B, H, L, dk), **f32), "dk": torch.empty((B, H, L, dk), **f32),
           "dv": torch.empty((B, H, L, dv), **f32),
           "dlog_alpha": torch.empty((B, H, L), **f32) if m in _DECAY else None,
           "dbeta": torch.empty((B, H, L), **f32) if m in _ERASE else None,
           "dS0": torch.empty((B, H, dk, dv), **f32) if want_dS0 else None}
    opts = _fused_opts(qk_l2norm, gate_act, gate_scale)
    need = chunk_bwd_workspace_bytes(B, H, L, dk, dv, mode=mode, C=C, dtype=dt, fused=opts)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    lib = _lib.get()
    if opts is not None:
        with torch.cuda.device(dev):
            rc = lib.la_chunk_bwd_fused(
                _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha if m in _DECAY else None),
                _ptr(beta if m in _ERASE else None), _ptr(S0), _ptr(dout), _ptr(dS_final),
                _ptr(res["dq"]), _ptr(res["dk"]), _ptr(res["dv"]), _ptr(res["dlog_alpha"]),
                _ptr(res["dbeta"]), _ptr(res["dS0"]), B, H, L, dk, dv, C, m, _DTYPES[dt],
                ctypes.byref(opts), _ptr(workspace), workspace.numel(), _stream(dev))
        _lib.check(rc)
        return res
    with torch.cuda.device(dev):
        rc = lib.la_chunk_bwd(_ptr(q), _ptr(k), _ptr(v),
                              _ptr(log_alpha if m in _DECAY else None),
                              _ptr(beta if m in _ERASE else None), _ptr(S0), _ptr(dout),
                              _ptr(dS_final), _ptr(res["dq"]), _ptr(res["dk"]), _ptr(res["dv"]),
                              _ptr(res["dlog_alpha"]), _ptr(res["dbeta"]), _ptr(res["dS0"]),
                              B, H, L, dk, dv, C, m, _DTYPES[dt], _ptr(workspace),
                              workspace.numel(), _stream(dev))
    _lib.check(rc)
    return res


def chunk_bwd_varlen_workspace_bytes(N, H, T, dk, dv, *, mode="gated_delta", C=64,
                                     dtype=torch.bfloat16):
    """Workspace bytes ``la_chunk_bwd_varlen`` needs for these sizes
    (``la_chunk_bwd_varlen_workspace_bytes``)."""
    code = _dtype_code(dtype, dtype)
    n = ctypes.c_size_t(0)
    _lib.check(_lib.get().la_chunk_bwd_varlen_workspace_bytes(N, H, T, dk, dv, C, _mode(mode),
                                                              code, ctypes.byref(n)))
    return n.value


def chunk_bwd_varlen(q, k, v, log_alpha, beta, S0, dout, cu_seqlens, dS_final=None, *,
                     mode="gated_delta", C=64, workspace=None, want_dS0=True):
    """Gradients of ``chunk_fwd_varlen`` (``la_chunk_bwd_varlen``): q, k
    ``[H, T, dk]``, v and ``dout`` ``[H, T, dv]`` (the inputs' dtype), gates
    ``[H, T]``, cu_seqlens ``[N + 1]`` int32 on the GPU, S0 and dS_final
    ``[N, H, dk, dv]`` float32 or None.  Returns a dict of float32 tensors as
    ``chunk_bwd`` does, in the packed layout."""
    m = _mode(mode)
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [H, T, d]")
    H, T, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dt not in _DTYPES:
        raise TypeError(f"q must be float32 or bfloat16, got {dt}")
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be [N + 1] with N >= 1")
    N = cu_seqlens.numel() - 1
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    _need(k, "k", (H, T, dk), dt, dev)
    _need(v, "v", (H, T, dv), dt, dev)
    _need(dout, "dout", (H, T, dv), dt, dev)
    _need(log_alpha if m in _DECAY else None, "log_alpha", (H, T), torch.float32, dev)
    _need(beta if m in _ERASE else None, "beta", (H, T), torch.float32, dev)
    _need(S0, "S0", (N, H, dk, dv), torch.float32, dev)
    _need(dS_final, "dS_final", (N, H, dk, dv), torch.float32, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    res = {"dq": torch.empty((H, T, dk), **f32), "dk": torch.empty((H, T, dk), **f32),
           "dv": torch.empty((H, T, dv), **f32),
           "dlog_alpha": torch.empty((H, T), **f32) if m in _DECAY else None,
           "dbeta": torch.empty((H, T), **f32) if m in _ERASE else None,
           "dS0": torch.empty((N, H, dk, dv), **f32) if want_dS0 else None}
    need = chunk_bwd_varlen_workspace_bytes(N, H, T, dk, dv, mode=mode, C=C, dtype=dt)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    lib = _lib.get()
    with torch.cuda.device(dev):
        rc = lib.la_chunk_bwd_varlen(_ptr(q), _ptr(k), _ptr(v),
                                     _ptr(log_alpha if m in _DECAY else None),
                                     _ptr(beta if m in _ERASE else None), _ptr(S0), _ptr(dout),
                                     _ptr(dS_final), _ptr(cu_seqlens), _ptr(res["dq"]),
                                     _ptr(res["dk"]), _ptr(res["dv"]), _ptr(res["dlog_alpha"]),
                                     _ptr(res["dbeta"]), _ptr(res["dS0"]), N, H, T, dk, dv, C,
                                     m, _DTYPES[dt], _ptr(workspace), workspace.numel(),
                                     _stream(dev))
    _lib.check(rc)
    return res
