"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, and rejects bad arguments before touching the GPU.

Only argument-validation paths are called here (NULL pointers, bad sizes,
unsupported shapes, overlapping fake pointers): each returns its error code
before any HIP call, so no GPU is needed and no device memory is touched.
"""
import ctypes
import os
import re

import pytest

from _lib_build import ROOT, ensure_built

ensure_built()
from chunkwise_gated_delta_la_amd import _lib  # noqa: E402

HEADER = os.path.join(ROOT, "include", "la.h")
OK, NULL, SHAPE, UNSUP, ALIAS, WS = 0, 1, 2, 3, 4, 6
TSOLVE_BYTES = 6 * 1024     # T operand fragments per chunk (bf16 delta modes)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = _lib.get()
    names = _declared_functions()
    assert {"la_chunk_fwd", "la_decode_step", "la_last_error", "la_version"} <= set(names)
    for name in names:
        assert hasattr(lib, name), f"{name} declared in la.h but not exported"


def test_version_and_empty_error():
    lib = _lib.get()
    assert lib.la_version().decode().startswith("lachunk ")
    assert lib.la_version().decode().endswith("gfx950")


P = 1 << 20            # fake, never dereferenced, well-separated pointers
P_BIG = P


def fake(i):
    return ctypes.c_void_p(P * (i + 1))


def chunk(lib, q=fake(0), k=fake(1), v=fake(2), la=fake(3), be=fake(4), s0=fake(5),
          out=fake(6), sf=fake(7), B=1, H=1, L=64, dk=64, dv=64, C=64, mode=2, dtype=1,
          ws=fake(8), wsb=P):
    return lib.la_chunk_fwd(q, k, v, la, be, s0, out, sf, B, H, L, dk, dv, C, mode, dtype,
                            ws, wsb, None)


def varlen(lib, q=fake(0), k=fake(1), v=fake(2), la=fake(3), be=fake(4), s0=fake(5),
           out=fake(6), sf=fake(7), cu=fake(9), N=2, H=1, T=64, dk=64, dv=64, C=64, mode=2,
           dtype=1, ws=fake(8), wsb=P):
    return lib.la_chunk_fwd_varlen(q, k, v, la, be, s0, out, sf, cu, N, H, T, dk, dv, C, mode,
                                   dtype, ws, wsb, None)


def varlen_ws(lib, N=2, H=1, T=64, dk=64, dv=64, C=64, mode=2, dtype=1):
    n = ctypes.c_size_t(0)
    rc = lib.la_chunk_varlen_workspace_bytes(N, H, T, dk, dv, C, mode, dtype, ctypes.byref(n))
    return rc, n.value


@pytest.mark.parametrize("kw,code", [
    (dict(cu=None), NULL), (dict(q=None), NULL), (dict(la=None), NULL),
    (dict(be=None, mode=1), NULL), (dict(N=0), SHAPE), (dict(T=-1), SHAPE), (dict(H=0), SHAPE),
    (dict(dk=96, dv=96), UNSUP), (dict(mode=4), UNSUP), (dict(C=32), UNSUP),
    (dict(out=ctypes.c_void_p(10 * P - 64)), ALIAS),       # out overlaps cu_seqlens
    (dict(ws=ctypes.c_void_p(10 * P - 1024)), ALIAS),      # workspace overlaps cu_seqlens
    (dict(sf=ctypes.c_void_p(2 * P + 64)), ALIAS),         # S_final overlaps k
    (dict(wsb=1), WS),
])
def test_chunk_fwd_varlen_rejects(kw, code):
    lib = _lib.get()
    assert varlen(lib, **kw) == code
    assert lib.la_last_error().decode() != ""


def test_varlen_workspace_size():
    """One T slot per chunk a sequence can start, per head: ceil(T/C) + N,
    whatever the offsets; nothing without erase or for float inputs."""
    lib = _lib.get()
    for (N, H, T) in ((1, 1, 1), (2, 3, 64), (5, 2, 1000), (100, 32, 65536)):
        for mode in (1, 2):
            assert varlen_ws(lib, N=N, H=H, T=T, mode=mode) == (
                OK, H * (-(-T // 64) + N) * TSOLVE_BYTES)
    assert varlen_ws(lib, mode=0) == (OK, 0)
    assert varlen_ws(lib, mode=3) == (OK, 0)
    assert varlen_ws(lib, dtype=0) == (OK, 0)
    assert varlen_ws(lib, T=0, N=3, H=2) == (OK, 2 * 3 * TSOLVE_BYTES)
    assert lib.la_chunk_varlen_workspace_bytes(1, 1, 64, 64, 64, 64, 2, 1, None) == NULL


def ws_bytes(lib, B=1, H=1, L=64, dk=64, dv=64, C=64, mode=2, dtype=1):
    n = ctypes.c_size_t(12345)
    rc = lib.la_chunk_workspace_bytes(B, H, L, dk, dv, C, mode, dtype, ctypes.byref(n))
    return rc, n.value


def decode(lib, q=fake(0), k=fake(1), v=fake(2), la=fake(3), be=fake(4), S=fake(5),
           out=fake(6), B=1, H=1, dk=64, dv=64, mode=2, dtype=1):
    return lib.la_decode_step(q, k, v, la, be, S, out, B, H, dk, dv, mode, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL), (dict(out=None), NULL),
    (dict(be=None), NULL), (dict(la=None), NULL), (dict(be=None, mode=1), NULL),
    (dict(B=0), SHAPE), (dict(H=-1), SHAPE), (dict(L=0), SHAPE), (dict(C=0), SHAPE),
    (dict(dk=64, dv=128), UNSUP), (dict(dk=96, dv=96), UNSUP),
    (dict(C=32, L=64), UNSUP), (dict(mode=4), UNSUP), (dict(dtype=7), UNSUP),
    (dict(la=None, mode=3), NULL),
    (dict(mode=-1), UNSUP), (dict(dtype=3), UNSUP),
])
def test_chunk_fwd_rejects(kw, code):
    lib = _lib.get()
    assert chunk(lib, **kw) == code
    assert lib.la_last_error().decode() != ""


def test_chunk_fwd_alias_rules():
    lib = _lib.get()
    # out overlapping q (q spans 64*64*2 bytes; out starts inside it)
    assert chunk(lib, out=ctypes.c_void_p(P + 128)) == ALIAS
    # S_final overlapping v
    assert chunk(lib, sf=ctypes.c_void_p(3 * P + 64)) == ALIAS
    # S_final partially overlapping S0 is rejected ...
    assert chunk(lib, sf=ctypes.c_void_p(6 * P + 4)) == ALIAS
    # ... out overlapping S_final too
    assert chunk(lib, out=ctypes.c_void_p(8 * P + 4)) == ALIAS


def test_workspace_size():
    """One T factor per chunk for bf16 inputs in the delta modes; nothing
    for float inputs or linear attention."""
    lib = _lib.get()
    for mode in (1, 2):
        for dtype in (1, 2):
            for (B, H, L, d) in ((1, 1, 64, 64), (2, 3, 256, 128), (1, 32, 65536, 128)):
                rc, n = ws_bytes(lib, B=B, H=H, L=L, dk=d, dv=d, mode=mode, dtype=dtype)
                assert rc == OK and n == B * H * (L // 64) * TSOLVE_BYTES
    assert ws_bytes(lib, mode=0) == (OK, 0)
    assert ws_bytes(lib, mode=3) == (OK, 0)
    assert ws_bytes(lib, dtype=0) == (OK, 0)
    # a partial last chunk gets its own T factor
    assert ws_bytes(lib, L=96) == (OK, 2 * TSOLVE_BYTES)
    assert ws_bytes(lib, L=1, B=3, H=2) == (OK, 6 * TSOLVE_BYTES)
    assert ws_bytes(lib, L=65537, H=32, dk=128, dv=128) == (OK, 32 * 1025 * TSOLVE_BYTES)
    assert ws_bytes(lib, dk=96, dv=96)[0] == UNSUP
    assert ws_bytes(lib, mode=5)[0] == UNSUP
    assert lib.la_chunk_workspace_bytes(1, 1, 64, 64, 64, 64, 2, 1, None) == NULL


@pytest.mark.parametrize("kw", [
    dict(ws=None), dict(wsb=TSOLVE_BYTES - 1), dict(ws=ctypes.c_void_p(9 * P + 8)),
    dict(B=2, wsb=TSOLVE_BYTES), dict(ws=None, wsb=P),
])
def test_chunk_fwd_workspace_rejects(kw):
    lib = _lib.get()
    assert chunk(lib, **kw) == WS
    assert "workspace" in lib.la_last_error().decode()


def test_chunk_fwd_workspace_alias_and_optional():
    lib = _lib.get()
    # workspace overlapping k, or out
    assert chunk(lib, ws=ctypes.c_void_p(2 * P - 1024)) == ALIAS
    assert chunk(lib, ws=ctypes.c_void_p(7 * P - 4096)) == ALIAS
    # float inputs and linear attention need none: a NULL workspace passes the
    # workspace checks and the call fails on the NULL q it was given instead
    assert chunk(lib, ws=None, wsb=0, dtype=0, q=None) == NULL
    assert chunk(lib, ws=None, wsb=0, mode=0, out=ctypes.c_void_p(P + 128)) == ALIAS


def test_chunk_fwd_unused_gates_may_alias_anything():
    """Gates a mode ignores are not part of its inputs: in linear mode a
    beta pointer equal to out is not an alias error (the call is only
    validated, never launched, because q is NULL)."""
    lib = _lib.get()
    assert chunk(lib, mode=0, be=fake(6), la=fake(6), q=None) == NULL
    # gated linear reads log_alpha but not beta: a NULL beta passes the gate
    # checks and the call stops at the alias check instead
    assert chunk(lib, mode=3, be=None, ws=None, wsb=0, out=ctypes.c_void_p(P + 128)) == ALIAS


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(S=None), NULL), (dict(out=None), NULL),
    (dict(be=None), NULL), (dict(la=None), NULL),
    (dict(B=0), SHAPE), (dict(dk=0), SHAPE), (dict(dk=32), UNSUP), (dict(dv=256), UNSUP),
    (dict(mode=7), UNSUP), (dict(dtype=5), UNSUP),
    (dict(out=ctypes.c_void_p(6 * P - 8)), ALIAS),      # out overlaps S's start
    (dict(S=ctypes.c_void_p(P + 64)), ALIAS),            # S overlaps q
])
def test_decode_rejects(kw, code):
    lib = _lib.get()
    assert decode(lib, **kw) == code
    assert lib.la_last_error().decode() != ""


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        _lib.get()


def segmented(lib, P=2, q=fake(0), k=fake(1), v=fake(2), la=fake(3), be=fake(4), s0=fake(5),
              out=fake(6), sf=fake(7), B=1, H=1, L=640, dk=64, dv=64, C=64, mode=2, dtype=1,
              ws=fake(8), wsb=P_BIG):
    return lib.la_chunk_fwd_segmented(q, k, v, la, be, s0, out, sf, B, H, L, dk, dv, C, mode,
                                      dtype, P, ws, wsb, None)


def seg_ws(lib, P, B=1, H=1, L=640, d=64, mode=2, dtype=1):
    n = ctypes.c_size_t(0)
    rc = lib.la_chunk_segmented_workspace_bytes(B, H, L, d, d, 64, mode, dtype, P,
                                                ctypes.byref(n))
    return rc, n.value


def plan(lib, B, H, L, d=128, mode=2, dtype=1):
    n = ctypes.c_int(0)
    assert lib.la_chunk_segments(B, H, L, d, d, 64, mode, dtype, ctypes.byref(n)) == OK
    return n.value


@pytest.mark.parametrize("kw,code", [
    (dict(P=0), SHAPE), (dict(P=-3), SHAPE), (dict(P=11), SHAPE),   # 10 chunks
    (dict(P=2, dtype=0), UNSUP), (dict(q=None), NULL), (dict(be=None), NULL),
    (dict(P=3, wsb=1), WS), (dict(sf=ctypes.c_void_p(2 * P + 64)), ALIAS),
])
def test_chunk_fwd_segmented_rejects(kw, code):
    lib = _lib.get()
    assert segmented(lib, **kw) == code
    assert lib.la_last_error().decode() != ""


def test_segmented_workspace_size():
    """The T factors (delta modes), then X, M and S_in of every segment:
    3 * B*H*P*d*d floats, placed at the next 256-byte boundary; P = 1 is
    la_chunk_fwd's walk and needs only the T factors."""
    lib = _lib.get()
    for (B, H, L, d) in ((1, 1, 640, 64), (2, 3, 1000, 128), (1, 4, 65536, 128)):
        nc = -(-L // 64)
        for mode in (0, 1, 2, 3):
            t = B * H * nc * TSOLVE_BYTES if mode in (1, 2) else 0
            assert seg_ws(lib, 1, B, H, L, d, mode) == (OK, t)
            for P in (2, 5, nc):
                want = -(-t // 256) * 256 + 3 * B * H * P * d * d * 4
                assert seg_ws(lib, P, B, H, L, d, mode) == (OK, want)
    assert seg_ws(lib, 1, dtype=0) == (OK, 0)
    assert seg_ws(lib, 2, dtype=0)[0] == UNSUP
    assert seg_ws(lib, 11)[0] == SHAPE
    assert lib.la_chunk_segmented_workspace_bytes(1, 1, 640, 64, 64, 64, 2, 1, 2, None) == NULL


def test_segment_plan():
    """The automatic plan: the whole-sequence walk wherever (b, h, column
    tile) chains already occupy the 256 compute units or the sequence is
    short; segments for few long sequences; and la_chunk_fwd's workspace
    size follows the plan."""
    lib = _lib.get()
    assert plan(lib, 1, 32, 65536) == 1            # 256 chains: every CU busy
    assert plan(lib, 8, 16, 4096, mode=0) == 1
    assert plan(lib, 4, 16, 8192, mode=1) == 1
    assert plan(lib, 1, 2, 256) == 1               # 4 chunks: too short to cut
    assert plan(lib, 1, 2, 256, dtype=0) == 1      # float inputs: never
    P = plan(lib, 1, 4, 65536)                     # one GPU's share of 32 heads over 8
    assert 4 <= P <= 64
    assert plan(lib, 1, 4, 65536) == P             # a function of the arguments only
    rc, n = ws_bytes(lib, B=1, H=4, L=65536, dk=128, dv=128)
    assert rc == OK and (OK, n) == seg_ws(lib, P, 1, 4, 65536, 128)
    for mode in (0, 1, 2, 3):
        for (B, H, L, d) in ((1, 1, 4096, 64), (1, 1, 100000, 128), (3, 1, 20000, 128)):
            P = plan(lib, B, H, L, d, mode)
            assert 1 <= P <= min(64, -(-L // 64))
            rc, n = ws_bytes(lib, B=B, H=H, L=L, dk=d, dv=d, mode=mode)
            assert (rc, n) == seg_ws(lib, P, B, H, L, d, mode)
    n = ctypes.c_int(0)
    assert lib.la_chunk_segments(1, 1, 64, 64, 64, 64, 2, 1, None) == NULL
    assert lib.la_chunk_segments(1, 1, 64, 96, 96, 64, 2, 1, ctypes.byref(n)) == UNSUP


def opts(flags=3, scale=0.0625, dskip=None, norm_w=None, eps=1e-6):
    return _lib.FusedOpts(flags, scale, dskip, norm_w, eps)


def fused(lib, flags=3, scale=0.0625, q=fake(0), k=fake(1), v=fake(2), la=fake(3), be=fake(4),
          s0=fake(5), out=fake(6), sf=fake(7), B=1, H=1, L=640, dk=64, dv=64, C=64, mode=2,
          dtype=1, ws=fake(8), wsb=P_BIG, dskip=None, norm_w=None, eps=1e-6):
    o = opts(flags, scale, dskip, norm_w, eps)
    return lib.la_chunk_fwd_fused(q, k, v, la, be, s0, out, sf, B, H, L, dk, dv, C, mode, dtype,
                                  ctypes.byref(o), ws, wsb, None)


def fused_ws(lib, flags, B=1, H=1, L=640, d=64, mode=2, dtype=1):
    n = ctypes.c_size_t(0)
    o = opts(flags, dskip=P if flags & 4 else None)
    rc = lib.la_chunk_fused_workspace_bytes(B, H, L, d, d, 64, mode, dtype, ctypes.byref(o),
                                            ctypes.byref(n))
    return rc, n.value


@pytest.mark.parametrize("kw,code", [
    (dict(flags=16), UNSUP), (dict(flags=-1), UNSUP), (dict(flags=1, scale=0.0), UNSUP),
    (dict(flags=3, scale=float("inf")), UNSUP), (dict(flags=2, dtype=0), UNSUP),
    (dict(flags=4, dtype=0, dskip=9 * P), UNSUP), (dict(flags=4), NULL),
    (dict(flags=8, eps=0.0), UNSUP), (dict(flags=8, eps=float("nan")), UNSUP),
    (dict(la=None), NULL), (dict(be=None, mode=1), NULL), (dict(wsb=1), WS),
    (dict(out=ctypes.c_void_p(P + 128)), ALIAS),
    (dict(flags=4, dskip=7 * P + 64), ALIAS),                # out overlaps D
    (dict(flags=8, norm_w=8 * P + 64), ALIAS),               # S_final overlaps the weight
])
def test_chunk_fwd_fused_rejects(kw, code):
    lib = _lib.get()
    assert fused(lib, **kw) == code
    assert lib.la_last_error().decode() != ""


def test_fused_flag_rules():
    """A zero scale only matters where a decay is activated; gate flags in
    LINEAR mode (no gates) reduce to no prologue -- float inputs then pass
    the flag check and stop at the NULL q they were given."""
    lib = _lib.get()
    assert fused(lib, flags=1, scale=0.0, mode=1, q=None) == NULL        # delta: no decay
    assert fused(lib, flags=1, scale=0.0, mode=0, dtype=0, q=None) == NULL
    assert fused(lib, flags=2, mode=0, dtype=0) == UNSUP                 # norm needs bf16
    # the norm weight is optional, and only counted when the norm is asked for
    assert fused(lib, flags=8, q=None) == NULL
    assert fused(lib, flags=4, dskip=9 * P, norm_w=6 * P, q=None) == NULL
    assert lib.la_chunk_fwd_fused(fake(0), fake(1), fake(2), fake(3), fake(4), None, fake(6),
                                  None, 1, 1, 64, 64, 64, 64, 2, 1, None, fake(8), P,
                                  None) != UNSUP


def test_fused_workspace_size():
    """la_chunk_fwd's workspace, then four float arrays of B*H*L tokens on
    256-byte boundaries; no prologue (flags 0, or gates in LINEAR mode) is
    la_chunk_fwd's size."""
    lib = _lib.get()
    for (B, H, L, d) in ((1, 1, 640, 64), (2, 3, 1000, 128), (1, 32, 65536, 128),
                         (1, 4, 65536, 128)):
        for mode in (0, 1, 2, 3):
            rc, base = ws_bytes(lib, B=B, H=H, L=L, dk=d, dv=d, mode=mode)
            assert rc == OK
            arr = -(-(B * H * L * 4) // 256) * 256
            for flags in (1, 2, 3):
                want = base if (flags == 1 and mode == 0) else (-(-base // 256) * 256 + 4 * arr)
                assert fused_ws(lib, flags, B, H, L, d, mode) == (OK, want)
                assert fused_ws(lib, flags | 12, B, H, L, d, mode) == (OK, want)
            assert fused_ws(lib, 4, B, H, L, d, mode) == (OK, base)       # epilogue only
            assert fused_ws(lib, 8, B, H, L, d, mode) == (OK, base)
            assert fused_ws(lib, 0, B, H, L, d, mode) == (OK, base)
    assert fused_ws(lib, 2, dtype=0)[0] == UNSUP
    assert fused_ws(lib, 0, dtype=0) == (OK, 0)
    o = opts(3)
    assert lib.la_chunk_fused_workspace_bytes(1, 1, 64, 64, 64, 64, 2, 1, ctypes.byref(o),
                                              None) == NULL


@pytest.mark.parametrize("kw,code", [
    (dict(flags=32), UNSUP), (dict(flags=1, scale=-1.0), UNSUP), (dict(q=None), NULL),
    (dict(la=None), NULL), (dict(S=ctypes.c_void_p(P + 64)), ALIAS), (dict(flags=4), NULL),
    (dict(flags=8, eps=-1.0), UNSUP), (dict(flags=4, dskip=6 * P + 8), ALIAS),
])
def test_decode_fused_rejects(kw, code):
    lib = _lib.get()
    a = dict(flags=3, scale=0.0625, q=fake(0), k=fake(1), v=fake(2), la=fake(3), be=fake(4),
             S=fake(5), out=fake(6), dskip=None, eps=1e-6)
    a.update(kw)
    o = opts(a["flags"], a["scale"], a["dskip"], None, a["eps"])
    rc = lib.la_decode_step_fused(a["q"], a["k"], a["v"], a["la"], a["be"], a["S"], a["out"],
                                  1, 1, 64, 64, 2, 1, ctypes.byref(o), None)
    assert rc == code
    assert lib.la_last_error().decode() != ""


def nc(lib, q=fake(0), k=fake(1), v=fake(2), s0=fake(5), out=fake(6), sf=fake(7), B=1, H=1,
       L=640, d=64, dtype=1, ws=fake(8), wsb=P_BIG):
    return lib.la_noncausal_fwd(q, k, v, s0, out, sf, B, H, L, d, d, dtype, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(out=None), NULL), (dict(dtype=0), UNSUP), (dict(d=96), UNSUP),
    (dict(L=0), SHAPE), (dict(ws=None), WS), (dict(wsb=16), WS),
    (dict(out=ctypes.c_void_p(P + 128)), ALIAS), (dict(sf=ctypes.c_void_p(6 * P + 4)), ALIAS),
    (dict(ws=ctypes.c_void_p(2 * P - 64)), ALIAS),
])
def test_noncausal_rejects(kw, code):
    lib = _lib.get()
    assert nc(lib, **kw) == code
    assert lib.la_last_error().decode() != ""


def test_noncausal_workspace_size():
    """Three state blocks per token block of K^T V (the partial states, an
    unused block and S); the block count, a function of the sizes only,
    gives about two workgroups per compute unit (one round), at most one per
    chunk and 64 per sequence."""
    lib = _lib.get()
    def blocks(B, H, L, d):
        n = ctypes.c_size_t(0)
        assert lib.la_noncausal_workspace_bytes(B, H, L, d, d, 1, ctypes.byref(n)) == OK
        unit = 3 * B * H * d * d * 4
        assert n.value % unit == 0
        return n.value // unit
    assert blocks(8, 16, 4096, 128) == 4
    assert blocks(1, 1, 65536, 128) == 64
    assert blocks(1, 2, 64, 64) == 1
    assert blocks(1, 1, 64 * 5 + 13, 128) == 6
    assert blocks(300, 16, 4096, 128) == 1
    assert lib.la_noncausal_workspace_bytes(1, 1, 64, 64, 64, 0, ctypes.byref(ctypes.c_size_t())) == UNSUP
    assert lib.la_noncausal_workspace_bytes(1, 1, 64, 64, 64, 1, None) == NULL


def test_library_resolves_every_symbol_at_load():
    """Loading with immediate binding fails on any undefined symbol (a lazy
    load only fails when the missing function is first called, on a GPU)."""
    import ctypes as ct
    ct.CDLL(_lib.LIB_PATH, mode=os.RTLD_NOW | os.RTLD_LOCAL)


# ------------------------------------------------------------- backward
def bwd(lib, q=fake(0), k=fake(1), v=fake(2), la=fake(3), be=fake(4), s0=fake(5), do=fake(6),
        dsf=fake(7), gq=fake(8), gk=fake(9), gv=fake(10), gla=fake(11), gbe=fake(12),
        gs0=fake(13), B=1, H=1, L=64, dk=64, dv=64, C=64, mode=2, dtype=1, ws=fake(14),
        wsb=P):
    return lib.la_chunk_bwd(q, k, v, la, be, s0, do, dsf, gq, gk, gv, gla, gbe, gs0,
                            B, H, L, dk, dv, C, mode, dtype, ws, wsb, None)


def bwd_ws_bytes(lib, B=1, H=1, L=64, d=64, mode=2, dtype=1):
    n = ctypes.c_size_t(12345)
    rc = lib.la_chunk_bwd_workspace_bytes(B, H, L, d, d, 64, mode, dtype, ctypes.byref(n))
    return rc, n.value


def expected_bwd_ws(B, H, L, d, erase):
    """Per chunk the entry state, the gradient of the leaving state and
    Q^T diag(gam) dO (d^2 floats each); T^T (C^2) with erase; per padded
    token g and P^T dO (d floats), and U and dR (d floats each) with erase;
    each array 256-byte aligned."""
    nc = -(-L // 64)
    pad = lambda n: -(-n * 4 // 256) * 256     # noqa: E731
    bh = B * H
    arrays = [bh * nc * 64, bh * nc * d * d, bh * nc * d * d, bh * nc * 64 * d, bh * nc * d * d]
    if erase:
        arrays += [bh * nc * 64 * 64]             # T^T, for both walks
    if erase:
        arrays += [bh * nc * 64 * d, bh * nc * 64 * d]
    return sum(pad(n) for n in arrays)


def test_bwd_workspace_size():
    lib = _lib.get()
    for mode in range(4):
        for (B, H, L, d) in ((1, 1, 64, 64), (2, 3, 200, 128), (1, 32, 65536, 128), (3, 1, 1, 64)):
            for dtype in (0, 1):
                rc, n = bwd_ws_bytes(lib, B, H, L, d, mode, dtype)
                assert rc == OK and n == expected_bwd_ws(B, H, L, d, mode in (1, 2))
    assert bwd_ws_bytes(lib, dtype=2)[0] == UNSUP
    assert bwd_ws_bytes(lib, d=96)[0] == UNSUP
    assert lib.la_chunk_bwd_workspace_bytes(1, 1, 64, 64, 64, 64, 2, 1, None) == NULL


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(do=None), NULL), (dict(gq=None), NULL), (dict(gk=None), NULL),
    (dict(gv=None), NULL), (dict(be=None), NULL), (dict(la=None), NULL),
    (dict(gla=None), NULL), (dict(gbe=None), NULL), (dict(gbe=None, mode=1), NULL),
    (dict(gla=None, mode=3), NULL),
    (dict(B=0), SHAPE), (dict(L=0), SHAPE), (dict(dk=64, dv=128), UNSUP), (dict(C=32), UNSUP),
    (dict(dtype=2), UNSUP), (dict(mode=4), UNSUP),
    (dict(ws=None), WS), (dict(wsb=1000), WS), (dict(ws=ctypes.c_void_p(15 * P + 8)), WS),
    (dict(gq=ctypes.c_void_p(P + 64)), ALIAS),          # grad_q overlaps q
    (dict(gk=ctypes.c_void_p(9 * P + 64)), ALIAS),      # grad_k overlaps grad_q
    (dict(gs0=ctypes.c_void_p(7 * P)), ALIAS),          # grad_S0 is dS_final
    (dict(ws=ctypes.c_void_p(11 * P - 4096)), ALIAS),   # workspace overlaps grad_v
])
def test_chunk_bwd_rejects(kw, code):
    lib = _lib.get()
    assert bwd(lib, **kw) == code
    assert lib.la_last_error().decode() != ""


def test_chunk_bwd_unused_gradients_and_gates():
    """Gradients and gates a mode does not have may be NULL (or anything):
    linear mode with every gate pointer NULL passes validation and stops at
    the alias of grad_q with q."""
    lib = _lib.get()
    assert bwd(lib, mode=0, la=None, be=None, gla=None, gbe=None,
               gq=ctypes.c_void_p(P + 64)) == ALIAS
    assert bwd(lib, mode=3, be=None, gbe=None, gq=ctypes.c_void_p(P + 64)) == ALIAS


def bwd_varlen(lib, cu=fake(15), N=2, H=1, T=128, **kw):
    a = dict(q=fake(0), k=fake(1), v=fake(2), la=fake(3), be=fake(4), s0=fake(5), do=fake(6),
             dsf=fake(7), gq=fake(8), gk=fake(9), gv=fake(10), gla=fake(11), gbe=fake(12),
             gs0=fake(13), dk=64, dv=64, C=64, mode=2, dtype=1, ws=fake(14), wsb=P)
    a.update(kw)
    return lib.la_chunk_bwd_varlen(a["q"], a["k"], a["v"], a["la"], a["be"], a["s0"], a["do"],
                                   a["dsf"], cu, a["gq"], a["gk"], a["gv"], a["gla"], a["gbe"],
                                   a["gs0"], N, H, T, a["dk"], a["dv"], a["C"], a["mode"],
                                   a["dtype"], a["ws"], a["wsb"], None)


def test_bwd_varlen_workspace_size():
    """Per-chunk arrays for H (ceil(T / C) + N) slots, whatever the offsets."""
    lib = _lib.get()
    for mode in range(4):
        for (N, H, T, d) in ((1, 1, 64, 64), (5, 3, 200, 128), (64, 32, 65536, 128), (3, 2, 0, 64)):
            n = ctypes.c_size_t(0)
            assert lib.la_chunk_bwd_varlen_workspace_bytes(N, H, T, d, d, 64, mode, 1,
                                                           ctypes.byref(n)) == OK
            slots = H * (-(-T // 64) + N)
            # the fixed-length formula with slots chunk-heads
            assert n.value == expected_bwd_ws(1, slots, 64, d, mode in (1, 2))
    n = ctypes.c_size_t(0)
    assert lib.la_chunk_bwd_varlen_workspace_bytes(1, 1, 64, 64, 64, 64, 2, 2,
                                                   ctypes.byref(n)) == UNSUP
    assert lib.la_chunk_bwd_varlen_workspace_bytes(1, 1, 64, 64, 64, 64, 2, 1, None) == NULL


@pytest.mark.parametrize("kw,code", [
    (dict(cu=None), NULL), (dict(q=None), NULL), (dict(gbe=None), NULL),
    (dict(gla=None, mode=3), NULL), (dict(N=0), SHAPE), (dict(T=-1), SHAPE),
    (dict(dk=96, dv=96), UNSUP), (dict(dtype=2), UNSUP), (dict(ws=None), WS),
    (dict(cu=ctypes.c_void_p(9 * P)), ALIAS),          # cu_seqlens inside grad_k
    (dict(gq=ctypes.c_void_p(15 * P)), ALIAS),         # grad_q is cu_seqlens
])
def test_chunk_bwd_varlen_rejects(kw, code):
    lib = _lib.get()
    assert bwd_varlen(lib, **kw) == code
    assert lib.la_last_error().decode() != ""


_Opts = _lib.FusedOpts


def test_bwd_fused_workspace_size():
    """The prologue's arrays (the inverse norms of q and k, the activated
    gates), each 256-byte aligned, then the backward's own workspace: the
    normalised rows are never stored."""
    lib = _lib.get()
    pad = lambda n: -(-n // 256) * 256     # noqa: E731
    for mode in range(4):
        for flags in (0, 1, 2, 3):
            for (B, H, L, d, dtype) in ((1, 1, 64, 64, 1), (2, 3, 200, 128, 0)):
                n = ctypes.c_size_t(0)
                o = _Opts(flags, 0.0625, None, None, 0.0)
                assert lib.la_chunk_bwd_fused_workspace_bytes(
                    B, H, L, d, d, 64, mode, dtype, ctypes.byref(o), ctypes.byref(n)) == OK
                rows = B * H * L
                extra = 0
                if flags & 2:
                    extra += 2 * pad(rows * 4)
                if flags & 1:
                    extra += pad(rows * 4) * ((mode in (2, 3)) + (mode in (1, 2)))
                assert n.value == extra + expected_bwd_ws(B, H, L, d, mode in (1, 2))


@pytest.mark.parametrize("flags,scale,eps,code", [
    (4, 0.0625, 0.0, NULL),            # LA_EPI_DSKIP without dskip (options checked first)
    (8, 0.0625, 1e-6, UNSUP),          # LA_EPI_OUT_NORM: no backward
    (1, 0.0, 0.0, UNSUP),              # gate_scale must be positive
    (16, 0.0625, 0.0, UNSUP),          # unknown flag
])
def test_chunk_bwd_fused_rejects(flags, scale, eps, code):
    lib = _lib.get()
    o = _Opts(flags, scale, None, None, eps)
    rc = lib.la_chunk_bwd_fused(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), fake(6),
                                fake(7), fake(8), fake(9), fake(10), fake(11), fake(12),
                                fake(13), 1, 1, 64, 64, 64, 64, 2, 1, ctypes.byref(o), fake(14),
                                P, None)
    assert rc == code
    assert lib.la_last_error().decode() != ""


@pytest.mark.parametrize("arg", [2, 5, 6, 7])      # v, S0, grad_out, grad_S_final
def test_chunk_bwd_fused_rejects_an_input_in_the_prologue_region(arg):
    """The fused backward's prologue writes the inverse norms of q and k and
    the gates at the start of the workspace before the backward proper reads v, grad_out,
    S0 and grad_S_final: any of them inside that region must be rejected
    (it would be overwritten first), not only inside the backward's own
    part of the workspace."""
    lib = _lib.get()
    o = _Opts(3, 0.0625, None, None, 0.0)
    n = ctypes.c_size_t(0)
    assert lib.la_chunk_bwd_fused_workspace_bytes(1, 1, 64, 64, 64, 64, 2, 1, ctypes.byref(o),
                                                  ctypes.byref(n)) == OK
    ws = 20 * P
    args = [fake(i) for i in range(14)]
    args[arg] = ctypes.c_void_p(ws + 256)               # inside the k norms (64 rows)
    rc = lib.la_chunk_bwd_fused(*args, 1, 1, 64, 64, 64, 64, 2, 1, ctypes.byref(o),
                                ctypes.c_void_p(ws), n.value, None)
    assert rc == ALIAS, lib.la_last_error().decode()


def test_chunk_fwd_noalloc_rejects_before_any_launch():
    """la_chunk_fwd_noalloc validates like la_chunk_fwd and rejects a call
    whose scratch would exceed the static array (the long-context workload
    needs 192 MiB of T factors, the array holds 128 MiB) before any HIP
    call; float inputs need no scratch at all."""
    lib = _lib.get()
    f = lib.la_chunk_fwd_noalloc
    args = [fake(i) for i in range(8)]
    assert f(*args, 1, 32, 65536, 128, 128, 64, 2, 1, None) == WS
    assert "scratch" in lib.la_last_error().decode()
    assert f(None, *args[1:], 1, 1, 64, 64, 64, 64, 2, 1, None) == NULL
    assert f(*args, 1, 1, 64, 96, 96, 64, 2, 1, None) == UNSUP
    a = list(args)
    a[6] = ctypes.c_void_p(P + 128)                     # out overlaps q
    assert f(*a, 1, 1, 64, 64, 64, 64, 2, 1, None) == ALIAS
    # the limit is the workspace la_chunk_fwd would need for the same call
    over = 0
    for (B, H, L) in ((8, 16, 4096), (1, 1, 64 * 21846), (4, 32, 8192), (1, 32, 65536)):
        n = ctypes.c_size_t(0)
        assert lib.la_chunk_workspace_bytes(B, H, L, 128, 128, 64, 2, 1, ctypes.byref(n)) == OK
        if n.value > 128 << 20:
            assert f(*args, B, H, L, 128, 128, 64, 2, 1, None) == WS
            over += 1
    assert over >= 2
