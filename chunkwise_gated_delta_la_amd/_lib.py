"""ctypes loader for liblachunk.so (the C ABI declared in include/la.h).

The shared library is built in-tree by ``csrc/build.py``.  There is no
fallback: if the library is missing or fails to load, every entry point
raises.
"""
import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblachunk.so")

LA_OK = 0
STATUS_NAMES = {0: "LA_OK", 1: "LA_ERR_NULL", 2: "LA_ERR_SHAPE", 3: "LA_ERR_UNSUPPORTED",
                4: "LA_ERR_ALIAS", 5: "LA_ERR_HIP", 6: "LA_ERR_WORKSPACE"}

_lock = threading.Lock()
_lib = None


class LAError(RuntimeError):
    """A non-OK status returned by the library, with its message."""

    def __init__(self, code, message):
        self.code = code
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {message}")


class FusedOpts(ctypes.Structure):
    """la_fused_opts_t of include/la.h."""
    _fields_ = [("flags", ctypes.c_int), ("gate_scale", ctypes.c_float),
                ("dskip", ctypes.c_void_p), ("norm_weight", ctypes.c_void_p),
                ("norm_eps", ctypes.c_float)]


def _declare(lib):
    vp, fp, i, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.la_chunk_fwd.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp,
                                 i, i, i, i, i, i, i, i, vp, sz, vp]
    lib.la_chunk_fwd.restype = i
    lib.la_chunk_fwd_noalloc.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp,
                                         i, i, i, i, i, i, i, i, vp]
    lib.la_chunk_fwd_noalloc.restype = i
    lib.la_chunk_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i, ctypes.POINTER(sz)]
    lib.la_chunk_workspace_bytes.restype = i
    lib.la_chunk_fwd_varlen.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, vp,
                                        i, i, i, i, i, i, i, i, vp, sz, vp]
    lib.la_chunk_fwd_varlen.restype = i
    lib.la_chunk_varlen_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i, ctypes.POINTER(sz)]
    lib.la_chunk_varlen_workspace_bytes.restype = i
    lib.la_chunk_fwd_segmented.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp,
                                           i, i, i, i, i, i, i, i, i, vp, sz, vp]
    lib.la_chunk_fwd_segmented.restype = i
    lib.la_chunk_segmented_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i, i,
                                                       ctypes.POINTER(sz)]
    lib.la_chunk_segmented_workspace_bytes.restype = i
    lib.la_chunk_segments.argtypes = [i, i, i, i, i, i, i, i, ctypes.POINTER(i)]
    lib.la_chunk_segments.restype = i
    lib.la_noncausal_fwd.argtypes = [vp, vp, vp, fp, vp, fp, i, i, i, i, i, i, vp, sz, vp]
    lib.la_noncausal_fwd.restype = i
    lib.la_noncausal_workspace_bytes.argtypes = [i, i, i, i, i, i, ctypes.POINTER(sz)]
    lib.la_noncausal_workspace_bytes.restype = i
    op = ctypes.POINTER(FusedOpts)
    lib.la_chunk_fwd_fused.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp,
                                       i, i, i, i, i, i, i, i, op, vp, sz, vp]
    lib.la_chunk_fwd_fused.restype = i
    lib.la_chunk_fused_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i, op,
                                                   ctypes.POINTER(sz)]
    lib.la_chunk_fused_workspace_bytes.restype = i
    lib.la_decode_step_fused.argtypes = [vp, vp, vp, fp, fp, fp, vp,
                                         i, i, i, i, i, i, op, vp]
    lib.la_decode_step_fused.restype = i
    lib.la_decode_step.argtypes = [vp, vp, vp, fp, fp, fp, vp,
                                   i, i, i, i, i, i, vp]
    lib.la_decode_step.restype = i
    lib.la_chunk_bwd.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, fp, fp, fp, fp, fp, fp,
                                 i, i, i, i, i, i, i, i, vp, sz, vp]
    lib.la_chunk_bwd.restype = i
    lib.la_chunk_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i, ctypes.POINTER(sz)]
    lib.la_chunk_bwd_workspace_bytes.restype = i
    lib.la_chunk_bwd_varlen.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, vp, fp, fp, fp, fp, fp,
                                        fp, i, i, i, i, i, i, i, i, vp, sz, vp]
    lib.la_chunk_bwd_varlen.restype = i
    lib.la_chunk_bwd_fused.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, fp, fp, fp, fp, fp, fp,
                                       i, i, i, i, i, i, i, i, op, vp, sz, vp]
    lib.la_chunk_bwd_fused.restype = i
    lib.la_chunk_bwd_fused_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i, op,
                                                       ctypes.POINTER(sz)]
    lib.la_chunk_bwd_fused_workspace_bytes.restype = i
    lib.la_chunk_bwd_varlen_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i,
                                                        ctypes.POINTER(sz)]
    lib.la_chunk_bwd_varlen_workspace_bytes.restype = i
    lib.la_last_error.argtypes = []
    lib.la_last_error.restype = ctypes.c_char_p
    lib.la_version.argtypes = []
    lib.la_version.restype = ctypes.c_char_p
    lib.la_profile_begin.argtypes = []
    lib.la_profile_begin.restype = i
    lib.la_profile_end.argtypes = [ctypes.POINTER(KernelTime), i, ctypes.POINTER(i)]
    lib.la_profile_end.restype = i
    return lib


class KernelTime(ctypes.Structure):
    """la_kernel_time_t"""
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int),
                ("total_ms", ctypes.c_double)]


def get():
    """The loaded library; raises RuntimeError if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with "
                    "`python chunkwise_gated_delta_la_amd/csrc/build.py` "
                    "(there is no fallback implementation)")
            _lib = _declare(ctypes.CDLL(LIB_PATH))
        return _lib


def check(rc):
    if rc != LA_OK:
        raise LAError(rc, get().la_last_error().decode())
