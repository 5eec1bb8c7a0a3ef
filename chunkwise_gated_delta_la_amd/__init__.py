"""chunkwise_gated_delta_la_amd -- chunkwise gated-delta linear attention on
AMD Instinct MI355X (gfx950).

A thin Python binding over liblachunk.so, whose C ABI is declared in
``include/la.h``.  Every step of the computation runs in the library's HIP
kernels; this package only checks and marshals torch tensors (device
memory) and passes torch's current HIP stream.

    out, S_final = chunk_fwd(q, k, v, log_alpha, beta, S0, mode="gated_delta")
    out, S_final = chunk_fwd_varlen(q, k, v, log_alpha, beta, S0, cu_seqlens)  # packed
    out, S_final = chunk_fwd(q, k, v, log_alpha, beta, S0, segments=8)  # sequence-parallel
    out = decode_step(q, k, v, log_alpha, beta, S, mode="gated_delta")  # S in place
    out, S = noncausal_fwd(q, k, v, S0)                                   # O = Q (S0 + K^T V)
"""
from ._lib import LAError, LIB_PATH  # noqa: F401
from .api import (MODES, chunk_fwd, chunk_fwd_noalloc, chunk_fwd_varlen, chunk_segments,  # noqa: F401
                  chunk_varlen_workspace_bytes, chunk_workspace_bytes, decode_step,
                  kernel_timer, noncausal_fwd, version, chunk_bwd,
                  chunk_bwd_workspace_bytes, chunk_bwd_varlen,
                  chunk_bwd_varlen_workspace_bytes)
