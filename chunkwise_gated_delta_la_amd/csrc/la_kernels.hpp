// Internal interface between the C-ABI host layer (la_api.hip) and the
// kernel translation units.  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace la {

enum : int { kModeLinear = 0, kModeDelta = 1, kModeGatedDelta = 2 };

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* log_alpha;
  const float* beta;
  float* S;
  void* out;
  int B, H, dk, dv, mode;
  bool in_bf16;   // q, k, v are bf16 (else float)
  bool out_bf16;  // out is bf16 (else float)
};

// Transient per-call workspace of the chunk forward (device memory).
//   W    [B*H*L, d]              input element type   (delta modes only)
//   U    [B*H*L, d]              float                (delta modes only)
//   Aqk  [B*H*L/C, P, C, C]      input element type; P = 2 planes (hi, lo)
//                                for bf16 inputs, 1 for float; only the
//                                32-column blocks on or below the diagonal
//                                are written
//   G    [B*H*L]                 float: in-chunk cumulative log-decay
//                                (delta modes only)
struct ChunkWorkspace {
  void* W;
  float* U;
  void* Aqk;
  float* G;
};

struct ChunkArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* log_alpha;
  const float* beta;
  const float* S0;
  void* out;
  float* S_final;
  int B, H, L, d, C, mode;
  bool in_bf16;   // q, k, v are bf16 (else float)
  bool out_bf16;  // out is bf16 (else float)
};

// Bytes of each workspace part for a call (0 when the mode does not use it).
struct WorkspaceSizes {
  size_t W, U, Aqk, G;
  size_t total() const { return W + U + Aqk + G; }
};
WorkspaceSizes chunk_workspace_sizes(const ChunkArgs& a);

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);
hipError_t launch_wy(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t st);
hipError_t launch_state(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t st);

}  // namespace la
