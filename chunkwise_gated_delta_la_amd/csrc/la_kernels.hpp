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
  bool bf16;
};

// Transient per-call workspace of the chunk forward (device memory).
//   W, U  [B*H*L, d]      element type of the inputs   (delta modes only)
//   Aqk   [B*H*L/C, C, C] element type of the inputs   lower triangle only
//   G     [B*H*L]         float: in-chunk cumulative log-decay (delta modes)
struct ChunkWorkspace {
  void* W;
  void* U;
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
  bool bf16;
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
