// Internal interface between the C-ABI host layer (la_api.hip) and the
// kernel translation units.  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace la {

enum : int { kModeLinear = 0, kModeDelta = 1, kModeGatedDelta = 2, kModeGatedLinear = 3 };

// The delta rule (beta, erase, the T factor) and the scalar decay (log
// alpha) are independent switches of the four modes.
__host__ __device__ constexpr bool mode_erase(int m) { return m == kModeDelta || m == kModeGatedDelta; }
__host__ __device__ constexpr bool mode_decay(int m) { return m == kModeGatedDelta || m == kModeGatedLinear; }

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
  void* workspace;  // chunk_workspace_bytes(*this) bytes, 256-byte aligned
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);
// Chunk forward: float inputs run one kernel (la_chunk.hip); bf16 inputs
// in the delta (erase) modes first solve T for every chunk (launch_tsolve,
// into the workspace), then run the chain kernel (la_chunk_pipe.hip).
size_t chunk_workspace_bytes(const ChunkArgs& a);
bool chunk_needs_tsolve(const ChunkArgs& a);
hipError_t launch_tsolve(const ChunkArgs& a, hipStream_t st);       // la_chunk_pipe.hip
hipError_t launch_chunk(const ChunkArgs& a, hipStream_t st);        // dispatcher
hipError_t launch_chunk_seq(const ChunkArgs& a, hipStream_t st);    // la_chunk.hip
hipError_t launch_chunk_pipe(const ChunkArgs& a, hipStream_t st);   // la_chunk_pipe.hip
size_t chunk_pipe_workspace_bytes(const ChunkArgs& a);               // la_chunk_pipe.hip

}  // namespace la
