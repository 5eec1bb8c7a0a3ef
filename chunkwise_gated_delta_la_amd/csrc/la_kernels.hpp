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
  // Packed variable-length batch: cu_seqlens [B + 1] on the device, tokens
  // laid out [H, L, d] (L = total tokens, B = number of sequences); NULL for
  // the fixed-length layout [B, H, L, d].
  const int* cu = nullptr;
};

// Where the tokens of one (sequence, head) pair bh = s * H + h live, shared
// by the host (sizes) and the kernels (indexing).
struct SeqMap {
  const int* cu;  // NULL: fixed length
  int N, H, L;    // sequences, heads, tokens per sequence (fixed) or in total
  int C;
  // T-factor slots per head: one per chunk (fixed); for a packed batch
  // sequence s's chunk j takes slot floor(cu[s] / C) + s + j, unique for
  // nondecreasing offsets and below ceil(L / C) + N
  __host__ __device__ size_t slots_per_head() const {
    const size_t nc = ((size_t)L + C - 1) / C;
    return cu ? nc + (size_t)N : nc;
  }
};

inline SeqMap seq_map(const ChunkArgs& a) { return SeqMap{a.cu, a.B, a.H, a.L, a.C}; }

// T-factor slots of a whole call
inline size_t chunk_slots(const ChunkArgs& a) {
  const SeqMap m = seq_map(a);
  return (a.cu ? (size_t)a.H : (size_t)a.B * a.H) * m.slots_per_head();
}

struct SeqInfo {
  size_t row0;    // first token row (in units of d elements)
  int len;        // tokens
  size_t slot0;   // first T-factor slot
};

// Offsets are clamped into [0, L] and made nondecreasing, so malformed
// cu_seqlens can give wrong results but no out-of-bounds access.
__device__ inline SeqInfo seq_info(const SeqMap& m, int bh) {
  if (!m.cu) {
    const size_t nc = ((size_t)m.L + m.C - 1) / m.C;
    return SeqInfo{(size_t)bh * m.L, m.L, (size_t)bh * nc};
  }
  const int s = bh / m.H, h = bh % m.H;
  const int a = min(max(m.cu[s], 0), m.L);
  const int b = min(max(m.cu[s + 1], a), m.L);
  return SeqInfo{(size_t)h * m.L + a, b - a, (size_t)h * m.slots_per_head() + a / m.C + s};
}

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
