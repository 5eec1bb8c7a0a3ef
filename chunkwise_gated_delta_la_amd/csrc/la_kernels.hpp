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
  int pro = 0;            // fused prologue flags (kProGates, kProQKNorm)
  float gate_scale = 0.f;
  // Fused epilogue: o += D * v (D [H, dv], NULL: none), then with
  // out_norm the output normalised over dv: o / sqrt(mean(o^2) + norm_eps)
  // times norm_w [H, dv] (NULL: ones).
  const float* dskip = nullptr;
  bool out_norm = false;
  const float* norm_w = nullptr;
  float norm_eps = 0.f;
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
  // Segments per (b, h) sequence of the sequence-parallel forward (bf16,
  // fixed-length layout only); 1 walks each sequence whole.
  int P = 1;
  // Fused prologue (bf16 inputs): kProGates -- log_alpha and beta hold raw
  // scores a, b, and the op uses beta = sigmoid(b), log alpha =
  // -gate_scale softplus(a); kProQKNorm -- q and k are L2-normalised per
  // token inside the op.  0: the inputs are used as given.
  int pro = 0;
  float gate_scale = 0.f;
  // Fused epilogue: o += D * v per channel (D [H, dv], NULL: none); with
  // out_norm the output normalised over dv per token and head, o /
  // sqrt(mean(o^2) + norm_eps) times norm_w [H, dv] (NULL: ones), by a
  // separate pass over out (the chain kernels own 16 columns each).
  const float* dskip = nullptr;
  bool out_norm = false;
  const float* norm_w = nullptr;
  float norm_eps = 0.f;
};

enum : int { kProGates = 1, kProQKNorm = 2 };
constexpr float kQKNormEps = 1e-6f;   // x / sqrt(sum x^2 + eps)

// Per-token values the fused prologue writes for the chain kernels, token
// rows laid out like the gates ([B, H, L] or [H, T]): the gates the op uses
// and the logs of the inverse norms of q and k (zero without kProQKNorm).
struct ProArrays {
  float* beta;
  float* log_alpha;
  float* lq;   // log(1 / |q_t|)
  float* lk;   // log(1 / |k_t|)
};

// Mode the chain kernels run: with q, k normalisation the per-token norms
// ride in the decay tables, so the modes without decay use their decayed
// kernel with log alpha = 0.
inline int kernel_mode(const ChunkArgs& a) {
  if (!(a.pro & kProQKNorm)) return a.mode;
  return mode_erase(a.mode) ? kModeGatedDelta : kModeGatedLinear;
}

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
__host__ __device__ inline SeqInfo seq_info(const SeqMap& m, int bh) {
  if (!m.cu) {
    const size_t nc = ((size_t)m.L + m.C - 1) / m.C;
    return SeqInfo{(size_t)bh * m.L, m.L, (size_t)bh * nc};
  }
  const int s = bh / m.H, h = bh % m.H;
  const int a = min(max(m.cu[s], 0), m.L);
  const int b = min(max(m.cu[s + 1], a), m.L);
  return SeqInfo{(size_t)h * m.L + a, b - a, (size_t)h * m.slots_per_head() + a / m.C + s};
}

// ---- sequence-parallel forward
//
// The state after a run of chunks is affine in the state before it:
// S_end = M S_start + X, where X is the end state from a zero start and M
// (dk x dk) the product of the chunks' transitions (gam_C I - K^T diag(gam_C
// / gam) W per chunk).  A (b, h) sequence cut into P chunk-aligned segments
// is therefore run in three steps:
//   state pass   every segment p < P - 1 from its local start (S0 for p = 0,
//                else zero) to X_p; for p >= 1 also M_p, as the same chain
//                with V = 0 started from the identity (erase modes only: the
//                others have M_p = exp(sum of log alpha over p) I);
//   scan         S_in(0) = S0, S_in(1) = X_0, S_in(p+1) = M_p S_in(p) + X_p;
//   output pass  every segment from S_in(p), with its outputs; the last one
//                writes S_final.
// The passes have P times the parallelism of the whole-sequence walk for
// 1/P of its serial depth; they pay when (b, h, column tile) chains alone
// leave compute units idle.
enum : int { kPassWhole = 0, kPassState = 1, kPassOut = 2 };

// Chunk c0 of segment p of a sequence of nc chunks (balanced split; every
// segment is non-empty for P <= nc).
__host__ __device__ inline int seg_chunk0(int p, int P, int nc) {
  return (int)(((long long)p * nc) / P);
}

// What one row of chain workgroups walks (one per column tile): a whole
// (b, h) sequence, or one stream of a sequence-parallel pass.
struct StreamMap {
  SeqMap sm;
  const float* S0;   // [BH, dk, dv] or NULL (zero)
  float* S_final;    // [BH, dk, dv] or NULL
  int pass;          // kPassWhole, kPassState or kPassOut
  int P;             // segments per sequence (passes only)
  bool erase;        // state pass also runs transition streams
  size_t dd;         // elements of one state, dk * dv
  float* xs;         // [BH, P, dk, dv]  X_p
  float* ms;         // [BH, P, dk, dk]  M_p
  float* sin;        // [BH, P, dk, dv]  S_in(p)
  // streams per sequence
  __host__ __device__ int per_seq() const {
    if (pass == kPassWhole) return 1;
    if (pass == kPassOut) return P;
    return (P - 1) + (erase ? P - 2 : 0);
  }
};

struct StreamInfo {
  size_t row0;        // first token row
  int len;            // tokens
  size_t slot0;       // T-factor slot of the first chunk
  int head;           // h of the stream's (b, h) or (sequence, h)
  const float* s0;    // start state, NULL: zero
  float* sf;          // end state, NULL: not stored
  bool eye;           // start from the identity, V read as zero
};

__host__ __device__ inline StreamInfo stream_info(const StreamMap& m, int s) {
  if (m.pass == kPassWhole) {
    const SeqInfo si = seq_info(m.sm, s);
    return StreamInfo{si.row0, si.len, si.slot0, s % m.sm.H,
                      m.S0 ? m.S0 + (size_t)s * m.dd : nullptr,
                      m.S_final ? m.S_final + (size_t)s * m.dd : nullptr, false};
  }
  const int n = m.per_seq();
  const int bh = s / n, j = s % n;
  const int nc = (m.sm.L + m.sm.C - 1) / m.sm.C;
  int p = j;
  bool eye = false;
  if (m.pass == kPassState && j >= m.P - 1) {
    p = j - (m.P - 1) + 1;       // transition stream of segment p >= 1
    eye = true;
  }
  const int c0 = seg_chunk0(p, m.P, nc), c1 = seg_chunk0(p + 1, m.P, nc);
  const int t0 = c0 * m.sm.C, t1 = min(c1 * m.sm.C, m.sm.L);
  const size_t st = ((size_t)bh * m.P + p) * m.dd;
  StreamInfo si{(size_t)bh * m.sm.L + t0, t1 - t0, (size_t)bh * nc + c0, bh % m.sm.H, nullptr,
                nullptr, eye};
  if (m.pass == kPassOut) {
    si.s0 = m.sin + st;
    si.sf = (p == m.P - 1 && m.S_final) ? m.S_final + (size_t)bh * m.dd : nullptr;
  } else if (eye) {
    si.sf = m.ms + st;
  } else {
    si.s0 = (p == 0 && m.S0) ? m.S0 + (size_t)bh * m.dd : nullptr;
    si.sf = m.xs + st;
  }
  return si;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);
// The output normalisation of the fused epilogue over out [rows, dv]
// (la_chunk_pipe.hip).
hipError_t launch_out_norm(const ChunkArgs& a, hipStream_t st);
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
// Segments per sequence the sequence-parallel forward uses for this call
// (1: none), from the shapes alone (la_chunk_pipe.hip).
int plan_segments(const ChunkArgs& a);
// The fused prologue's per-token arrays inside the workspace (valid when
// a.pro != 0; la_chunk_pipe.hip).
ProArrays pro_arrays(const ChunkArgs& a);
// Non-causal form O = Q (S0 + K^T V), bf16, a.mode LINEAR (la_chunk_pipe.hip):
// its token blocks per sequence (a.P), its workspace, its launches.
int plan_sum_segments(const ChunkArgs& a);
size_t noncausal_workspace_bytes(const ChunkArgs& a);
hipError_t launch_noncausal(const ChunkArgs& a, hipStream_t st);
// With P > 1: the state pass, then the scan, before launch_chunk runs the
// output pass (la_chunk_pipe.hip).
hipError_t launch_chunk_state(const ChunkArgs& a, hipStream_t st);
hipError_t launch_seg_scan(const ChunkArgs& a, hipStream_t st);

}  // namespace la
