// Backward of the chunkwise forward: the gradients of every input for a
// scalar loss with upstream gradients dO (of the outputs) and dS_final (of
// the final state).
//
// The pages print no gradient formulas; they say that training runs the
// chunked form and keeps the state of every chunk for it ("FWP分块并行机制"
// in the hybrid-attention notes "混合注意力学习(1): 线性注意力"; train with
// the parallel form, infer with the recurrent one: "朴素线性注意力" in
// "【CS336】lecture4 线性注意力|Mamba|GDN|DSA").  The formulas below are the
// derivative of the forward's chunk step (the WY/UT form of
// "HouseHolder变换和WY表示" with the scalar decay of "Gated DeltaNet", same
// notes).  Per chunk, with S the state entering it, g the in-chunk cumsum of
// log alpha, gam = exp(g), f = exp(g_C - g), Gamma_ri = exp(g_r - g_i) for
// i <= r, P = (Q K^T) * M * Gamma, A = strict_lower(diag(beta) K K^T *
// Gamma), T = (I + A)^-1, R = diag(beta)(V - diag(gam) K S), U = T R (U = V
// without erase), O = diag(gam) Q S + P U, S' = gam_C S + K^T diag(f) U, and
// dS' the gradient of S':
//
//   dU  = P^T dO + diag(f) K dS'
//   dR  = T^T dU                          (erase modes; dV = diag(beta) dR,
//                                          else dV = dU)
//   dS  = gam_C dS' + Q^T diag(gam) dO - K^T diag(beta gam) dR
//
// is the only serial part (a reverse walk over chunks); everything else
// follows per chunk from S, dS', dO and the chunk's own inputs:
//
//   E   = (dO U^T) * M * Gamma,  dA = strict_lower(-dR U^T),
//   H   = dA * beta_r Gamma,     G  = H + H^T
//   dQ  = diag(gam) dO S^T + E K
//   dK  = diag(f) U dS'^T - diag(beta gam) dR S^T + E^T Q + G K
//   dbeta_r = V_r . dR_r - gam_r K_r . (dR S^T)_r + sum_i dA_ri (K K^T *
//             Gamma)_ri
//   dg  = rowsum(GG) - colsum(GG) + gam * (Q . dO S^T - beta K . dR S^T)
//         - f * (K . U dS'^T), GG = (dO U^T) * P + dA * A, plus at the last
//         row gam_C <dS', S> + sum_r f_r (K . U dS'^T)_r
//   dlog_alpha_i = sum over rows r >= i of the chunk of dg_r.
//
// Kernels (one call runs all four on one stream):
//   bwd_prep     per (b, h, chunk): g, T by forward substitution, and the
//                two dS-independent terms P^T dO and Q^T diag(gam) dO
//   bwd_states   per (b, h, 16 state columns): the forward walk, storing
//                the state entering each chunk and U
//   bwd_rev      per (b, h, 16 state columns): the reverse walk, storing dS'
//                of each chunk and dR, writing dv and dS0
//   bwd_grads    per (b, h, chunk): dq, dk, dbeta, dlog_alpha
// The walks keep their 16-column state (or state-gradient) tile in the MFMA
// accumulators of waves 0 and 1, each holding half of its rows; waves 2
// and 3 load the chain's operands two chunks ahead into registers and write
// them into a double buffer in LDS the step before their use, and wave 4
// writes out what the chain hands it through LDS, so each chunk step has
// one barrier.
//
// A ragged last chunk is padded with rows that change nothing: q, k, v, dO
// and beta read as zero and log alpha as zero, so the padded rows of T are
// identity rows, their U, dU and dR are zero, and the last row's g is the
// chunk's total decay.  Their gradients are not stored.
//
// Precision: float inputs run float MFMAs throughout; bf16 inputs are exact
// bf16 MFMA operands, and every float operand (states, U, dR, scores, T) is
// split into bf16 hi + lo parts (about 16 bits).  Gradients are float32.
#include "la_device.hpp"
#include "la_kernels.hpp"
#include "la_bwd.hpp"

#include <type_traits>

namespace la {
namespace {

constexpr int C = 64;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int LDC = C + 4;     // row pitch of float C x C tiles in LDS
constexpr int LDX = 20;        // row pitch of float 16-column tiles in LDS
// The walks: two chain waves (one per half of the state's rows), two waves
// loading the chain's operands into LDS, and one wave storing what the
// chain hands over (no wave has loads and stores in flight together: they
// share one counter, and a wait for a load would wait for every store
// issued before it).  The fifth wave shares a SIMD with a chain half; its
// work per step is light.
constexpr int kWalkChain = 2 * kWave;
constexpr int kStatesLoad = 2 * kWave;         // loading threads of the forward walk
constexpr int kRevLoad = 2 * kWave;            // and of the reverse walk
constexpr int kStatesThreads = kWalkChain + kStatesLoad + kWave;
constexpr int kRevThreads = kWalkChain + kRevLoad + kWave;

// Per-chunk arrays are indexed by the chunk's slot: bh * NC + c for the
// fixed-length layout, the forward's packed-batch slots (SeqMap) otherwise
// (shapes below are the fixed-length ones).
struct BwdWs {
  float* g;     // [BH, NC * C]     in-chunk cumsum of log alpha (padded rows: the total)
  float* Sent;  // [BH, NC, D, D]   state entering each chunk
  float* U;     // [BH, NC * C, D]  T R (erase modes)
  float* dSx;   // [BH, NC, D, D]   gradient of the state leaving each chunk
  float* dR;    // [BH, NC * C, D]  T^T dU (erase modes)
  float* X1;    // [BH, NC, D, C]   (P^T dO)^T: per chunk, column-major
  float* X2;    // [BH, NC, D, D]   (Q^T diag(gam) dO)^T: per chunk, column-major
  float* TT;    // [BH, NC, C, C]   T^T, in SplitMat form (erase modes)
  size_t nS;    // elements of Sent and dSx
  size_t nU;    // elements of U and dR
  size_t nT;    // elements of TT
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }


SeqMap seq_map(const BwdArgs& a) { return SeqMap{a.cu, a.B, a.H, a.L, C}; }

// Chunk slots of a call: one per chunk-head (fixed length), H (ceil(T / C)
// + N) for a packed batch.
size_t slots(const BwdArgs& a) {
  const size_t nc = ((size_t)a.L + C - 1) / C;
  return (a.cu || a.packed) ? (size_t)a.H * (nc + (size_t)a.B) : (size_t)a.B * a.H * nc;
}

// Bytes of the workspace; with ws != NULL also its arrays in a.workspace.
size_t carve(const BwdArgs& a, BwdWs* ws) {
  const size_t ns = slots(a), D = a.d;
  const bool erase = mode_erase(a.mode);
  const size_t n[8] = {ns * C,     ns * D * D, erase ? ns * C * D : 0, ns * D * D,
                       erase ? ns * C * D : 0, ns * C * D, ns * D * D, erase ? ns * C * C : 0};
  float* p[8];
  size_t off = 0;
  char* base = static_cast<char*>(a.workspace);
  for (int i = 0; i < 8; ++i) {
    p[i] = (base && n[i]) ? reinterpret_cast<float*>(base + off) : nullptr;
    off += align256(n[i] * sizeof(float));
  }
  if (ws) *ws = BwdWs{p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], n[1], n[2], n[7]};
  return off;
}

// The chunk a parallel kernel's workgroup `item` (a slot) covers: its first
// token row and row count; false for a packed-batch slot no chunk maps to.
__device__ __forceinline__ bool chunk_of_slot(const SeqMap& sm, size_t item, size_t& row0,
                                              int& nrows) {
  if (!sm.cu) {
    const int NC = (sm.L + C - 1) / C;
    const size_t bh = item / NC;
    const int c = (int)(item % NC);
    row0 = bh * sm.L + (size_t)c * C;
    nrows = min(C, sm.L - c * C);
    return true;
  }
  const size_t sph = sm.slots_per_head();
  const int h = (int)(item / sph), j = (int)(item % sph);
  auto start = [&](int s) { return min(max(sm.cu[s], 0), sm.L); };
  auto first_slot = [&](int s) { return start(s) / C + s; };
  if (first_slot(0) > j) return false;
  int lo = 0, hi = sm.N - 1;      // the last sequence whose first slot is <= j
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (first_slot(mid) <= j) lo = mid;
    else hi = mid - 1;
  }
  const int a = start(lo), len = min(max(sm.cu[lo + 1], a), sm.L) - a;
  const int c = j - first_slot(lo);
  if (c * C >= len) return false;
  row0 = (size_t)h * sm.L + a + (size_t)c * C;
  nrows = min(C, len - c * C);
  return true;
}

template <typename T>
__device__ __forceinline__ Frag<T> frag_zero() {
  Frag<T> f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f.set(j, 0.f);
  return f;
}

// Operand row `r` of a chunk's token rows (row pitch D) in global memory;
// rows at or past nrows read as zero.
template <typename T, int D>
__device__ __forceinline__ Frag<T> chunk_row(const T* base, int r, int nrows, int c0, int g) {
  const Frag<T> f = frag_row(base + (size_t)min(r, nrows - 1) * D + c0, g);
  return r < nrows ? f : frag_zero<T>();
}

// Operand column `col` of a chunk's token rows over the 32-deep block at
// row k0: 8 values base[(k0 + kidx(g, j)) * D + col], zero past nrows.
template <typename T, int D>
__device__ __forceinline__ Frag<T> chunk_col(const T* base, int k0, int col, int nrows, int g) {
  Frag<T> f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = k0 + kidx(g, j);
    const T x = base[(size_t)min(r, nrows - 1) * D + col];
    f.v[j] = r < nrows ? x : T(0.f);
  }
  return f;
}

// Split operand from 8 float values (slot order), two instructions per
// value for bf16 (frag2_pack).
template <typename T>
__device__ __forceinline__ Frag2<T> frag2_of(const float (&x)[8]) {
  if constexpr (IsBf16<T>::value) {
    return frag2_pack(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
  } else {
    Frag2<T> f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f.set(j, x[j]);
    return f;
  }
}

// Split operand from a float row p[kidx(g, j)].
template <typename T>
__device__ __forceinline__ Frag2<T> frag2_rowx(const float* p, int g) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p + 4 * g);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 16 + 4 * g);
  const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return frag2_of<T>(x);
}

// Split operand gathered from a float column: p[kidx(g, j) * ld].
template <typename T>
__device__ __forceinline__ Frag2<T> frag2_col(const float* p, int ld, int g) {
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = p[kidx(g, j) * ld];
  return frag2_of<T>(x);
}

// A float matrix the walks hand to the gradient kernel, in the form that
// kernel's MFMAs take it: float32 for float inputs; for bf16 inputs two
// bf16 planes, hi = bf16(x) and lo = bf16(x - hi) (x to about 16 bits), so
// the gradient kernel loads split operands without converting.  Either form
// fills the same bytes of the workspace.
template <typename T>
struct SplitMat;

template <>
struct SplitMat<float> {
  float* p;
  __device__ static SplitMat make(float* region, size_t) { return SplitMat{region}; }
  __device__ __forceinline__ void put(size_t i, float x) const { p[i] = x; }
  __device__ __forceinline__ float get(size_t i) const { return p[i]; }
  __device__ __forceinline__ Frag2<float> row(size_t i, int g) const {
    Frag2<float> f;
    f.hi = frag_row(p + i, g);
    return f;
  }
  // x[0..7] to elements i .. i + 7 (i a multiple of 8)
  __device__ __forceinline__ void put8(size_t i, const float (&x)[8]) const {
    *reinterpret_cast<f32x4*>(p + i) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(p + i + 4) = f32x4{x[4], x[5], x[6], x[7]};
  }
};

template <>
struct SplitMat<__bf16> {
  __bf16* p;
  size_t plane;   // the lo plane starts plane elements after the hi plane
  __device__ static SplitMat make(float* region, size_t n) {
    return SplitMat{reinterpret_cast<__bf16*>(region), n};
  }
  __device__ __forceinline__ void put(size_t i, float x) const {
    const __bf16 h = (__bf16)x;
    p[i] = h;
    p[plane + i] = (__bf16)(x - (float)h);
  }
  __device__ __forceinline__ float get(size_t i) const {
    return (float)p[i] + (float)p[plane + i];
  }
  __device__ __forceinline__ Frag2<__bf16> row(size_t i, int g) const {
    Frag2<__bf16> f;
    f.hi = frag_row(p + i, g);
    f.lo = frag_row(p + plane + i, g);
    return f;
  }
  __device__ __forceinline__ void put8(size_t i, const float (&x)[8]) const {
    const Frag2<__bf16> f = frag2_pack(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
    *reinterpret_cast<u32x4*>(p + i) = __builtin_bit_cast(u32x4, f.hi.v);
    *reinterpret_cast<u32x4*>(p + plane + i) = __builtin_bit_cast(u32x4, f.lo.v);
  }
};

// acc += a * b with a split and b exact
template <typename T>
__device__ __forceinline__ void mma_a2b(const Frag2<T>& a, const Frag<T>& b, f32x4& acc) {
  if constexpr (IsBf16<T>::value) mma(a.lo, b, acc);
  mma(a.hi, b, acc);
}

// A float tile of R rows x 16 columns handed from a walk's chain wave to
// its storing wave through LDS, kept transposed ([16][R + 4]) so that a
// chain lane writes its four rows of one accumulator tile with one 16-byte
// write; the storing wave then stores it to a workspace matrix (row pitch D,
// the tile's 16 columns) in that matrix's form, 8 columns per thread (NT
// threads, t < NT; a fixed trip count, so the compiler tracks the loads in
// flight across it instead of waiting for them at a loop head).
template <int R>
__device__ __forceinline__ void tile_put(float* X, const f32x4* acc, int g, int n) {
#pragma unroll
  for (int t = 0; t < R / 16; ++t)
    *reinterpret_cast<f32x4*>(X + n * (R + 4) + 16 * t + 4 * g) = acc[t];
}

template <typename T, int D, int R, int NT>
__device__ __forceinline__ void tile_flush(const float* X, const SplitMat<T>& M, size_t base,
                                           int t) {
  __builtin_assume(t >= 0 && t < NT);
#pragma unroll
  for (int i = 0; i < (2 * R + NT - 1) / NT; ++i) {
    const int p = t + i * NT;
    if (p >= 2 * R) break;
    const int r = p / 2, c0 = 8 * (p % 2);
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = X[(c0 + j) * (R + 4) + r];
    M.put8(base + (size_t)r * D + c0, x);
  }
}

// sum_j a_j b_j of two split operands (hi + lo each)
template <typename T>
__device__ __forceinline__ float frag_dot(const Frag2<T>& a, const Frag2<T>& b) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float x = to_f32(a.hi.v[j]), y = to_f32(b.hi.v[j]);
    if constexpr (IsBf16<T>::value) {
      x += to_f32(a.lo.v[j]);
      y += to_f32(b.lo.v[j]);
    }
    s = fmaf(x, y, s);
  }
  return s;
}

// Sum over the 16 lanes of a lane group (lanes with the same l / 16).
__device__ __forceinline__ float sum16(float x) {
  x += __shfl_xor(x, 8);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 1);
  return x;
}

__device__ __forceinline__ float sum64(float x) {
  x += __shfl_xor(x, 32);
  x += __shfl_xor(x, 16);
  return sum16(x);
}

// Block -> (head, 16-column tile), the tiles of one head on one XCD
// (workgroups are dealt to the 8 XCDs round-robin) when the head count
// allows it, so they share the head's rows through that XCD's L2.
__device__ __forceinline__ void tile_of_block(int b, int BH, int NCT, int& bh, int& ct) {
  if (BH % 8 == 0) {
    const int x = b % 8, s = b / 8;
    ct = s % NCT;
    bh = (s / NCT) * 8 + x;
  } else {
    bh = b / NCT;
    ct = b % NCT;
  }
}

// The K^T operand of a walk's state update (state tile tj, token block kb)
// from the row-major K tile in LDS (row pitch LD elements): lane (g, n)
// gets K[32 kb + kidx(g, j)][16 tj + n].  For bf16, two transposed reads
// (ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives
// element i % 4 of the 4-element runs addressed by lanes i / 4 + 4 j), lane
// k of group g addressing row 32 kb + 4 g + k / 4 (then 16 rows further) at
// the columns 16 tj + 4 (k % 4) .. + 3; for float, a strided column read.
typedef short bwd_s16x4 __attribute__((ext_vector_type(4)));
template <typename T, int LD>
__device__ __forceinline__ Frag<T> frag_kt(const T* Kt, int kb, int tj, int g, int n) {
  if constexpr (IsBf16<T>::value) {
    typedef __attribute__((address_space(3))) bwd_s16x4 lds_s16x4;
    const T* p = Kt + (32 * kb + 4 * g + (n >> 2)) * LD + 16 * tj + 4 * (n & 3);
    const bwd_s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
    const bwd_s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 16 * LD));
    Frag<T> f;
    f.v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
    return f;
  } else {
    return frag_col(Kt + 32 * kb * LD + 16 * tj + n, LD, g);
  }
}

// The chain operands of one chunk -- K rows, T (erase modes), 16 columns of
// V (forward walk), the decays (as exp(g) and exp(g_C - g)) and beta -- read
// by the NT threads of the loading waves in one batch (every load issued,
// at clamped indices, before the first LDS write), then written to one half
// of the walk's double buffer.  Rows past the end of the sequence are
// written as zero: the mask is applied when the loaded values go to LDS, a
// step after the loads, so no instruction touches a load's registers before
// then (a select right after the load would wait for it there).
//
// With TS, T (the forward walk) or T^T (the reverse walk) comes in SplitMat
// form: for bf16 its hi and lo planes, as the prep kernel wrote them, are
// staged as two bf16 [C][C + 8] tiles, the chain's split operands as they
// are; for float as the float tile.
//
// With NORM the K rows are the raw ones and each row's inverse norm goes
// into both decay tables (every product of the walks that reads a K row
// scales it by one of them); gam_C then comes from a slot of its own.
template <typename T, int D, bool ERASE, bool WITH_V, bool WITH_X, bool TS, int NT_,
          bool NORM = false>
struct ChunkStage {
  static constexpr int NT = NT_;
  static constexpr int PE = 16 / sizeof(T);
  static constexpr int LDK = D + PE;
  static constexpr int VPR = D / PE;
  static constexpr int NK = C * VPR;
  static constexpr int IK = (NK + NT - 1) / NT;
  static constexpr int NTV = C * C / 4;          // 16-byte vectors of T (either form)
  static constexpr bool kTPlanes = TS && IsBf16<T>::value;
  static constexpr int LDTT = C + 8;              // row pitch of the bf16 T planes
  static constexpr int IT = ERASE ? (NTV + NT - 1) / NT : 1;
  static constexpr int VV = 16 / PE;              // 16-byte vectors per 16-column row
  static constexpr int NV = C * VV;
  static constexpr int IV = WITH_V ? (NV + NT - 1) / NT : 1;
  // 16 columns of X1^T [D][C] and X2^T [D][D]: 16 rows of C / 4 and D / 4 vectors
  static constexpr int NX1 = 16 * C / 4, NX2 = 16 * D / 4;
  static constexpr int IX1 = WITH_X ? (NX1 + NT - 1) / NT : 1;
  static constexpr int IX2 = WITH_X ? (NX2 + NT - 1) / NT : 1;
  u32x4 kx[IK];
  f32x4 tx[IT];
  u32x4 vx[IV];
  f32x4 x1[IX1], x2[IX2];
  float gx, gcx, bx, rkx;
  int nr;                                          // valid rows of the loaded chunk

  __device__ __forceinline__ void load(const T* __restrict__ k, const T* __restrict__ v,
                                       const float* __restrict__ beta, const float* Tg,
                                       const float* gg, size_t row0, int nrows, int col0,
                                       int t, const float* X1g = nullptr,
                                       const float* X2g = nullptr, const T* Th = nullptr,
                                       const T* Tl = nullptr, const float* rk = nullptr) {
    nr = nrows;
    if constexpr (WITH_X) {
      // 16 columns (col0 ..) of the chunk's X1 [C, D] and X2 [D, D]
#pragma unroll
      for (int i = 0; i < IX1; ++i) {
        const int p = min(t + i * NT, NX1 - 1);
        x1[i] = *reinterpret_cast<const f32x4*>(X1g + (size_t)(col0 + p / (C / 4)) * C +
                                                4 * (p % (C / 4)));
      }
#pragma unroll
      for (int i = 0; i < IX2; ++i) {
        const int p = min(t + i * NT, NX2 - 1);
        x2[i] = *reinterpret_cast<const f32x4*>(X2g + (size_t)(col0 + p / (D / 4)) * D +
                                                4 * (p % (D / 4)));
      }
    }
#pragma unroll
    for (int i = 0; i < IK; ++i) {
      const int p = min(t + i * NT, NK - 1), r = p / VPR, cv = p % VPR;
      kx[i] = *reinterpret_cast<const u32x4*>(k + (row0 + min(r, nrows - 1)) * D + cv * PE);
    }
    if constexpr (ERASE) {
#pragma unroll
      for (int i = 0; i < IT; ++i) {
        const int p = min(t + i * NT, NTV - 1);
        if constexpr (kTPlanes) {
          // plane p / 512, row (p % 512) / 8, 8 elements from (p % 8) * 8
          const int pl = p / (NTV / 2), rem = p % (NTV / 2);
          const T* src = (pl ? Tl : Th) + (rem / 8) * C + 8 * (rem % 8);
          tx[i] = __builtin_bit_cast(f32x4, *reinterpret_cast<const u32x4*>(src));
        } else {
          const int r = p / (C / 4), cv = p % (C / 4);
          tx[i] = *reinterpret_cast<const f32x4*>(Tg + r * C + 4 * cv);
        }
      }
    }
    if constexpr (WITH_V) {
#pragma unroll
      for (int i = 0; i < IV; ++i) {
        const int p = min(t + i * NT, NV - 1), r = p / VV, cv = p % VV;
        vx[i] = *reinterpret_cast<const u32x4*>(v + (row0 + min(r, nrows - 1)) * D + col0 +
                                                cv * PE);
      }
    }
    const int tr = min(t, C - 1);
    gx = gg[tr];
    gcx = gg[C - 1];
    bx = 0.f;
    if constexpr (ERASE) bx = beta[row0 + min(tr, nrows - 1)];
    if constexpr (NORM) rkx = rk[row0 + min(tr, nrows - 1)];
  }

  __device__ __forceinline__ void store(T* Kb, float* Tb, float* Vb, float* gsb, float* fsb,
                                        float* bsb, int t, float* X1b = nullptr,
                                        float* X2b = nullptr, float* gcb = nullptr) const {
    __builtin_assume(t >= 0 && t < NT);
    const u32x4 z = u32x4{0u, 0u, 0u, 0u};
    if constexpr (WITH_X) {
#pragma unroll
      for (int i = 0; i < IX1; ++i) {
        const int p = t + i * NT;
        if (p < NX1)
          *reinterpret_cast<f32x4*>(X1b + (p / (C / 4)) * (C + 4) + 4 * (p % (C / 4))) = x1[i];
      }
#pragma unroll
      for (int i = 0; i < IX2; ++i) {
        const int p = t + i * NT;
        if (p < NX2)
          *reinterpret_cast<f32x4*>(X2b + (p / (D / 4)) * (D + 4) + 4 * (p % (D / 4))) = x2[i];
      }
    }
#pragma unroll
    for (int i = 0; i < IK; ++i) {
      const int p = t + i * NT;
      if (p < NK)
        *reinterpret_cast<u32x4*>(Kb + (p / VPR) * LDK + (p % VPR) * PE) =
            p / VPR < nr ? kx[i] : z;
    }
    if constexpr (ERASE) {
#pragma unroll
      for (int i = 0; i < IT; ++i) {
        const int p = t + i * NT;
        if (p < NTV) {
          if constexpr (kTPlanes) {
            const int pl = p / (NTV / 2), rem = p % (NTV / 2);
            T* dst = reinterpret_cast<T*>(Tb) + pl * C * LDTT + (rem / 8) * LDTT + 8 * (rem % 8);
            *reinterpret_cast<u32x4*>(dst) = __builtin_bit_cast(u32x4, tx[i]);
          } else {
            *reinterpret_cast<f32x4*>(Tb + (p / (C / 4)) * LDC + 4 * (p % (C / 4))) = tx[i];
          }
        }
      }
    }
    if constexpr (WITH_V) {
#pragma unroll
      for (int i = 0; i < IV; ++i) {
        const int p = t + i * NT;
        if (p < NV) {
          float* dst = Vb + (p / VV) * LDX + (p % VV) * PE;
          const u32x4 xv = p / VV < nr ? vx[i] : z;
          if constexpr (IsBf16<T>::value) {
            const bf16x8 x = __builtin_bit_cast(bf16x8, xv);
#pragma unroll
            for (int j = 0; j < 8; ++j) dst[j] = (float)x[j];
          } else {
            const f32x4 x = __builtin_bit_cast(f32x4, xv);
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[j] = x[j];
          }
        }
      }
    }
    if (t < C) {
      // the decays the chain needs per row: gam = exp(g) and f = exp(g_C - g)
      if constexpr (NORM) {
        gsb[t] = __expf(gx) * rkx;
        fsb[t] = __expf(gcx - gx) * rkx;
        if (t == 0) *gcb = __expf(gcx);
      } else {
        gsb[t] = __expf(gx);
        fsb[t] = __expf(gcx - gx);
      }
      bsb[t] = t < nr ? bx : 0.f;
    }
  }
};

// ---------------------------------------------------------------- prep
// Per chunk-head (parallel): g, T = (I + A)^-1 (erase modes) and the two
// terms of the reverse walk that do not depend on the state gradient,
// X1 = P^T dO [C, d] and X2 = Q^T diag(gam) dO [d, d].  P^T stays in LDS;
// Q and dO are staged transposed so that every operand is read along its
// contraction index.  With NORM, q and k are the raw rows and rq, rk their
// inverse norms: the scores and A take them as row and column factors, X2
// with gam.
template <typename T, int D, int MODE, bool NORM>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ dout,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    const float* __restrict__ rq, const float* __restrict__ rk, BwdWs ws, SeqMap sm) {
  constexpr bool kErase = mode_erase(MODE);
  constexpr bool kGated = mode_decay(MODE);
  constexpr int NKB = D / 32;
  constexpr int PE = 16 / sizeof(T);
  constexpr int LDT = C + PE;         // row pitch of the transposed tiles
  constexpr int VPR = D / PE;
  constexpr int NT16 = D / 16;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave, g = lane / 16, n = lane % 16;
  size_t row0;
  int nrows;
  if (!chunk_of_slot(sm, blockIdx.x, row0, nrows)) return;
  const size_t cid = blockIdx.x;
  const T* qc = q + row0 * D;
  const T* kc = k + row0 * D;

  __shared__ __attribute__((aligned(16))) float gs[C];
  __shared__ __attribute__((aligned(16))) float gam[C];
  __shared__ __attribute__((aligned(16))) float bs[C];
  __shared__ __attribute__((aligned(16))) float rqs[NORM ? C : 1];
  __shared__ __attribute__((aligned(16))) float rks[NORM ? C : 1];
  __shared__ __attribute__((aligned(16))) float Pt[C * LDC];
  __shared__ __attribute__((aligned(16))) float As[kErase ? C * LDC : 4];
  __shared__ __attribute__((aligned(16))) T QT[D * LDT];
  __shared__ __attribute__((aligned(16))) T OT[D * LDT];

  // Q and dO rows, transposed into LDS (rows past the end as zero): all
  // loads go out before the first write.  The row index runs fastest across
  // lanes, so a transposed write of one column touches consecutive LDS words.
  constexpr int NQV = 2 * C * VPR / kThreads;
  u32x4 qv[NQV];
#pragma unroll
  for (int i = 0; i < NQV; ++i) {
    const int p = tid + i * kThreads;
    const int m = p / (C * VPR), rem = p % (C * VPR), r = rem % C, c0 = (rem / C) * PE;
    const u32x4 x = *reinterpret_cast<const u32x4*>((m == 0 ? q : dout) +
                                                   (row0 + min(r, nrows - 1)) * D + c0);
    qv[i] = r < nrows ? x : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < NQV; ++i) {
    const int p = tid + i * kThreads;
    const int m = p / (C * VPR), rem = p % (C * VPR), r = rem % C, c0 = (rem / C) * PE;
    T* dst = (m == 0 ? QT : OT) + c0 * LDT + r;
    if constexpr (IsBf16<T>::value) {
      const bf16x8 x = __builtin_bit_cast(bf16x8, qv[i]);
#pragma unroll
      for (int j = 0; j < PE; ++j) dst[j * LDT] = x[j];
    } else {
      const f32x4 x = __builtin_bit_cast(f32x4, qv[i]);
#pragma unroll
      for (int j = 0; j < PE; ++j) dst[j * LDT] = x[j];
    }
  }
  if (wave == 0) {
    float la = 0.f, b = 0.f;
    if (lane < nrows) {
      if constexpr (kGated) la = log_alpha[row0 + lane];
      if constexpr (kErase) b = beta[row0 + lane];
    }
    const float gg = kGated ? wave_inclusive_scan(la) : 0.f;
    gs[lane] = gg;
    gam[lane] = kGated ? __expf(gg) : 1.f;
    bs[lane] = b;
    if constexpr (NORM) {
      // gam scales dO's rows for X2 = Q^T diag(gam) dO only: the q norms go with it
      const float a = lane < nrows ? rq[row0 + lane] : 0.f;
      rqs[lane] = a;
      rks[lane] = lane < nrows ? rk[row0 + lane] : 0.f;
      gam[lane] *= a;
    }
    ws.g[cid * C + lane] = gg;
  }
  __syncthreads();

  // wave w computes the tiles (ti, w): its Q (and K) rows of block w and
  // the K rows of every block load once, up front
  const int tj = wave;
  Frag<T> kr[4][NKB], qb[NKB], kb2[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    qb[kb] = chunk_row<T, D>(qc, 16 * tj + n, nrows, 32 * kb, g);
    if constexpr (kErase) kb2[kb] = chunk_row<T, D>(kc, 16 * tj + n, nrows, 32 * kb, g);
  }
#pragma unroll
  for (int ti = 0; ti < 4; ++ti)
    if (kErase || ti <= tj)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        kr[ti][kb] = chunk_row<T, D>(kc, 16 * ti + n, nrows, 32 * kb, g);
#pragma unroll
  for (int ti = 0; ti < 4; ++ti) {
    // P^T tile: rows i = 16 ti + 4 g + e (keys), columns r = 16 tj + n
    // (queries), nonzero for r >= i
    f32x4 acc = zero4();
    if (tj >= ti) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) mma(kr[ti][kb], qb[kb], acc);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * ti + 4 * g + e, r = 16 * tj + n;
      float x = 0.f;
      if (r >= i) x = acc[e] * (kGated ? __expf(gs[r] - gs[i]) : 1.f);
      if constexpr (NORM) x *= rks[i] * rqs[r];
      Pt[i * LDC + r] = x;
    }
    if constexpr (kErase) {
      // A tile: rows r = 16 ti + 4 g + e, columns i = 16 tj + n, i < r
      f32x4 a2 = zero4();
      if (ti >= tj) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) mma(kr[ti][kb], kb2[kb], a2);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * ti + 4 * g + e, i = 16 * tj + n;
        float x = 0.f;
        if (r > i) x = bs[r] * a2[e] * (kGated ? __expf(gs[r] - gs[i]) : 1.f);
        if constexpr (NORM) x *= rks[r] * rks[i];
        As[r * LDC + i] = x;
      }
    }
  }
  __syncthreads();

  if (kErase && wave == 0) {
    // T = (I + A)^-1: lane j solves column j,
    //   x_r = [r == j] - sum_{i < r} A_ri x_i
    float x[C];
#pragma unroll
    for (int r = 0; r < C; ++r) {
      float s0 = r == lane ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
      for (int i4 = 0; 4 * i4 < r; ++i4) {
        const f32x4 av = *reinterpret_cast<const f32x4*>(As + r * LDC + 4 * i4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * i4 + e;
          if (i < r) {
            if (i % 2 == 0) s0 = fmaf(-av[e], x[i], s0);
            else s1 = fmaf(-av[e], x[i], s1);
          }
        }
      }
      x[r] = s0 + s1;
    }
    // row `lane` of T^T, in SplitMat form: the walks' T and T^T operands
    const SplitMat<T> Tt = SplitMat<T>::make(ws.TT, ws.nT);
#pragma unroll
    for (int q8 = 0; q8 < C / 8; ++q8) {
      const float y[8] = {x[8 * q8], x[8 * q8 + 1], x[8 * q8 + 2], x[8 * q8 + 3],
                          x[8 * q8 + 4], x[8 * q8 + 5], x[8 * q8 + 6], x[8 * q8 + 7]};
      Tt.put8((cid * C + lane) * C + 8 * q8, y);
    }
    return;
  }

  // X1 tiles (rows i of P^T, columns j of dO): 4 x NT16; X2 tiles: NT16 x NT16,
  // over the waves not solving T, a column tile of dO per wave at a time (its
  // operand and the gam-scaled split of it serve 4 + NT16 tiles); both
  // stored transposed (per column), the layout the reverse walk stages 16
  // columns of
  const int w0 = kErase ? 1 : 0, nw = kWaves - w0;
  for (int ct = wave - w0; ct < NT16; ct += nw) {
    const int c0 = 16 * ct;
    Frag<T> bo[2];
    Frag2<T> bog[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bo[kb] = frag_row(OT + (c0 + n) * LDT + 32 * kb, g);
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = to_f32(bo[kb].v[j]) * gam[32 * kb + kidx(g, j)];
      bog[kb] = frag2_of<T>(x);
    }
    // transposed stores: this lane's four rows are contiguous
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        mma_a2b(frag2_rowx<T>(Pt + (16 * it + n) * LDC + 32 * kb, g), bo[kb], acc);
      *reinterpret_cast<f32x4*>(ws.X1 + (cid * D + c0 + n) * C + 16 * it + 4 * g) = acc;
    }
#pragma unroll
    for (int it = 0; it < NT16; ++it) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        mma_ab2(frag_row(QT + (16 * it + n) * LDT + 32 * kb, g), bog[kb], acc);
      *reinterpret_cast<f32x4*>(ws.X2 + (cid * D + c0 + n) * D + 16 * it + 4 * g) = acc;
    }
  }
}

// ------------------------------------------------------- forward walk
// Five waves, as in the reverse walk: waves 0 and 1 carry the state, each
// on half of its rows (dk), and form the whole K S (the other half's rows
// from the float tile of the state entering the chunk, which both hand to
// the storing wave), R and U = T R (T lower triangular: row tiles 0 and 1
// skip the block above the diagonal, exact zeros), then update only their
// rows; waves 2 and 3 stage the operands, wave 4 stores S and U.  With
// NORM, k is the raw rows and rk their inverse norms (in the decay tables).
template <typename T, int D, int MODE, bool NORM>
__global__ __launch_bounds__(kStatesThreads) void bwd_states_kernel(
    const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ beta,
    const float* __restrict__ rk, const float* __restrict__ S0, BwdWs ws, SeqMap sm, int BH) {
  constexpr bool kErase = mode_erase(MODE);
  constexpr bool kGated = mode_decay(MODE);
  constexpr int PE = 16 / sizeof(T);
  constexpr int LDK = D + PE;
  constexpr int NKT = D / 16, NKB = D / 32, NCT = D / 16;
  constexpr int HT = NKT / 2, HB = NKB / 2;      // of one chain half

  // bf16: T^T as its bf16 hi and lo planes [C][C + 8] (the prep kernel's
  // form; the chain reads T's rows as its columns)
  constexpr bool kTPlanes = IsBf16<T>::value;
  constexpr int LDTT = C + 8;
  constexpr int kTWords = kTPlanes ? C * LDTT : C * LDC;   // floats per buffer
  __shared__ __attribute__((aligned(16))) T Kb[2][C * LDK];
  __shared__ __attribute__((aligned(16))) float Tb[2][kErase ? kTWords : 4];
  __shared__ __attribute__((aligned(16))) float Vb[2][C * LDX];
  // the state entering chunk c in slot c % 3: written by the chain halves
  // at the end of step c - 1, read by the other half in step c, stored in
  // step c + 1
  __shared__ __attribute__((aligned(16))) float SxT[3][16 * (D + 4)];
  __shared__ __attribute__((aligned(16))) float UxT[2][kErase ? 16 * (C + 4) : 4];  // U
  __shared__ __attribute__((aligned(16))) float gsb[2][C];   // exp(g)
  __shared__ __attribute__((aligned(16))) float fsb[2][C];   // exp(g_C - g)
  __shared__ __attribute__((aligned(16))) float bsb[2][C];
  __shared__ float gcb[2];                                   // exp(g_C) (NORM)

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave, g = lane / 16, n = lane % 16;
  int bh, ct;
  tile_of_block(blockIdx.x, BH, NCT, bh, ct);
  const int col0 = 16 * ct;
  const SeqInfo si = seq_info(sm, bh);
  const int L = si.len;                        // tokens of this sequence
  const int NC = (L + C - 1) / C;
  if (NC == 0) return;                         // nothing to store
  constexpr bool kTab = kGated || NORM;        // the decay tables are not all ones

  // Waves 2 and 3 stage the chain's operands: chunk c's loads go out during
  // the step two before its use and land in LDS during the step before it
  // (the barriers wait for LDS traffic only, so the loads stay in flight).
  ChunkStage<T, D, kErase, true, false, true, kStatesLoad, NORM> st;
  constexpr int kStore = 2 + kStatesLoad / kWave;   // the storing wave
  const int tld = tid - kWalkChain;            // loading thread index
  auto load = [&](int c) {
    const int nrows = min(C, L - c * C);
    const size_t row0 = si.row0 + (size_t)c * C;
    const size_t cid = si.slot0 + c;
    const SplitMat<T> Tt = SplitMat<T>::make(ws.TT, ws.nT);
    const T* th = nullptr;
    const T* tl = nullptr;
    if constexpr (kTPlanes && kErase) {
      th = Tt.p + cid * C * C;
      tl = Tt.p + Tt.plane + cid * C * C;
    }
    st.load(k, v, beta, kErase && !kTPlanes ? ws.TT + cid * C * C : nullptr, ws.g + cid * C, row0,
            nrows, col0, tld, nullptr, nullptr, th, tl, rk);
  };
  auto store = [&](int b) {
    st.store(Kb[b], Tb[kErase ? b : 0], Vb[b], gsb[b], fsb[b], bsb[b], tld, nullptr, nullptr,
             &gcb[b]);
  };

  const int h = wave;                          // chain half (waves 0, 1)
  f32x4 S[HT];                                 // rows 16 (h HT + j) + 4 g + e
  if (wave < 2) {
    const size_t sb = (size_t)bh * D * D;
#pragma unroll
    for (int j = 0; j < HT; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        S[j][e] = S0 ? S0[sb + (size_t)(16 * (h * HT + j) + 4 * g + e) * D + col0 + n] : 0.f;
#pragma unroll
    for (int j = 0; j < HT; ++j)
      *reinterpret_cast<f32x4*>(&SxT[0][n * (D + 4) + 16 * (h * HT + j) + 4 * g]) = S[j];
  } else if (wave < kStore) {
    load(0);
    store(0);
    load(min(1, NC - 1));
  }
  __syncthreads();

  // each role runs its own loop (one barrier per chunk in all), so the
  // staging loads meet no other role's registers and are not waited for early
  if (wave >= 2 && wave < kStore) {
    for (int c = 0; c < NC; ++c) {
      if (c + 1 < NC) store((c & 1) ^ 1);
      load(min(c + 2, NC - 1));
      __syncthreads();
    }
    return;
  }
  if (wave == kStore) {
    // the state and U tiles of chunk c, handed over by the chain, go to the
    // workspace during the next step
    const SplitMat<T> Se = SplitMat<T>::make(ws.Sent, ws.nS);
    const SplitMat<T> Um = SplitMat<T>::make(ws.U, ws.nU);
    auto flush = [&](int c) {
      tile_flush<T, D, D, kWave>(SxT[c % 3], Se, (si.slot0 + c) * D * D + col0, lane);
      if constexpr (kErase)
        tile_flush<T, D, C, kWave>(UxT[c & 1], Um, (si.slot0 + c) * C * D + col0, lane);
    };
    for (int c = 0; c < NC; ++c) {
      if (c >= 1) flush(c - 1);
      __syncthreads();
    }
    flush(NC - 1);
    return;
  }
  for (int c = 0; c < NC; ++c) {
    const int b = c & 1;
    {
      const float* gmc = gsb[b];     // exp(g) (times the row's inverse norm with NORM)
      const float* fc = fsb[b];      // exp(g_C - g) (the same)
      const float gamC = kGated ? (NORM ? gcb[b] : gmc[C - 1]) : 1.f;
      // decay factors f of the rows 32 kb + 4 g + e (lo) and 32 kb + 16 + 4 g + e (hi)
      float flo[2][4], fhi[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(fc + 32 * kb + 4 * g);
        const f32x4 c2 = *reinterpret_cast<const f32x4*>(fc + 32 * kb + 16 + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          flo[kb][e] = kTab ? a[e] : 1.f;
          fhi[kb][e] = kTab ? c2[e] : 1.f;
        }
      }
      Frag2<T> bX[2];
      if constexpr (kErase) {
        // S split over dk: this half's rows from registers, the other's from
        // the tile it wrote at the end of the last step (register arrays
        // only ever indexed by compile-time values)
        Frag2<T> bS[NKB];
        const float* xo = SxT[c % 3] + n * (D + 4) + 4 * g;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          if (kb / HB == h) {
            bS[kb] = frag2_from_acc<T>(S[2 * (kb % HB)], S[2 * (kb % HB) + 1]);
          } else {
            bS[kb] = frag2_from_acc<T>(*reinterpret_cast<const f32x4*>(xo + 32 * kb),
                                       *reinterpret_cast<const f32x4*>(xo + 32 * kb + 16));
          }
        }
        f32x4 R[4];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
          f32x4 ks = zero4();
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
            mma_ab2(frag_row(&Kb[b][(16 * ti + n) * LDK + 32 * kb], g), bS[kb], ks);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * ti + 4 * g + e;
            const float gam = kTab ? gmc[r] : 1.f;
            R[ti][e] = bsb[b][r] * (Vb[b][r * LDX + n] - gam * ks[e]);
          }
        }
        const Frag2<T> bR[2] = {frag2_from_acc<T>(R[0], R[1]), frag2_from_acc<T>(R[2], R[3])};
        f32x4 U[4];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
          U[ti] = zero4();
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            if (kb > ti / 2) continue;      // T is zero above the diagonal blocks
            // row 16 ti + n of T, over columns 32 kb + kidx(g, j): a column of
            // the T^T tile, read transposed (bf16 planes) or strided (float)
            Frag2<T> at;
            if constexpr (kTPlanes) {
              const T* tp = reinterpret_cast<const T*>(Tb[b]);
              at.hi = frag_kt<T, LDTT>(tp, kb, ti, g, n);
              at.lo = frag_kt<T, LDTT>(tp + C * LDTT, kb, ti, g, n);
            } else {
              at = frag2_col<T>(&Tb[b][32 * kb * LDC + 16 * ti + n], LDC, g);
            }
            mma_a2b2(at, bR[kb], U[ti]);
          }
        }
        // each half hands over two of the four row tiles of U
#pragma unroll
        for (int t = 0; t < 2; ++t)
          *reinterpret_cast<f32x4*>(&UxT[b][n * (C + 4) + 16 * (2 * h + t) + 4 * g]) =
              h == 0 ? U[t] : U[2 + t];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          bX[kb] = frag2_from_acc_scaled<T>(U[2 * kb], U[2 * kb + 1], flo[kb], fhi[kb]);
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          f32x4 vlo, vhi;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            vlo[e] = Vb[b][(32 * kb + 4 * g + e) * LDX + n];
            vhi[e] = Vb[b][(32 * kb + 16 + 4 * g + e) * LDX + n];
          }
          bX[kb] = frag2_from_acc_scaled<T>(vlo, vhi, flo[kb], fhi[kb]);
        }
      }
      // S <- gam_C S + K^T diag(f) U, this half's rows
#pragma unroll
      for (int j = 0; j < HT; ++j) {
        const int tj = h * HT + j;
#pragma unroll
        for (int e = 0; e < 4; ++e) S[j][e] *= gamC;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) mma_ab2(frag_kt<T, LDK>(Kb[b], kb, tj, g, n), bX[kb], S[j]);
      }
      // this half's rows of the state entering the next chunk (after the last
      // chunk into a slot no one reads: no branch in the loop body)
#pragma unroll
      for (int j = 0; j < HT; ++j)
        *reinterpret_cast<f32x4*>(&SxT[(c + 1) % 3][n * (D + 4) + 16 * (h * HT + j) + 4 * g]) =
            S[j];
    }
    __syncthreads();
  }
}

// ------------------------------------------------------- reverse walk
// Five waves: waves 0 and 1 carry the chain, each on half of the state
// gradient's rows (dk); waves 2 and 3 stage the operands, wave 4 stores the
// results.
// Each chain half forms the whole dU = X1 + diag(f) K dS' and dR = T^T dU
// (dS' from its own rows in registers and the other half's from the float
// tile both hand to the storing wave) and updates only its rows of dS; the
// two never wait for each other inside a chunk.  T^T is upper triangular,
// so its row tiles 2 and 3 skip the 32-deep block below the diagonal (exact
// zeros: the sums are unchanged).  With NORM, k is the raw rows and rk
// their inverse norms (in the decay tables).
template <typename T, int D, int MODE, bool NORM>
__global__ __launch_bounds__(kRevThreads) void bwd_rev_kernel(
    const T* __restrict__ k, const float* __restrict__ beta, const float* __restrict__ rk,
    const float* __restrict__ dS_final, float* __restrict__ dv_out, float* __restrict__ dS0,
    BwdWs ws, SeqMap sm, int BH) {
  constexpr bool kErase = mode_erase(MODE);
  constexpr bool kGated = mode_decay(MODE);
  constexpr int PE = 16 / sizeof(T);
  constexpr int LDK = D + PE;
  constexpr int NKT = D / 16, NKB = D / 32, NCT = D / 16;
  constexpr int HT = NKT / 2, HB = NKB / 2;      // of one chain half

  constexpr bool kTPlanes = IsBf16<T>::value;
  constexpr int LDTT = C + 8;
  // T^T: bf16 hi and lo planes [C][C + 8] (bf16 inputs) or float [C][C + 4]
  constexpr int kTWords = kTPlanes ? C * LDTT : C * LDC;   // floats per buffer
  __shared__ __attribute__((aligned(16))) T Kb[2][C * LDK];
  __shared__ __attribute__((aligned(16))) float Tb[2][kErase ? kTWords : 4];
  // 16 columns of X1 = P^T dO and X2 = Q^T diag(gam) dO, transposed
  __shared__ __attribute__((aligned(16))) float X1[2][16 * (C + 4)];
  __shared__ __attribute__((aligned(16))) float X2[2][16 * (D + 4)];
  // dS' entering step s in slot s % 3: written by the chain halves at the end
  // of step s - 1, read by the other half in step s, stored in step s + 1
  __shared__ __attribute__((aligned(16))) float dSxT[3][16 * (D + 4)];
  __shared__ __attribute__((aligned(16))) float dRxT[2][kErase ? 16 * (C + 4) : 4];  // dR
  // dv (beta dR, or dU) handed over like dR where LDS allows (not float at
  // d = 128: the chain stores it itself there)
  constexpr bool kDvTile = IsBf16<T>::value || D == 64;
  __shared__ __attribute__((aligned(16))) float dvxT[2][kDvTile ? 16 * (C + 4) : 4];
  __shared__ __attribute__((aligned(16))) float gsb[2][C];   // exp(g)
  __shared__ __attribute__((aligned(16))) float fsb[2][C];   // exp(g_C - g)
  __shared__ __attribute__((aligned(16))) float bsb[2][C];
  __shared__ float gcb[2];                                   // exp(g_C) (NORM)
  constexpr bool kTab = kGated || NORM;        // the decay tables are not all ones

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave, g = lane / 16, n = lane % 16;
  int bh, ct;
  tile_of_block(blockIdx.x, BH, NCT, bh, ct);
  const int col0 = 16 * ct;
  const SeqInfo si = seq_info(sm, bh);
  const int L = si.len;                        // tokens of this sequence
  const int NC = (L + C - 1) / C;
  if (NC == 0) {
    // an empty sequence passes the state gradient through
    if (wave == 0 && dS0) {
      const size_t sb = (size_t)bh * D * D;
#pragma unroll
      for (int tj = 0; tj < NKT; ++tj)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const size_t o = sb + (size_t)(16 * tj + 4 * g + e) * D + col0 + n;
          dS0[o] = dS_final ? dS_final[o] : 0.f;
        }
    }
    return;
  }

  // Waves 2 and 3 stage the chain's operands of each chunk -- K, T, the
  // gates and the tile's 16 columns of X1 = P^T dO and X2 = Q^T diag(gam) dO
  // (formed in parallel beforehand) -- two chunks ahead, as in the forward
  // walk; wave 4 stores the results.
  ChunkStage<T, D, kErase, false, true, true, kRevLoad, NORM> st;
  constexpr int kStore = 2 + kRevLoad / kWave;     // the storing wave
  const int tld = tid - kWalkChain;            // loading thread index
  auto load = [&](int c) {
    const int nrows = min(C, L - c * C);
    const size_t row0 = si.row0 + (size_t)c * C;
    const size_t cid = si.slot0 + c;
    const SplitMat<T> Tt = SplitMat<T>::make(ws.TT, ws.nT);
    const T* th = nullptr;
    const T* tl = nullptr;
    if constexpr (kTPlanes && kErase) {
      th = Tt.p + cid * C * C;
      tl = Tt.p + Tt.plane + cid * C * C;
    }
    st.load(k, nullptr, beta, kErase && !kTPlanes ? ws.TT + cid * C * C : nullptr,
            ws.g + cid * C, row0, nrows, col0, tld, ws.X1 + cid * C * D,
            ws.X2 + cid * D * D, th, tl, rk);
  };
  auto store = [&](int b) {
    st.store(Kb[b], Tb[kErase ? b : 0], nullptr, gsb[b], fsb[b], bsb[b], tld, X1[b], X2[b],
             &gcb[b]);
  };

  const int h = wave;                          // chain half (waves 0, 1)
  f32x4 dS[HT];                                // rows 16 (h HT + j) + 4 g + e
  if (wave < 2) {
    const size_t sb = (size_t)bh * D * D;
#pragma unroll
    for (int j = 0; j < HT; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dS[j][e] = dS_final
                       ? dS_final[sb + (size_t)(16 * (h * HT + j) + 4 * g + e) * D + col0 + n]
                       : 0.f;
#pragma unroll
    for (int j = 0; j < HT; ++j)
      *reinterpret_cast<f32x4*>(&dSxT[0][n * (D + 4) + 16 * (h * HT + j) + 4 * g]) = dS[j];
  } else if (wave < kStore) {
    load(NC - 1);
    store(0);
    load(max(NC - 2, 0));
  }
  __syncthreads();
  if (wave >= 2 && wave < kStore) {
    for (int s = 0; s < NC; ++s) {
      if (s + 1 < NC) store((s & 1) ^ 1);
      load(max(NC - 3 - s, 0));
      __syncthreads();
    }
    return;
  }
  if (wave == kStore) {
    // dS' and dR of the chunk of step s, handed over by the chain, go to the
    // workspace during step s + 1
    const SplitMat<T> dSe = SplitMat<T>::make(ws.dSx, ws.nS);
    const SplitMat<T> dRm = SplitMat<T>::make(ws.dR, ws.nU);
    auto flush = [&](int s) {
      const int c = NC - 1 - s, b = s & 1;
      tile_flush<T, D, D, kWave>(dSxT[s % 3], dSe, (si.slot0 + c) * D * D + col0, lane);
      if constexpr (kErase)
        tile_flush<T, D, C, kWave>(dRxT[b], dRm, (si.slot0 + c) * C * D + col0, lane);
      if constexpr (kDvTile) {
        // dv rows of the chunk (those inside the sequence), 8 columns a thread
        const int nrows = min(C, L - c * C);
        float* dvc = dv_out + (si.row0 + (size_t)c * C) * D + col0;
#pragma unroll
        for (int i = 0; i < 2 * C / kWave; ++i) {
          const int p = lane + i * kWave;
          if (p >= 2 * C) break;
          const int r = p / 2, c0 = 8 * (p % 2);
          if (r < nrows) {
            float x[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = dvxT[b][(c0 + j) * (C + 4) + r];
            *reinterpret_cast<f32x4*>(dvc + (size_t)r * D + c0) = f32x4{x[0], x[1], x[2], x[3]};
            *reinterpret_cast<f32x4*>(dvc + (size_t)r * D + c0 + 4) =
                f32x4{x[4], x[5], x[6], x[7]};
          }
        }
      }
    };
    for (int s = 0; s < NC; ++s) {
      if (s >= 1) flush(s - 1);
      __syncthreads();
    }
    flush(NC - 1);
    return;
  }

  for (int s = 0; s < NC; ++s) {
    const int c = NC - 1 - s, b = s & 1;
    {
      const float* gmc = gsb[b];     // exp(g) (times the row's inverse norm with NORM)
      const float* fc = fsb[b];      // exp(g_C - g) (the same)
      const float gamC = kGated ? (NORM ? gcb[b] : gmc[C - 1]) : 1.f;
      const int nrows = min(C, L - c * C);
      const size_t row0 = si.row0 + (size_t)c * C;
      // dS' split over dk: this half's rows from registers, the other's from
      // the tile it wrote at the end of the last step (register arrays only
      // ever indexed by compile-time values)
      Frag2<T> bS[NKB];
      const float* xo = dSxT[s % 3] + n * (D + 4) + 4 * g;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        if (kb / HB == h) {
          bS[kb] = frag2_from_acc<T>(dS[2 * (kb % HB)], dS[2 * (kb % HB) + 1]);
        } else {
          bS[kb] = frag2_from_acc<T>(*reinterpret_cast<const f32x4*>(xo + 32 * kb),
                                     *reinterpret_cast<const f32x4*>(xo + 32 * kb + 16));
        }
      }
      // dU = P^T dO + diag(f) K dS'
      f32x4 dU[4];
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        f32x4 y = zero4();
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          mma_ab2(frag_row(&Kb[b][(16 * ti + n) * LDK + 32 * kb], g), bS[kb], y);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(&X1[b][n * (C + 4) + 16 * ti + 4 * g]);
        const f32x4 fr = *reinterpret_cast<const f32x4*>(fc + 16 * ti + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) dU[ti][e] = x1[e] + (kTab ? fr[e] : 1.f) * y[e];
      }
      float* dvo = dv_out + row0 * D + col0 + n;
      // each half hands over (or stores) two of the four row tiles of dv and dR
      auto hand = [&](float* X, const f32x4 (&v)[4]) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
          *reinterpret_cast<f32x4*>(X + n * (C + 4) + 16 * (2 * h + t) + 4 * g) =
              h == 0 ? v[t] : v[2 + t];
      };
      auto store_dv = [&](const f32x4 (&v)[4]) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * (2 * h + t) + 4 * g + e;
            if (r < nrows) dvo[(size_t)r * D] = h == 0 ? v[t][e] : v[2 + t][e];
          }
      };
      if constexpr (kErase) {
        const Frag2<T> bU[2] = {frag2_from_acc<T>(dU[0], dU[1]), frag2_from_acc<T>(dU[2], dU[3])};
        f32x4 dR[4];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
          dR[ti] = zero4();
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            if (kb < ti / 2) continue;      // T^T is zero below the diagonal blocks
            Frag2<T> at;
            if constexpr (kTPlanes) {
              const T* tp = reinterpret_cast<const T*>(Tb[b]) + (16 * ti + n) * LDTT + 32 * kb;
              at.hi = frag_row(tp, g);
              at.lo = frag_row(tp + C * LDTT, g);
            } else {
              at = frag2_rowx<T>(&Tb[b][(16 * ti + n) * LDC + 32 * kb], g);
            }
            mma_a2b2(at, bU[kb], dR[ti]);
          }
        }
        hand(dRxT[b], dR);
        f32x4 dvv[4];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
          const f32x4 br = *reinterpret_cast<const f32x4*>(&bsb[b][16 * ti + 4 * g]);
#pragma unroll
          for (int e = 0; e < 4; ++e) dvv[ti][e] = br[e] * dR[ti][e];
        }
        if constexpr (kDvTile) hand(dvxT[b], dvv);
        else store_dv(dvv);
        // dS <- gam_C dS' + Q^T diag(gam) dO - K^T diag(beta gam) dR, this
        // half's rows
        Frag2<T> bR[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          float slo[4], shi[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int rl = 32 * kb + 4 * g + e, rh = rl + 16;
            slo[e] = -bsb[b][rl] * (kTab ? gmc[rl] : 1.f);
            shi[e] = -bsb[b][rh] * (kTab ? gmc[rh] : 1.f);
          }
          bR[kb] = frag2_from_acc_scaled<T>(dR[2 * kb], dR[2 * kb + 1], slo, shi);
        }
#pragma unroll
        for (int j = 0; j < HT; ++j) {
          const int tj = h * HT + j;
          {
            const f32x4 x2 = *reinterpret_cast<const f32x4*>(&X2[b][n * (D + 4) + 16 * tj + 4 * g]);
#pragma unroll
            for (int e = 0; e < 4; ++e) dS[j][e] = gamC * dS[j][e] + x2[e];
          }
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            mma_ab2(frag_kt<T, LDK>(Kb[b], kb, tj, g, n), bR[kb], dS[j]);
        }
      } else {
        if constexpr (kDvTile) hand(dvxT[b], dU);
        else store_dv(dU);
#pragma unroll
        for (int j = 0; j < HT; ++j) {
          const int tj = h * HT + j;
          const f32x4 x2 = *reinterpret_cast<const f32x4*>(&X2[b][n * (D + 4) + 16 * tj + 4 * g]);
#pragma unroll
          for (int e = 0; e < 4; ++e) dS[j][e] = gamC * dS[j][e] + x2[e];
        }
      }
      // this half's rows of dS' entering the next step
#pragma unroll
      for (int j = 0; j < HT; ++j)
        *reinterpret_cast<f32x4*>(&dSxT[(s + 1) % 3][n * (D + 4) + 16 * (h * HT + j) + 4 * g]) =
            dS[j];
    }
    __syncthreads();
  }
  if (dS0) {
    const size_t sb = (size_t)bh * D * D;
#pragma unroll
    for (int j = 0; j < HT; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dS0[sb + (size_t)(16 * (h * HT + j) + 4 * g + e) * D + col0 + n] = dS[j][e];
  }
}

// ------------------------------------------------------ per-chunk grads
// The 10 lower-triangular 16 x 16 tiles of a C x C matrix.
__device__ __forceinline__ void lower_tile(int t, int& ti, int& tj) {
  ti = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
  tj = t - ti * (ti + 1) / 2;
}

// One column tile of the C x D phase, staged in LDS by all waves: the 16
// rows of S and dS' (B^T operands: hi and lo planes for bf16 inputs) and,
// with kQK, the 16 columns of K and Q (B operands of the products over the
// chunk, and the row dots; without it the kernel holds whole K and Q rows).
// Loaded into registers one tile ahead, stored after the barrier that ends
// the previous tile.
template <typename T, int D, bool kQK>
struct ColStage {
  static constexpr bool kSplit = IsBf16<T>::value;
  static constexpr int PE = 16 / sizeof(T);
  static constexpr int NP = kSplit ? 4 : 2;       // S hi, (S lo), dS hi, (dS lo)
  static constexpr int LDB = D + PE;              // row pitch of the S / dS' planes
  static constexpr int LDQ = 16 + PE;             // row pitch of the K / Q columns
  static constexpr int VPRD = D / PE;             // 16-byte vectors per state row
  static constexpr int NS = NP * 16 * VPRD;       // state vectors (1024)
  static constexpr int IS = NS / kThreads;
  static constexpr int VV = 16 / PE;              // vectors per 16-column token row
  static constexpr int NQ = kQK ? 2 * C * VV : 0;
  static constexpr int IQ = (NQ + kThreads - 1) / kThreads;
  u32x4 sx[IS], qx[IQ > 0 ? IQ : 1];

  __device__ __forceinline__ void load(const SplitMat<T>& Sm, const SplitMat<T>& dSm, size_t s0,
                                       const T* kc, const T* qc, int nrows, int cb0, int t) {
#pragma unroll
    for (int i = 0; i < IS; ++i) {
      const int p = t + i * kThreads;
      const int pl = p / (16 * VPRD), rem = p % (16 * VPRD);
      const size_t o = s0 + (size_t)(cb0 + rem / VPRD) * D + (rem % VPRD) * PE;
      const T* src;
      if constexpr (kSplit) {
        const SplitMat<T>& m = pl < 2 ? Sm : dSm;
        src = m.p + (pl & 1 ? m.plane : 0) + o;
      } else {
        src = (pl == 0 ? Sm.p : dSm.p) + o;
      }
      sx[i] = *reinterpret_cast<const u32x4*>(src);
    }
    const u32x4 z = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < IQ; ++i) {
      const int p = min(t + i * kThreads, NQ - 1);
      const int m = p / (C * VV), rem = p % (C * VV), r = rem / VV;
      const T* base = m == 0 ? kc : qc;
      const u32x4 x = *reinterpret_cast<const u32x4*>(base + (size_t)min(r, nrows - 1) * D +
                                                      cb0 + (rem % VV) * PE);
      qx[i] = r < nrows ? x : z;
    }
  }

  __device__ __forceinline__ void store(T* Sb, T* Kc, T* Qc, int t) const {
#pragma unroll
    for (int i = 0; i < IS; ++i) {
      const int p = t + i * kThreads;
      const int pl = p / (16 * VPRD), rem = p % (16 * VPRD);
      *reinterpret_cast<u32x4*>(Sb + (pl * 16 + rem / VPRD) * LDB + (rem % VPRD) * PE) = sx[i];
    }
#pragma unroll
    for (int i = 0; i < IQ; ++i) {
      const int p = t + i * kThreads;
      if (p < NQ) {
        const int m = p / (C * VV), rem = p % (C * VV);
        T* dst = m == 0 ? Kc : Qc;
        *reinterpret_cast<u32x4*>(dst + (rem / VV) * LDQ + (rem % VV) * PE) = qx[i];
      }
    }
  }
};

// With NORM, q and k are the raw rows and rq, rk their inverse norms: the
// scores and K K^T take them as row and column factors, E, E^T and G as
// factors over their contraction, the row dots as row factors; dq and dk
// are the gradients of the normalised rows.
template <typename T, int D, int MODE, bool NORM>
__global__ __launch_bounds__(kThreads) void bwd_grads_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ beta, const T* __restrict__ dout, const float* __restrict__ rq,
    const float* __restrict__ rk, float* __restrict__ dq, float* __restrict__ dk,
    float* __restrict__ dla, float* __restrict__ dbeta, BwdWs ws, SeqMap sm) {
  constexpr bool kErase = mode_erase(MODE);
  constexpr bool kGated = mode_decay(MODE);
  constexpr bool kSplit = IsBf16<T>::value;
  constexpr int NKB = D / 32, NCT = D / 16;
  // K and Q rows of the chunk staged in LDS once (rows of 256 bytes at
  // most), read by both product phases; wider rows (float, d = 128) go by
  // 16-column slices with each column tile
  constexpr bool kFull = D * (int)sizeof(T) <= 256;
  using CS = ColStage<T, D, !kFull>;
  constexpr int LDK = D + CS::PE;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave, g = lane / 16, n = lane % 16;
  size_t row0;
  int nrows;
  if (!chunk_of_slot(sm, blockIdx.x, row0, nrows)) return;
  const size_t cid = blockIdx.x;
  const size_t urow0 = cid * C;   // row of U, dR
  const T* qc = q + row0 * D;
  const T* kc = k + row0 * D;
  const T* vc = v + row0 * D;
  const T* dOc = dout + row0 * D;
  const SplitMat<T> Um = SplitMat<T>::make(ws.U, ws.nU);
  const SplitMat<T> dRm = SplitMat<T>::make(ws.dR, ws.nU);
  const SplitMat<T> Sm = SplitMat<T>::make(ws.Sent, ws.nS);
  const SplitMat<T> dSm = SplitMat<T>::make(ws.dSx, ws.nS);
  const size_t u0 = urow0 * D, s0 = cid * D * D;

  __shared__ __attribute__((aligned(16))) float gs[C];
  __shared__ __attribute__((aligned(16))) float gam[C];
  __shared__ __attribute__((aligned(16))) float fs[C];
  __shared__ __attribute__((aligned(16))) float bs[C];
  __shared__ __attribute__((aligned(16))) float rqs[NORM ? C : 1];
  __shared__ __attribute__((aligned(16))) float rks[NORM ? C : 1];
  // the C x C tiles E and H live until each wave holds its fragments of
  // them; the column-tile staging reuses their bytes after that
  constexpr int kEH = (kErase ? 2 : 1) * C * LDC * (int)sizeof(float);
  constexpr int kStage =
      (CS::NP * 16 * CS::LDB + (kFull ? 0 : 2 * C * CS::LDQ)) * (int)sizeof(T);
  __shared__ __attribute__((aligned(16))) float pool[(kEH > kStage ? kEH : kStage) / 4];
  __shared__ __attribute__((aligned(16))) T KQ[kFull ? 2 * C * LDK : 8];
  float* const Em = pool;
  float* const Hm = pool + C * LDC;
  T* const Sb = reinterpret_cast<T*>(pool);
  T* const Kcs = Sb + CS::NP * 16 * CS::LDB;
  T* const Qcs = Kcs + C * CS::LDQ;
  T* const Kl = KQ;
  T* const Ql = KQ + C * LDK;
  __shared__ float dgam[C], dfv[C], vdr[C];
  // per-tile partial sums, added in a fixed order (deterministic results):
  // row sums of GG and of dA * (K K^T * Gamma) by column tile, column sums
  // of GG by row tile
  __shared__ float rsP[3][4][C];   // [0]: GG rows, [1]: dbeta rows, [2]: GG columns
  __shared__ float red[kWaves];

  // K and Q rows (zero past nrows), then the first column tile's loads
  constexpr int VR = D * (int)sizeof(T) / 16;      // 16-byte vectors per row
  constexpr int IK = kFull ? 2 * C * VR / kThreads : 0;
  u32x4 kq[IK > 0 ? IK : 1];
#pragma unroll
  for (int i = 0; i < IK; ++i) {
    const int p = tid + i * kThreads, m = p / (C * VR), r = (p / VR) % C, c = p % VR;
    const u32x4 x = *reinterpret_cast<const u32x4*>((m == 0 ? kc : qc) +
                                                   (size_t)min(r, nrows - 1) * D + c * CS::PE);
    kq[i] = r < nrows ? x : u32x4{0u, 0u, 0u, 0u};
  }
  CS st;
  st.load(Sm, dSm, s0, kc, qc, nrows, 0, tid);

  for (int p = tid; p < C * LDC; p += kThreads) {
    Em[p] = 0.f;
    if constexpr (kErase) Hm[p] = 0.f;
  }
  if (tid < C) {
    const float gg = ws.g[cid * C + tid];
    gs[tid] = gg;
    gam[tid] = kGated ? __expf(gg) : 1.f;
    bs[tid] = (kErase && tid < nrows) ? beta[row0 + tid] : 0.f;
    if constexpr (NORM) {
      rqs[tid] = tid < nrows ? rq[row0 + tid] : 0.f;
      rks[tid] = tid < nrows ? rk[row0 + tid] : 0.f;
    }
  }
#pragma unroll
  for (int i = 0; i < IK; ++i) {
    const int p = tid + i * kThreads, m = p / (C * VR), r = (p / VR) % C, c = p % VR;
    *reinterpret_cast<u32x4*>((m == 0 ? Kl : Ql) + r * LDK + c * CS::PE) = kq[i];
  }
  {
    float* part = &rsP[0][0][0];
    for (int p = tid; p < 3 * 4 * C; p += kThreads) part[p] = 0.f;   // rsP, dbP, csP
  }
  if constexpr (kErase) {
    // V_r . dR_r: four threads per row
    const int r = tid / 4, q4 = tid % 4;
    constexpr int W = D / 4;
    float x = 0.f;
    if (r < nrows) {
#pragma unroll
      for (int j = 0; j < W; ++j) {
        const int cc = q4 * W + j;
        x += to_f32(vc[(size_t)r * D + cc]) * dRm.get(u0 + (size_t)r * D + cc);
      }
    }
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    if (q4 == 0) vdr[r] = x;
  }
  __syncthreads();
  if (tid < C) fs[tid] = kGated ? __expf(gs[C - 1] - gs[tid]) : 1.f;

  // C x C products on the lower tiles: scores, dO U^T, and (erase) K K^T,
  // dR U^T; GG = (dO U^T) * P + dA * A goes straight into its per-tile row
  // and column sums.  Wave w owns the row block w (tiles (w, 0) .. (w, w)):
  // its dO and dR (or V) rows load once and stay as operands of the C x D
  // products below.
  const int ti = wave, ra = 16 * ti + n;
  Frag<T> aDO[NKB], aV[NKB];
  Frag2<T> aDR[NKB], aU[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    aDO[kb] = chunk_row<T, D>(dOc, ra, nrows, 32 * kb, g);
    if constexpr (kErase) {
      aDR[kb] = dRm.row(u0 + (size_t)ra * D + 32 * kb, g);
      aU[kb] = Um.row(u0 + (size_t)ra * D + 32 * kb, g);
    } else {
      aV[kb] = chunk_row<T, D>(vc, ra, nrows, 32 * kb, g);
    }
  }
  // a K or Q row of the chunk: from LDS when staged there, else global
  auto kqrow = [&](const T* lds, const T* glob, int r, int c0) {
    if constexpr (kFull) return frag_row(lds + r * LDK + c0, g);
    else return chunk_row<T, D>(glob, r, nrows, c0, g);
  };
  // the B operand rows of U (erase) or V; the diagonal tile takes the
  // wave's own rows, already in registers
  using BOp = std::conditional_t<kErase, Frag2<T>, Frag<T>>;
  auto brow = [&](int rb, int kb) -> BOp {
    if constexpr (kErase) return Um.row(u0 + (size_t)rb * D + 32 * kb, g);
    else return chunk_row<T, D>(vc, rb, nrows, 32 * kb, g);
  };
  auto tile = [&](int tj, const BOp(&bo)[NKB]) {
    const int rb = 16 * tj + n;
    f32x4 qk = zero4(), dp = zero4(), kk = zero4(), dru = zero4();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const Frag<T> bk = kqrow(Kl, kc, rb, 32 * kb);
      mma(kqrow(Ql, qc, ra, 32 * kb), bk, qk);
      if constexpr (kErase) {
        mma(kqrow(Kl, kc, ra, 32 * kb), bk, kk);
        mma_ab2(aDO[kb], bo[kb], dp);
        mma_a2b2(aDR[kb], bo[kb], dru);
      } else {
        mma(aDO[kb], bo[kb], dp);
      }
    }
    float csp = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * ti + 4 * g + e, i = 16 * tj + n;
      if constexpr (NORM) {
        qk[e] *= rqs[r] * rks[i];
        kk[e] *= rks[r] * rks[i];
      }
      const float Gm = r >= i ? (kGated ? __expf(gs[r] - gs[i]) : 1.f) : 0.f;
      float gg = dp[e] * qk[e] * Gm;
      Em[r * LDC + i] = dp[e] * Gm;
      if constexpr (kErase) {
        const float Kg = r > i ? kk[e] * Gm : 0.f;
        const float dA = r > i ? -dru[e] : 0.f;
        Hm[r * LDC + i] = dA * bs[r] * Gm;
        gg += dA * bs[r] * Kg;
        const float part = sum16(dA * Kg);
        if (n == 0) rsP[1][tj][r] = part;
      }
      const float rs = sum16(gg);
      if (n == 0) rsP[0][tj][r] = rs;
      csp += gg;
    }
    csp += __shfl_xor(csp, 16);
    csp += __shfl_xor(csp, 32);
    if (g == 0) rsP[2][ti][16 * tj + n] = csp;
  };
#pragma unroll 1
  for (int tj = 0; tj < ti; ++tj) {
    BOp bu[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) bu[kb] = brow(16 * tj + n, kb);
    tile(tj, bu);
  }
  if constexpr (kErase) tile(ti, aU);
  else tile(ti, aV);
  __syncthreads();

  // C x D products: wave w owns the rows 16 w .. 16 w + 15; the column
  // tiles go by in order, staged in LDS for all four waves
  Frag2<T> aE[2], aEt[2], aG[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    if constexpr (NORM) {
      // E K and G K read K's rows i, E^T Q Q's rows: their norms, per i
      float xe[8], xt[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = 32 * kb + kidx(g, j);
        xe[j] = Em[ra * LDC + i] * rks[i];
        xt[j] = Em[i * LDC + ra] * rqs[i];
      }
      aE[kb] = frag2_of<T>(xe);
      aEt[kb] = frag2_of<T>(xt);
    } else {
      aE[kb] = frag2_rowx<T>(Em + ra * LDC + 32 * kb, g);
      aEt[kb] = frag2_col<T>(Em + 32 * kb * LDC + ra, LDC, g);
    }
    if constexpr (kErase) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = 32 * kb + kidx(g, j);
        x[j] = Hm[ra * LDC + i] + Hm[i * LDC + ra];
        if constexpr (NORM) x[j] *= rks[i];
      }
      aG[kb] = frag2_of<T>(x);
    }
  }
  // the row factors of the dots with this lane's Q and K rows
  float rqr[4], rkr[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    rqr[e] = NORM ? rqs[16 * ti + 4 * g + e] : 1.f;
    rkr[e] = NORM ? rks[16 * ti + 4 * g + e] : 1.f;
  }
  float dgc_part = 0.f;
  float rdg[4] = {0.f, 0.f, 0.f, 0.f}, rdf[4] = {0.f, 0.f, 0.f, 0.f},
        rdb[4] = {0.f, 0.f, 0.f, 0.f};
  const T* Sp[CS::NP];
#pragma unroll
  for (int pl = 0; pl < CS::NP; ++pl) Sp[pl] = Sb + (pl * 16 + n) * CS::LDB;
#pragma unroll 1
  for (int cj = 0; cj < NCT; ++cj) {
    const int cb = 16 * cj + n;
    __syncthreads();   // E and H fragments taken (first tile), the previous tile's reads done
    st.store(Sb, Kcs, Qcs, tid);
    __syncthreads();
    if (cj + 1 < NCT) st.load(Sm, dSm, s0, kc, qc, nrows, 16 * (cj + 1), tid);
    f32x4 m1 = zero4(), m2 = zero4(), m3 = zero4();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      Frag2<T> bS, bdS;
      bS.hi = frag_row(Sp[0] + 32 * kb, g);
      if constexpr (kSplit) {
        bS.lo = frag_row(Sp[1] + 32 * kb, g);
        bdS.hi = frag_row(Sp[2] + 32 * kb, g);
        bdS.lo = frag_row(Sp[3] + 32 * kb, g);
      } else {
        bdS.hi = frag_row(Sp[1] + 32 * kb, g);
      }
      // <dS', S>, each column tile by one wave
      if ((cj & 3) == wave) dgc_part += frag_dot(bS, bdS);
      mma_ab2(aDO[kb], bS, m1);
      if constexpr (kErase) {
        mma_a2b2(aDR[kb], bS, m2);
        mma_a2b2(aU[kb], bdS, m3);
      } else {
        mma_ab2(aV[kb], bdS, m3);
      }
    }
    // this column tile's K and Q columns
    constexpr int LQ = kFull ? LDK : CS::LDQ;
    const T* const Kt = kFull ? Kl + 16 * cj : Kcs;
    const T* const Qt = kFull ? Ql + 16 * cj : Qcs;
    f32x4 ek = zero4(), etq = zero4(), gk = zero4();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const Frag<T> bK = frag_col(Kt + 32 * kb * LQ + n, LQ, g);
      mma_a2b(aE[kb], bK, ek);
      mma_a2b(aEt[kb], frag_col(Qt + 32 * kb * LQ + n, LQ, g), etq);
      if constexpr (kErase) mma_a2b(aG[kb], bK, gk);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * ti + 4 * g + e;
      float qv = to_f32(Qt[r * LQ + n]);
      float kv = to_f32(Kt[r * LQ + n]);
      if constexpr (NORM) {
        qv *= rqr[e];
        kv *= rkr[e];
      }
      float dQ = gam[r] * m1[e] + ek[e];
      float dK = fs[r] * m3[e] + etq[e];
      rdg[e] += qv * m1[e];
      rdf[e] += kv * m3[e];
      if constexpr (kErase) {
        dK += gk[e] - bs[r] * gam[r] * m2[e];
        rdg[e] -= bs[r] * kv * m2[e];
        rdb[e] -= gam[r] * kv * m2[e];
      }
      if (r < nrows) {
        dq[(row0 + r) * D + cb] = dQ;
        dk[(row0 + r) * D + cb] = dK;
      }
    }
  }
  {
    const float acc = sum64(dgc_part);
    if (lane == 0) red[wave] = acc;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = 16 * ti + 4 * g + e;
    const float a = sum16(rdg[e]), b = sum16(rdf[e]), cc = sum16(rdb[e]);
    if (n == 0) {
      dgam[r] = a;
      dfv[r] = b;
      if constexpr (kErase)
        vdr[r] += cc + rsP[1][0][r] + rsP[1][1][r] + rsP[1][2][r] + rsP[1][3][r];
    }
  }
  __syncthreads();
  if (wave == 0) {
    const int r = lane;
    const float dgC = red[0] + red[1] + red[2] + red[3];
    const float rsum = rsP[0][0][r] + rsP[0][1][r] + rsP[0][2][r] + rsP[0][3][r];
    const float csum = rsP[2][0][r] + rsP[2][1][r] + rsP[2][2][r] + rsP[2][3][r];
    float dg = rsum - csum + dgam[r] * gam[r] - dfv[r] * fs[r];
    const float dff = sum64(dfv[r] * fs[r]);
    if (r == C - 1) dg += dgC * gam[C - 1] + dff;
    const float inc = wave_inclusive_scan(dg);
    const float tot = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inc), C - 1));
    if (r < nrows) {
      if constexpr (kGated) dla[row0 + r] = tot - inc + dg;
      if constexpr (kErase) dbeta[row0 + r] = vdr[r];
    }
  }
}

// ------------------------------------------------------ fused prologue
// The fused forward's prologue, for its backward: per token row, the op's
// inputs from the raw ones -- the inverse norms r = (|x|^2 + 1e-6)^(-1/2)
// of q and k (the normalised rows x r are never formed: the backward takes
// r as a row factor); beta = sigmoid(b); log alpha = -scale softplus(a) -- and,
// after the backward proper, the chain rule back to the raw inputs:
// dx = r (dx_hat - x_hat (x_hat . dx_hat)), db = dbeta sigmoid(b)(1 -
// sigmoid(b)), da = -scale sigmoid(a) dlog_alpha.  d / 8 lanes per row.

__device__ __forceinline__ float sigmoidf(float x) { return 1.f / (1.f + __expf(-x)); }
__device__ __forceinline__ float softplusf(float x) {
  return fmaxf(x, 0.f) + log1pf(__expf(-fabsf(x)));
}

// Lanes per token row: each lane holds 8 consecutive elements (16 bytes of
// bf16, two 16-byte vectors of float).
template <int D>
constexpr int pro_lanes() { return D / 8; }

// Sum over the `W` lanes of a row group (W = 8 or 16, aligned groups).
template <int W>
__device__ __forceinline__ float sum_lanes(float x) {
  if constexpr (W >= 16) x += __shfl_xor(x, 8);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 1);
  return x;
}

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&x)[8]) {
  if constexpr (IsBf16<T>::value) {
    const bf16x8 v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = (float)v[j];
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = a[j];
      x[4 + j] = b[j];
    }
  }
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&x)[8]) {
  if constexpr (IsBf16<T>::value) {
    bf16x8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (__bf16)x[j];
    *reinterpret_cast<u32x4*>(p) = __builtin_bit_cast(u32x4, v);
  } else {
    *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_pro_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const float* __restrict__ a_raw,
    const float* __restrict__ b_raw, float* __restrict__ rq, float* __restrict__ rk,
    float* __restrict__ la,
    float* __restrict__ be, size_t rows, int norm, int gates_a, int gates_b, float scale) {
  constexpr int W = pro_lanes<D>();
  const int sub = threadIdx.x % W;
  const size_t row = (size_t)blockIdx.x * (kThreads / W) + threadIdx.x / W;
  if (row >= rows) return;
  if (norm) {
    const T* src[2] = {q, k};
    float* rr[2] = {rq, rk};
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      float x[8];
      load8(src[m] + row * D + 8 * sub, x);
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += x[j] * x[j];
      const float r = 1.f / sqrtf(sum_lanes<W>(ss) + kQKNormEps);
      if (sub == 0) rr[m][row] = r;
    }
  }
  if (sub == 0) {
    if (gates_a) la[row] = -scale * softplusf(a_raw[row]);
    if (gates_b) be[row] = sigmoidf(b_raw[row]);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_pro_grad_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const float* __restrict__ a_raw,
    const float* __restrict__ b_raw, const float* __restrict__ rq, const float* __restrict__ rk,
    float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ da,
    float* __restrict__ db, size_t rows, int norm, int gates_a, int gates_b, float scale) {
  constexpr int W = pro_lanes<D>();
  const int sub = threadIdx.x % W;
  const size_t row = (size_t)blockIdx.x * (kThreads / W) + threadIdx.x / W;
  if (row >= rows) return;
  if (norm) {
    const T* src[2] = {q, k};
    const float* rr[2] = {rq, rk};
    float* g[2] = {dq, dk};
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const float r = rr[m][row];
      float xh[8], dx[8];
      load8(src[m] + row * D + 8 * sub, xh);
      load8(g[m] + row * D + 8 * sub, dx);
      float dot = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        xh[j] *= r;
        dot += xh[j] * dx[j];
      }
      dot = sum_lanes<W>(dot);
#pragma unroll
      for (int j = 0; j < 8; ++j) dx[j] = r * (dx[j] - xh[j] * dot);
      store8(g[m] + row * D + 8 * sub, dx);
    }
  }
  if (sub == 0) {
    if (gates_a) da[row] = -scale * sigmoidf(a_raw[row]) * da[row];
    if (gates_b) {
      const float s = sigmoidf(b_raw[row]);
      db[row] = s * (1.f - s) * db[row];
    }
  }
}

// ---------------------------------------------------------------- launch
template <typename X>
struct Type {
  using type = X;
};

template <typename F>
hipError_t dispatch(const BwdArgs& a, F&& f) {
  auto by_mode = [&](auto t, auto d) -> hipError_t {
    switch (a.mode) {
      case kModeLinear: return f(t, d, std::integral_constant<int, kModeLinear>{});
      case kModeDelta: return f(t, d, std::integral_constant<int, kModeDelta>{});
      case kModeGatedDelta: return f(t, d, std::integral_constant<int, kModeGatedDelta>{});
      case kModeGatedLinear: return f(t, d, std::integral_constant<int, kModeGatedLinear>{});
      default: return hipErrorInvalidValue;
    }
  };
  if (a.d != 64 && a.d != 128) return hipErrorInvalidValue;
  if (a.in_bf16)
    return a.d == 64 ? by_mode(Type<__bf16>{}, std::integral_constant<int, 64>{})
                     : by_mode(Type<__bf16>{}, std::integral_constant<int, 128>{});
  return a.d == 64 ? by_mode(Type<float>{}, std::integral_constant<int, 64>{})
                   : by_mode(Type<float>{}, std::integral_constant<int, 128>{});
}

// f(std::bool_constant<NORM>): NORM when the call folds the q and k norms
template <typename F>
void by_norm(const BwdArgs& a, F&& f) {
  if (a.rk) f(std::true_type{});
  else f(std::false_type{});
}

}  // namespace

size_t bwd_workspace_bytes(const BwdArgs& a) { return carve(a, nullptr); }

hipError_t launch_bwd_prep(const BwdArgs& a, hipStream_t st) {
  BwdWs ws;
  carve(a, &ws);
  const unsigned grid = (unsigned)slots(a);
  const SeqMap sm = seq_map(a);
  return dispatch(a, [&](auto t, auto d, auto m) {
    using T = typename decltype(t)::type;
    by_norm(a, [&](auto nm) {
      hipLaunchKernelGGL(
          (bwd_prep_kernel<T, decltype(d)::value, decltype(m)::value, decltype(nm)::value>),
          dim3(grid), dim3(kThreads), 0, st, static_cast<const T*>(a.q),
          static_cast<const T*>(a.k), static_cast<const T*>(a.dout), a.log_alpha, a.beta, a.rq,
          a.rk, ws, sm);
    });
    return hipGetLastError();
  });
}

hipError_t launch_bwd_states(const BwdArgs& a, hipStream_t st) {
  BwdWs ws;
  carve(a, &ws);
  const int BH = a.B * a.H;
  const unsigned grid = (unsigned)((size_t)BH * (a.d / 16));
  return dispatch(a, [&](auto t, auto d, auto m) {
    using T = typename decltype(t)::type;
    by_norm(a, [&](auto nm) {
      hipLaunchKernelGGL(
          (bwd_states_kernel<T, decltype(d)::value, decltype(m)::value, decltype(nm)::value>),
          dim3(grid), dim3(kStatesThreads), 0, st, static_cast<const T*>(a.k),
          static_cast<const T*>(a.v), a.beta, a.rk, a.S0, ws, seq_map(a), BH);
    });
    return hipGetLastError();
  });
}

hipError_t launch_bwd_rev(const BwdArgs& a, hipStream_t st) {
  BwdWs ws;
  carve(a, &ws);
  const int BH = a.B * a.H;
  const unsigned grid = (unsigned)((size_t)BH * (a.d / 16));
  return dispatch(a, [&](auto t, auto d, auto m) {
    using T = typename decltype(t)::type;
    by_norm(a, [&](auto nm) {
      hipLaunchKernelGGL(
          (bwd_rev_kernel<T, decltype(d)::value, decltype(m)::value, decltype(nm)::value>),
          dim3(grid), dim3(kRevThreads), 0, st, static_cast<const T*>(a.k), a.beta, a.rk,
          a.dS_final, a.dv, a.dS0, ws, seq_map(a), BH);
    });
    return hipGetLastError();
  });
}

hipError_t launch_bwd_grads(const BwdArgs& a, hipStream_t st) {
  BwdWs ws;
  carve(a, &ws);
  const unsigned grid = (unsigned)slots(a);
  return dispatch(a, [&](auto t, auto d, auto m) {
    using T = typename decltype(t)::type;
    by_norm(a, [&](auto nm) {
      hipLaunchKernelGGL(
          (bwd_grads_kernel<T, decltype(d)::value, decltype(m)::value, decltype(nm)::value>),
          dim3(grid), dim3(kThreads), 0, st, static_cast<const T*>(a.q),
          static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.beta,
          static_cast<const T*>(a.dout), a.rq, a.rk, a.dq, a.dk, a.dlog_alpha, a.dbeta, ws,
          seq_map(a));
    });
    return hipGetLastError();
  });
}

hipError_t launch_bwd_pro(const BwdProArgs& p, bool grad, hipStream_t st) {
  if (p.d != 64 && p.d != 128) return hipErrorInvalidValue;
  auto go = [&](auto t, auto d) -> hipError_t {
    using T = typename decltype(t)::type;
    constexpr int D = decltype(d)::value;
    constexpr size_t per_block = kThreads / pro_lanes<D>();
    const unsigned grid = (unsigned)((p.rows + per_block - 1) / per_block);
    if (!grad)
      hipLaunchKernelGGL((bwd_pro_kernel<T, D>), dim3(grid), dim3(kThreads), 0, st,
                         static_cast<const T*>(p.q), static_cast<const T*>(p.k), p.a_raw,
                         p.b_raw, p.rq, p.rk, p.la, p.be, p.rows, p.norm, p.gates_a, p.gates_b, p.scale);
    else
      hipLaunchKernelGGL((bwd_pro_grad_kernel<T, D>), dim3(grid), dim3(kThreads), 0, st,
                         static_cast<const T*>(p.q), static_cast<const T*>(p.k), p.a_raw,
                         p.b_raw, p.rq, p.rk, p.dq, p.dk, p.da, p.db, p.rows, p.norm,
                         p.gates_a, p.gates_b, p.scale);
    return hipGetLastError();
  };
  if (p.in_bf16)
    return p.d == 64 ? go(Type<__bf16>{}, std::integral_constant<int, 64>{})
                     : go(Type<__bf16>{}, std::integral_constant<int, 128>{});
  return p.d == 64 ? go(Type<float>{}, std::integral_constant<int, 64>{})
                   : go(Type<float>{}, std::integral_constant<int, 128>{});
}

}  // namespace la
