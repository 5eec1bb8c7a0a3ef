// Fused chunkwise forward: one kernel that carries the state across chunks
// and produces the output, reading q, k, v and the gates once.
//
// For one (batch, head) with dk = dv = D and a chunk of C = 64 rows with
// keys K, values V, queries Q, write strengths beta and log-decays:
//
//   g_r    = sum_{i <= r} log_alpha_i          (in-chunk cumulative decay)
//   gam_r  = exp(g_r),  Gamma_ri = exp(g_r - g_i) for i <= r
//   A      = strict_lower(diag(beta) (K K^T) * Gamma)
//   T      = (I + A)^{-1}                      (unit lower-triangular)
//   R      = diag(beta) (V - diag(gam) K S)
//   U_new  = T R                               (the true per-row updates)
//   O      = diag(gam) Q S + ((Q K^T) * M * Gamma) U_new
//   S'     = gam_C S + K^T diag(gam_C / gam) U_new
//
// This is the inductive redefinition of the per-token update vectors
// ("重新定义降低内存占用" in the hybrid-attention notes "混合注意力学习(1):
// 线性注意力") in its WY/UT form ("HouseHolder变换和WY表示", same notes):
// with W = T diag(beta gam) K and U = T diag(beta) V one has U_new =
// U - W S = T R, so the chunk needs T and never a past per-token state.
// The scalar decay of "Gated DeltaNet" (same notes) is folded in through
// Gamma and gam.  Delta mode is alpha = 1 (g = 0); plain linear attention
// ("FWP分块并行机制", same notes; "FLASH" in "LinearAttention 概述") is
// U_new = V, g = 0: O = Q S + ((Q K^T) * M) V, S' = S + K^T V.
//
// Mapping to gfx950.  The dv columns of the state evolve independently, so
// one 256-thread workgroup owns one 16-column tile of one (batch, head)
// state and walks the chunks of that sequence in order; the B * H * dv / 16
// workgroups run in parallel.  The 16 x dk state tile stays in MFMA
// accumulator registers of wave 0 for the whole sequence.  Blocks are
// numbered so that the dv / 16 workgroups of one head land on the same XCD
// (workgroups are dealt to the 8 XCDs round-robin), so the q, k and gate
// rows every tile of a head reads are fetched from HBM once and served to
// the others from that XCD's L2.
//
// Per chunk, with the next chunk's inputs already loaded into registers:
//   stage    all waves  write Q, K, K^T (transposed), V^T (this tile's 16
//                       columns), beta and g to LDS; issue the next
//                       chunk's global loads
//   scores   all waves  the 10 lower-triangular 16 x 16 tiles of Q K^T and
//                       (delta modes) of K K^T on MFMA, with decay and mask;
//                       each wave owns two row tiles of one product
//   T        wave 0     the four 16 x 16 diagonal blocks of T by forward
//                       substitution (one lane per column)
//            waves 0-2  wave j: the blocks below the diagonal in column
//                       block j, T_ij = -T_ii sum_k A_ik T_kj, on MFMA
//   chain    wave 0     K S, R, U_new = T R, S update (MFMA)
//            waves 1-3  Q S for their row tiles (MFMA), from the entry
//                       state that wave 0 published in LDS
//   output   waves 1-3  O = diag(gam) Q S + Aqk U_new; wave 0 publishes the
//                       new state for the next chunk's Q S
// With one wave per SIMD nothing hides LDS latency, so every phase loads
// all of its operands into registers before its first product.
//
// Precision (bf16 inputs).  Q, K, V are exact bf16 MFMA operands.  Every
// float quantity that feeds a bf16 MFMA -- the state S, R, U_new, the
// masked scores, the A blocks and partial T blocks of the solve -- is split
// into bf16 hi + lo parts, so those products carry about 16 bits.  T itself
// enters U_new = T R as a single bf16 (its rounding changes the result by a
// small fraction of the tolerance).  The state is accumulated in float.

#include "la_device.hpp"
#include "la_kernels.hpp"

namespace la {
namespace {

constexpr int C = 64;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// 16-deep operand: values p[4 g + j] for j < 4 and zero in the upper four
// slots (the second 16 of a 32-deep block), matching kidx().
template <typename T>
__device__ __forceinline__ Frag2<T> frag2_row16(const float* p, int g) {
  Frag2<T> f;
  const f32x4 a = *reinterpret_cast<const f32x4*>(p + 4 * g);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f.set(i, a[i]);
    f.set(4 + i, 0.f);
  }
  return f;
}

// The 16-bit element `half` (0 = low, 1 = high) of the dwords a and b,
// packed as (a's, b's) into one dword: two rows of a column of a bf16 tile.
__device__ __forceinline__ uint32_t pack_halves(uint32_t a, uint32_t b, int half) {
  return half ? (a >> 16) | (b & 0xffff0000u) : (a & 0xffffu) | (b << 16);
}

// Column swizzle of the transposed K tile: the 16-byte units of row r are
// permuted by XOR with ((r / 8) mod 8), which spreads both the transposing
// writes (16 lanes writing one column of 16 different rows) and the row
// reads over the LDS banks.  Returns the XOR in elements.
template <typename T>
__device__ __forceinline__ constexpr int tswz(int r) {
  return ((r >> 3) & 7) * (16 / (int)sizeof(T));
}

// Operand row of the swizzled tile: 8 values rowp[(c0 + kidx(g, j)) ^ swz];
// c0 is a multiple of 32 elements, swz a multiple of 16 bytes.
template <typename T>
__device__ __forceinline__ Frag<T> frag_row_swz(const T* rowp, int c0, int g, int swz) {
  Frag<T> f;
  const int a = (c0 + 4 * g) ^ swz, b = (c0 + 16 + 4 * g) ^ swz;
  if constexpr (IsBf16<T>::value) {
    const bf16x4 x = *reinterpret_cast<const bf16x4*>(rowp + a);
    const bf16x4 y = *reinterpret_cast<const bf16x4*>(rowp + b);
    f.v = __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
  } else {
    const f32x4 x = *reinterpret_cast<const f32x4*>(rowp + a);
    const f32x4 y = *reinterpret_cast<const f32x4*>(rowp + b);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f.v[i] = x[i];
      f.v[4 + i] = y[i];
    }
  }
  return f;
}

// Scores of two row tiles R0 and R1 of X K^T.  X = Q: the masked, decayed
// scores (Q K^T) * M * Gamma go to Aq as hi/lo planes; X = K:
// A = strict_lower(diag(beta) (K K^T) * Gamma) goes to As.  All operands
// are loaded before the first product; the 16 x 16 tiles strictly below the
// diagonal need no mask.
template <typename T, int D, bool GATED, bool QK, int R0, int R1, int LDQ, int LDT, int LDF>
__device__ __forceinline__ void score_rows(const T* X, const T* Ks, const float* gs,
                                           const float* bs, T* Aq, float* As, int g, int n,
                                           int nq) {
  constexpr int NKB = D / 32;
  constexpr int NT = (R0 > R1 ? R0 : R1) + 1;
  constexpr bool kSplit = IsBf16<T>::value;
  Frag<T> a0[NKB], a1[NKB], b[NT][NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    a0[kb] = frag_row(X + 16 * LDQ * R0 + nq + 32 * kb, g);
    a1[kb] = frag_row(X + 16 * LDQ * R1 + nq + 32 * kb, g);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) b[t][kb] = frag_row(Ks + 16 * LDQ * t + nq + 32 * kb, g);
  // gates: rows 16 R + 4 g + i of this lane, column 16 t + n
  f32x4 gr0 = zero4(), gr1 = zero4(), br0 = zero4(), br1 = zero4();
  float gc[NT];
  if constexpr (GATED) {
    gr0 = *reinterpret_cast<const f32x4*>(gs + 16 * R0 + 4 * g);
    gr1 = *reinterpret_cast<const f32x4*>(gs + 16 * R1 + 4 * g);
#pragma unroll
    for (int t = 0; t < NT; ++t) gc[t] = gs[16 * t + n];
  }
  if constexpr (!QK) {
    br0 = *reinterpret_cast<const f32x4*>(bs + 16 * R0 + 4 * g);
    br1 = *reinterpret_cast<const f32x4*>(bs + 16 * R1 + 4 * g);
  }
  f32x4 acc0[R0 + 1], acc1[R1 + 1];
#pragma unroll
  for (int t = 0; t <= R0; ++t) acc0[t] = zero4();
#pragma unroll
  for (int t = 0; t <= R1; ++t) acc1[t] = zero4();
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
    for (int t = 0; t <= R0; ++t) mma(a0[kb], b[t][kb], acc0[t]);
#pragma unroll
    for (int t = 0; t <= R1; ++t) mma(a1[kb], b[t][kb], acc1[t]);
  }
  auto epilogue = [&](const f32x4& acc, int R, int t, const f32x4& gr, const f32x4& br) {
    const int cc = 16 * t + n;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * R + 4 * g + i;
      const bool keep = R > t || (QK ? r >= cc : r > cc);
      float decay = 1.f;
      if constexpr (GATED) decay = __expf(keep ? gr[i] - gc[t] : 0.f);
      float x = acc[i] * decay;
      if constexpr (!QK) x *= br[i];
      x = keep ? x : 0.f;
      if constexpr (QK) {
        const T h = from_f32<T>(x);
        Aq[r * LDT + cc] = h;
        if constexpr (kSplit) Aq[C * LDT + r * LDT + cc] = from_f32<T>(x - to_f32(h));
      } else {
        As[r * LDF + cc] = x;
      }
    }
  };
#pragma unroll
  for (int t = 0; t <= R0; ++t) epilogue(acc0[t], R0, t, gr0, br0);
#pragma unroll
  for (int t = 0; t <= R1; ++t) epilogue(acc1[t], R1, t, gr1, br1);
}

// The four 16 x 16 diagonal blocks of T, one wave: lane (g, n) solves
// column n of block g by forward substitution,
//   x_r = [r == n] - sum_{i < r} A[16 g + r][16 g + i] x_i,
// with the block's rows loaded first and each sum split over two
// accumulators to halve the dependent chain.
template <typename T, int LDF, int LDT>
__device__ __forceinline__ void tdiag_solve(const float* As, float* Tf, T* Tb, int g, int n) {
  const float* Ab = As + (16 * g) * LDF + 16 * g;
  f32x4 arow[16][4];
#pragma unroll
  for (int r = 1; r < 16; ++r)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4)
      if (4 * i4 < r) arow[r][i4] = *reinterpret_cast<const f32x4*>(Ab + r * LDF + 4 * i4);
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float s0 = r == n ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < r; ++i) {
      const float a = arow[r][i / 4][i % 4];
      if (i % 2 == 0) s0 = fmaf(-a, x[i], s0);
      else s1 = fmaf(-a, x[i], s1);
    }
    x[r] = s0 + s1;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    Tf[(16 * g + r) * LDF + 16 * g + n] = x[r];
    if constexpr (IsBf16<T>::value) Tb[(16 * g + r) * LDT + 16 * g + n] = from_f32<T>(x[r]);
  }
}

// Column block J of T = (I + A)^{-1} below the diagonal, given the
// diagonal blocks T_ii in Tf:  T_iJ = -T_ii (sum_{k=J}^{i-1} A_ik T_kJ) for
// i = J+1 .. 3, in order.  The finished tiles stay in accumulator layout,
// which is directly the B operand of the next product.  The results go to
// Tb (bf16 copy) for split inputs, to Tf otherwise.
template <typename T, int J, int LDF, int LDT>
__device__ __forceinline__ void tcol_solve(const float* As, float* Tf, T* Tb, int g, int n) {
  f32x4 tc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) tc[J][i] = Tf[(16 * J + 4 * g + i) * LDF + 16 * J + n];
#pragma unroll
  for (int i = J + 1; i < 4; ++i) {
    f32x4 xacc = zero4();
#pragma unroll
    for (int kk = J; kk < i; kk += 2) {
      const float* arow = As + (16 * i + n) * LDF + 16 * kk;
      if (kk + 1 < i) {
        mma_a2b2(frag2_row<T>(arow, g), frag2_from_acc<T>(tc[kk], tc[kk + 1]), xacc);
      } else {
        mma_a2b2(frag2_row16<T>(arow, g), frag2_from_acc<T>(tc[kk], zero4()), xacc);
      }
    }
    f32x4 y = zero4();
    mma_a2b2(frag2_row16<T>(Tf + (16 * i + n) * LDF + 16 * i, g),
             frag2_from_acc<T>(xacc, zero4()), y);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y[e] = -y[e];
      const int r = 16 * i + 4 * g + e;
      if constexpr (IsBf16<T>::value) Tb[r * LDT + 16 * J + n] = from_f32<T>(y[e]);
      else Tf[r * LDF + 16 * J + n] = y[e];
    }
    tc[i] = y;
  }
}

// Q S for NTI row tiles (TI0, TI1) of the chunk, from the entry state that
// wave 0 published in Sx as split B-operand fragments.
template <typename T, int D, int NTI, int TI0, int TI1, int LDQ>
__device__ __forceinline__ void qs_rows(const T* Qs, const Frag<T>* Sx, f32x4 (&qs)[2], int g,
                                        int nq, int lane) {
  constexpr int NKB = D / 32;
  constexpr int kPlanes = IsBf16<T>::value ? 2 : 1;
  Frag2<T> sx[NKB];
  Frag<T> qf[NTI][NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    sx[kb].hi = Sx[(kPlanes * kb) * kWave + lane];
    if constexpr (kPlanes == 2) sx[kb].lo = Sx[(2 * kb + 1) * kWave + lane];
  }
#pragma unroll
  for (int u = 0; u < NTI; ++u)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      qf[u][kb] = frag_row(Qs + 16 * LDQ * (u == 0 ? TI0 : TI1) + nq + 32 * kb, g);
#pragma unroll
  for (int u = 0; u < NTI; ++u) {
    qs[u] = zero4();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) mma_ab2(qf[u][kb], sx[kb], qs[u]);
  }
}

// O = diag(gam) Q S + Aqk U_new for NTI row tiles (TI0, TI1); the modes
// without erase use V for U_new.  ob0 indexes (first row of the chunk, this lane's
// column) of the output.
template <typename T, int D, int MODE, int NTI, int TI0, int TI1, int LDT>
__device__ __forceinline__ void out_rows(const T* Aq, const Frag<T>* Ux, const T* Vt,
                                         const float* gs, const f32x4 (&qs)[2], void* out_,
                                         size_t ob0, int out_bf16, int g, int nt, int lane,
                                         int nrows) {
  constexpr bool kDelta = mode_erase(MODE);
  constexpr bool kGated = mode_decay(MODE);
  constexpr bool kSplit = IsBf16<T>::value;
  constexpr int kPlanes = kSplit ? 2 : 1;
  Frag2<T> uf[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    if constexpr (kDelta) {
      uf[kb].hi = Ux[(kPlanes * kb) * kWave + lane];
      if constexpr (kSplit) uf[kb].lo = Ux[(2 * kb + 1) * kWave + lane];
    } else {
      uf[kb].hi = frag_row(Vt + nt + 32 * kb, g);
    }
  }
  Frag2<T> af[NTI][2];
  f32x4 gg[NTI];
#pragma unroll
  for (int u = 0; u < NTI; ++u) {
    const int ti = u == 0 ? TI0 : TI1;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (kb == 1 && ti < 2) continue;       // Aq is zero above the diagonal
      af[u][kb].hi = frag_row(Aq + 16 * LDT * ti + nt + 32 * kb, g);
      if constexpr (kSplit) af[u][kb].lo = frag_row(Aq + C * LDT + 16 * LDT * ti + nt + 32 * kb, g);
    }
    if constexpr (kGated) gg[u] = *reinterpret_cast<const f32x4*>(gs + 16 * ti + 4 * g);
  }
#pragma unroll
  for (int u = 0; u < NTI; ++u) {
    const int ti = u == 0 ? TI0 : TI1;
    f32x4 o = qs[u];
    if constexpr (kGated) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] *= __expf(gg[u][i]);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (kb == 1 && ti < 2) continue;
      if constexpr (kDelta) {
        mma_a2b2(af[u][kb], uf[kb], o);
      } else {
        // linear: V is exact in the input type
        if constexpr (kSplit) mma(af[u][kb].lo, uf[kb].hi, o);
        mma(af[u][kb].hi, uf[kb].hi, o);
      }
    }
    // rows at or past nrows lie past the end of the sequence
    const int r0 = 16 * ti + 4 * g;
    const size_t ob = ob0 + (size_t)r0 * D;
    if (out_bf16) {
      __bf16* out = static_cast<__bf16*>(out_);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (r0 + i < nrows) out[ob + (size_t)i * D] = (__bf16)o[i];
    } else {
      float* out = static_cast<float*>(out_);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (r0 + i < nrows) out[ob + (size_t)i * D] = o[i];
    }
  }
}

template <typename T, int D, int MODE>
__global__ __launch_bounds__(kThreads) void chunk_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    const float* __restrict__ S0, void* __restrict__ out_, float* __restrict__ S_final,
    SeqMap sm, int BH, int out_bf16) {
  constexpr bool kDelta = mode_erase(MODE);      // delta rule: beta, T
  constexpr bool kGated = mode_decay(MODE);      // scalar decay: log alpha
  constexpr bool kSplit = IsBf16<T>::value;
  constexpr int kPlanes = kSplit ? 2 : 1;
  constexpr int PE = 16 / sizeof(T);             // elements per 16 bytes
  constexpr int LDQ = D + PE;                    // row pitch of Q, K tiles
  constexpr int LDT = C + PE;                    // row pitch of K^T, V^T, T, Aqk
  constexpr int LDF = C + 4;                     // row pitch of float C x C
  constexpr int NKT = D / 16;                    // 16-row tiles of the state
  constexpr int NKB = D / 32;                    // 32-deep blocks over dk
  constexpr int NCT = D / 16;                    // column tiles per head
  // A transposed copy of K serves K^T U_new; without room for it (float,
  // D = 128) K^T's operand columns are gathered from K directly.
  constexpr bool kKt = sizeof(T) == 2 || D == 64;
  // Prefetch layout: thread t holds 16-byte vector t % VPR of the rows
  // 2 p and 2 p + 1, p = t / VPR + NRP * pass.
  constexpr int VPR = D / PE;                    // 16-byte vectors per row
  constexpr int NRP = kThreads / VPR;            // row pairs per pass
  constexpr int NPASS = C / (2 * NRP);
  constexpr int NVQ = 2 * NPASS;                 // Q (and K) vectors per thread
  static_assert(NPASS * 2 * NRP == C, "tile split");
  constexpr int VVR = 16 / PE;                   // V vectors per 16-column row
  constexpr int NVV = C * VVR / kWave;           // V vectors per lane of wave 0

  __shared__ __attribute__((aligned(16))) T Qs[C * LDQ];
  __shared__ __attribute__((aligned(16))) T Ks[C * LDQ];
  __shared__ __attribute__((aligned(16))) T Kt[kKt ? D * LDT : PE];
  __shared__ __attribute__((aligned(16))) T Vt[16 * LDT];
  __shared__ __attribute__((aligned(16))) T Aq[kPlanes * C * LDT];
  __shared__ __attribute__((aligned(16))) float As[kDelta ? C * LDF : 4];
  __shared__ __attribute__((aligned(16))) float Tf[kDelta ? C * LDF : 4];
  __shared__ __attribute__((aligned(16))) T Tb[kDelta && kSplit ? C * LDT : PE];
  __shared__ __attribute__((aligned(16))) Frag<T> Sx[kPlanes * NKB * kWave];
  __shared__ __attribute__((aligned(16))) Frag<T> Ux[kPlanes * 2 * kWave];
  __shared__ __attribute__((aligned(16))) float gs[C];
  __shared__ __attribute__((aligned(16))) float bs[C];

  const int tid = threadIdx.x;
  // wave-uniform, kept in a scalar register: role branches are scalar and
  // tile indices derived from it need no per-lane arithmetic
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int g = lane / 16;
  const int n = lane % 16;

  // Block -> (head, column tile), keeping the NCT tiles of a head on the
  // XCD that block % 8 selects when the head count allows it.
  int bh, ct;
  {
    const int b = blockIdx.x;
    if (BH % 8 == 0) {
      const int x = b % 8, s = b / 8;
      ct = s % NCT;
      bh = (s / NCT) * 8 + x;
    } else {
      bh = b / NCT;
      ct = b % NCT;
    }
  }
  const int col0 = ct * 16;
  const int col = col0 + n;
  // Per-lane LDS row offsets, computed once: inside the chunk loop every
  // tile address is this plus a wave-uniform or constant term, so the
  // vector address arithmetic there is additions only.
  const int nq = n * LDQ;       // row n of a Q / K tile
  const int nt = n * LDT;       // row n of a V^T / T / Aqk tile
  const int pcv = tid % VPR;    // prefetch: 16-byte vector within the row
  const int prp = tid / VPR;    // prefetch: row pair within a pass

  const SeqInfo si = seq_info(sm, bh);
  const size_t hbase = si.row0;                 // first token row of the head
  const int L = si.len;                         // tokens of this sequence
  if (L == 0) {
    // empty sequence: the state passes through
    if (wave == 0 && S_final) {
      const size_t sb = (size_t)bh * D * D;
#pragma unroll
      for (int r = 0; r < D / 4; ++r) {
        const size_t e = sb + (size_t)(4 * r + g) * D + col;
        S_final[e] = S0 ? S0[e] : 0.f;
      }
    }
    return;
  }

  // T as the A operand of U_new = T R: bf16 copy (split inputs) or Tf.
  const T* Top;
  if constexpr (kDelta && kSplit) Top = Tb;
  else Top = reinterpret_cast<const T*>(Tf);
  constexpr int LDTop = kDelta && kSplit ? LDT : LDF;

  // ---- blocks that stay zero for the whole sequence.  The output reads
  // Aq, and U_new = T R reads T, in 32-column blocks: the upper 16 x 16
  // blocks (0, 1) and (2, 3) that share such a block with a lower block are
  // never written by the chunk loop and must read as zero.
  if (wave == kWaves - 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g + i;
#pragma unroll
      for (int p = 0; p < kPlanes; ++p) {
        Aq[p * C * LDT + r * LDT + 16 + n] = from_f32<T>(0.f);
        Aq[p * C * LDT + (32 + r) * LDT + 48 + n] = from_f32<T>(0.f);
      }
      if constexpr (kDelta) {
        if constexpr (kSplit) {
          Tb[r * LDT + 16 + n] = from_f32<T>(0.f);
          Tb[(32 + r) * LDT + 48 + n] = from_f32<T>(0.f);
        } else {
          Tf[r * LDF + 16 + n] = 0.f;
          Tf[(32 + r) * LDF + 48 + n] = 0.f;
        }
      }
    }
  }

  // ---- state tile (wave 0): S[tj][i] = S[16 tj + 4 g + i][col]
  f32x4 S[NKT];
  const size_t sbase = (size_t)bh * D * D;
  if (wave == 0) {
    if (S0) {
#pragma unroll
      for (int tj = 0; tj < NKT; ++tj)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[tj][i] = S0[sbase + (size_t)(16 * tj + 4 * g + i) * D + col];
    } else {
#pragma unroll
      for (int tj = 0; tj < NKT; ++tj) S[tj] = zero4();
    }
    // publish the entry state for the first chunk's Q S
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const Frag2<T> f = frag2_from_acc<T>(S[2 * kb], S[2 * kb + 1]);
      Sx[(kPlanes * kb) * kWave + lane] = f.hi;
      if constexpr (kSplit) Sx[(2 * kb + 1) * kWave + lane] = f.lo;
    }
  }

  // ---- prefetch registers for one chunk
  u32x4 pq[NVQ], pk[NVQ];
  u32x4 pv[NVV];            // wave 0: this tile's 16 columns of V
  float pla = 0.f, pb = 0.f;
  // V row of wave-0 prefetch vector m: bf16 lanes take row pairs
  // (2 p, 2 p + 1), float lanes rows p + 16 m; the 16-byte unit is lane % VVR.
  auto vrow = [&](int m) {
    if constexpr (kSplit) return 2 * (lane / 2) + m;
    else return lane / VVR + (C / NVV) * m;
  };
  // Chunks; the last may hold fewer than C rows.  Rows past the sequence
  // act as tokens that change nothing: their Q and K reads are clamped to
  // the last valid row, V, beta and log alpha are zero (no write, no erase,
  // no decay; identity rows of T), and their outputs are not stored.  Valid
  // rows never see them: every product inside a chunk is causal.
  const int NC = (L + C - 1) / C;
  auto rows_of = [&](int c) { return min(C, L - c * C); };
  auto load_chunk = [&](int c) {
    const size_t row0 = hbase + (size_t)c * C;
    const int nv = rows_of(c);
#pragma unroll
    for (int m = 0; m < NVQ; ++m) {
      const int r = min(2 * (prp + NRP * (m / 2)) + (m % 2), nv - 1);
      pq[m] = *reinterpret_cast<const u32x4*>(q + (row0 + r) * D + pcv * PE);
      pk[m] = *reinterpret_cast<const u32x4*>(k + (row0 + r) * D + pcv * PE);
    }
    if (wave == 0) {
#pragma unroll
      for (int m = 0; m < NVV; ++m) {
        const int r = vrow(m);
        pv[m] = *reinterpret_cast<const u32x4*>(v + (row0 + min(r, nv - 1)) * D + col0 +
                                               (lane % VVR) * PE);
        if (r >= nv) pv[m] = u32x4{0u, 0u, 0u, 0u};
      }
      const int lr = min(lane, nv - 1);
      if (kGated) pla = lane < nv ? log_alpha[row0 + lr] : 0.f;
      if (kDelta) pb = lane < nv ? beta[row0 + lr] : 0.f;
    }
  };

  load_chunk(0);

  for (int c = 0; c < NC; ++c) {
    const size_t row0 = hbase + (size_t)c * C;

    // ---------------- stage: registers -> LDS, then prefetch the next chunk
#pragma unroll
    for (int m = 0; m < NVQ; ++m) {
      const int r = 2 * (prp + NRP * (m / 2)) + (m % 2);
      *reinterpret_cast<u32x4*>(Qs + r * LDQ + pcv * PE) = pq[m];
      *reinterpret_cast<u32x4*>(Ks + r * LDQ + pcv * PE) = pk[m];
    }
    if constexpr (kKt) {
      // K^T[j][r] = K[r][j], swizzled; for bf16 rows r, r + 1 go as one dword
#pragma unroll
      for (int m = 0; m < NVQ; m += 2) {
        const int r = 2 * (prp + NRP * (m / 2));
#pragma unroll
        for (int j = 0; j < PE; ++j) {
          const int row = pcv * PE + j;
          const int sw = tswz<T>(row);
          if constexpr (kSplit) {
            *reinterpret_cast<uint32_t*>(Kt + row * LDT + (r ^ sw)) =
                pack_halves(pk[m][j / 2], pk[m + 1][j / 2], j % 2);
          } else {
            reinterpret_cast<uint32_t*>(Kt)[row * LDT + (r ^ sw)] = pk[m][j];
            reinterpret_cast<uint32_t*>(Kt)[row * LDT + ((r + 1) ^ sw)] = pk[m + 1][j];
          }
        }
      }
    }
    if (wave == 0) {
      // V^T[j][r] = V[r][col0 + j]
      if constexpr (kSplit) {
        const int r = 2 * (lane / 2), h = lane % 2;
#pragma unroll
        for (int j = 0; j < PE; ++j)
          *reinterpret_cast<uint32_t*>(Vt + (h * PE + j) * LDT + r) =
              pack_halves(pv[0][j / 2], pv[1][j / 2], j % 2);
      } else {
#pragma unroll
        for (int m = 0; m < NVV; ++m)
#pragma unroll
          for (int j = 0; j < PE; ++j)
            reinterpret_cast<uint32_t*>(Vt)[((lane % VVR) * PE + j) * LDT + vrow(m)] = pv[m][j];
      }
      if constexpr (kGated) gs[lane] = wave_inclusive_scan(pla);
      else gs[lane] = 0.f;
      bs[lane] = pb;
    }
    if (c + 1 < NC) load_chunk(c + 1);
    __syncthreads();

    // ---------------- scores: lower tiles of Q K^T (-> Aq) and K K^T (-> As)
    // wave 0: Q rows 0, 3; wave 1: Q rows 1, 2; wave 2: K rows 0, 3;
    // wave 3: K rows 1, 2 -- five 16 x 16 tiles each.  Linear mode has no
    // K K^T: waves 2 and 3 idle here.
    if (wave == 0) {
      score_rows<T, D, kGated, true, 0, 3, LDQ, LDT, LDF>(Qs, Ks, gs, bs, Aq, As, g, n, nq);
    } else if (wave == 1) {
      score_rows<T, D, kGated, true, 1, 2, LDQ, LDT, LDF>(Qs, Ks, gs, bs, Aq, As, g, n, nq);
    } else if constexpr (kDelta) {
      if (wave == 2)
        score_rows<T, D, kGated, false, 0, 3, LDQ, LDT, LDF>(Ks, Ks, gs, bs, Aq, As, g, n, nq);
      else
        score_rows<T, D, kGated, false, 1, 2, LDQ, LDT, LDF>(Ks, Ks, gs, bs, Aq, As, g, n, nq);
    }
    __syncthreads();

    if constexpr (kDelta) {
      // ---------------- T = (I + A)^{-1}: diagonal blocks (wave 0)
      if (wave == 0) tdiag_solve<T, LDF, LDT>(As, Tf, Tb, g, n);
      __syncthreads();
      // ---------------- T: blocks below the diagonal, column block j = wave
      //   T_ij = -T_ii (sum_{k=j}^{i-1} A_ik T_kj),  i = j+1 .. 3
      if (wave == 0) tcol_solve<T, 0, LDF, LDT>(As, Tf, Tb, g, n);
      else if (wave == 1) tcol_solve<T, 1, LDF, LDT>(As, Tf, Tb, g, n);
      else if (wave == 2) tcol_solve<T, 2, LDF, LDT>(As, Tf, Tb, g, n);
      __syncthreads();
    }

    // ---------------- chain (wave 0) and Q S (waves 1-3)
    f32x4 qs[2];
    if (wave == 0) {
      // operands of the whole step, loaded before the first product
      Frag<T> ktf[NKT][2];
#pragma unroll
      for (int tj = 0; tj < NKT; ++tj)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if constexpr (kKt) {
            const int row = 16 * tj + n;
            ktf[tj][kb] = frag_row_swz(Kt + row * LDT, 32 * kb, g, tswz<T>(row));
          } else {
            ktf[tj][kb] = frag_col(Ks + 32 * kb * LDQ + 16 * tj + n, LDQ, g);
          }
        }
      if constexpr (kDelta) {
        Frag<T> kf[4][NKB], tf[4][2];
        f32x4 vv[4], bb[4], gg[4];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
            kf[ti][kb] = frag_row(Ks + 16 * LDQ * ti + nq + 32 * kb, g);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            if (kb <= ti / 2) tf[ti][kb] = frag_row(Top + (16 * LDTop) * ti + n * LDTop + 32 * kb, g);
          const int r0 = 16 * ti + 4 * g;
#pragma unroll
          for (int i = 0; i < 4; ++i) vv[ti][i] = to_f32(Vt[nt + r0 + i]);
          bb[ti] = *reinterpret_cast<const f32x4*>(bs + r0);
          gg[ti] = *reinterpret_cast<const f32x4*>(gs + r0);
        }
        const float gC = gs[C - 1];
        Frag2<T> sf[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) sf[kb] = frag2_from_acc<T>(S[2 * kb], S[2 * kb + 1]);
        // R = diag(beta) (V - diag(gam) K S), rows 16 ti + 4 g + i
        f32x4 ks[4], rr[4];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) ks[ti] = zero4();
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int ti = 0; ti < 4; ++ti) mma_ab2(kf[ti][kb], sf[kb], ks[ti]);
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float gam = kGated ? __expf(gg[ti][i]) : 1.f;
            rr[ti][i] = bb[ti][i] * (vv[ti][i] - gam * ks[ti][i]);
          }
        // U_new = T R (T lower triangular: row tile ti needs blocks <= ti / 2)
        Frag2<T> rf[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) rf[kb] = frag2_from_acc<T>(rr[2 * kb], rr[2 * kb + 1]);
        f32x4 un[4];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
          un[ti] = zero4();
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            if (kb <= ti / 2) mma_ab2(tf[ti][kb], rf[kb], un[ti]);
        }
        // publish U_new for the output, then
        // S' = gam_C S + K^T diag(gam_C / gam) U_new
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const Frag2<T> f = frag2_from_acc<T>(un[2 * kb], un[2 * kb + 1]);
          Ux[(kPlanes * kb) * kWave + lane] = f.hi;
          if constexpr (kSplit) Ux[(2 * kb + 1) * kWave + lane] = f.lo;
        }
        Frag2<T> ut[2];
        if constexpr (kGated) {
          float slo[2][4], shi[2][4];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              slo[kb][i] = __expf(gC - gg[2 * kb][i]);
              shi[kb][i] = __expf(gC - gg[2 * kb + 1][i]);
            }
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            ut[kb] = frag2_from_acc_scaled<T>(un[2 * kb], un[2 * kb + 1], slo[kb], shi[kb]);
          const float decC = __expf(gC);
#pragma unroll
          for (int tj = 0; tj < NKT; ++tj) S[tj] *= decC;
        } else {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) ut[kb] = frag2_from_acc<T>(un[2 * kb], un[2 * kb + 1]);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int tj = 0; tj < NKT; ++tj) mma_ab2(ktf[tj][kb], ut[kb], S[tj]);
      } else if constexpr (kGated) {
        // gated linear: S' = gam_C S + K^T diag(gam_C / gam) V; operand
        // element j of block kb is token 32 kb + kidx(g, j)
        const float gC = gs[C - 1];
        Frag2<T> vf[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const Frag<T> raw = frag_row(Vt + nt + 32 * kb, g);
#pragma unroll
          for (int j = 0; j < 8; ++j)
            vf[kb].set(j, to_f32(raw.v[j]) * __expf(gC - gs[32 * kb + kidx(g, j)]));
        }
        const float decC = __expf(gC);
#pragma unroll
        for (int tj = 0; tj < NKT; ++tj) S[tj] *= decC;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int tj = 0; tj < NKT; ++tj) mma_ab2(ktf[tj][kb], vf[kb], S[tj]);
      } else {
        // linear: S' = S + K^T V
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const Frag<T> vf = frag_row(Vt + nt + 32 * kb, g);
#pragma unroll
          for (int tj = 0; tj < NKT; ++tj) mma(ktf[tj][kb], vf, S[tj]);
        }
      }
    } else if (wave == 1) {
      // Q S for row tiles: wave 1 -> 0 and 3, wave 2 -> 1, wave 3 -> 2
      qs_rows<T, D, 2, 0, 3, LDQ>(Qs, Sx, qs, g, nq, lane);
    } else if (wave == 2) {
      qs_rows<T, D, 1, 1, 1, LDQ>(Qs, Sx, qs, g, nq, lane);
    } else {
      qs_rows<T, D, 1, 2, 2, LDQ>(Qs, Sx, qs, g, nq, lane);
    }
    __syncthreads();

    // ---------------- output (waves 1-3); wave 0 publishes the new state
    if (wave == 0) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const Frag2<T> f = frag2_from_acc<T>(S[2 * kb], S[2 * kb + 1]);
        Sx[(kPlanes * kb) * kWave + lane] = f.hi;
        if constexpr (kSplit) Sx[(2 * kb + 1) * kWave + lane] = f.lo;
      }
    } else {
      const size_t ob0 = row0 * D + col;
      const int nv = rows_of(c);
      if (wave == 1) {
        out_rows<T, D, MODE, 2, 0, 3, LDT>(Aq, Ux, Vt, gs, qs, out_, ob0, out_bf16, g, nt, lane, nv);
      } else if (wave == 2) {
        out_rows<T, D, MODE, 1, 1, 1, LDT>(Aq, Ux, Vt, gs, qs, out_, ob0, out_bf16, g, nt, lane, nv);
      } else {
        out_rows<T, D, MODE, 1, 2, 2, LDT>(Aq, Ux, Vt, gs, qs, out_, ob0, out_bf16, g, nt, lane, nv);
      }
    }
    __syncthreads();
  }

  if (wave == 0 && S_final) {
#pragma unroll
    for (int tj = 0; tj < NKT; ++tj)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S_final[sbase + (size_t)(16 * tj + 4 * g + i) * D + col] = S[tj][i];
  }
}

template <typename T, int D, int MODE>
hipError_t launch_one(const ChunkArgs& a, hipStream_t st) {
  const int BH = a.B * a.H;
  const dim3 grid((unsigned)((size_t)BH * (D / 16))), block(kThreads);
  chunk_kernel<T, D, MODE><<<grid, block, 0, st>>>(
      static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
      a.log_alpha, a.beta, a.S0, a.out, a.S_final, seq_map(a), BH, a.out_bf16 ? 1 : 0);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const ChunkArgs& a, hipStream_t st) {
  switch (a.mode) {
    case kModeLinear: return launch_one<T, D, kModeLinear>(a, st);
    case kModeDelta: return launch_one<T, D, kModeDelta>(a, st);
    case kModeGatedLinear: return launch_one<T, D, kModeGatedLinear>(a, st);
    default: return launch_one<T, D, kModeGatedDelta>(a, st);
  }
}

}  // namespace

hipError_t launch_chunk_seq(const ChunkArgs& a, hipStream_t st) {
  return a.d == 64 ? launch_d<float, 64>(a, st) : launch_d<float, 128>(a, st);
}

// bf16 inputs run the two-kernel path of la_chunk_pipe.hip; float inputs,
// which have no transposed LDS reads, run the phase-sequential kernel
// above.
bool chunk_needs_tsolve(const ChunkArgs& a) {
  return a.in_bf16 && (mode_erase(a.mode) || a.pro != 0);
}

size_t chunk_workspace_bytes(const ChunkArgs& a) {
  return a.in_bf16 ? chunk_pipe_workspace_bytes(a) : 0;
}

hipError_t launch_chunk(const ChunkArgs& a, hipStream_t st) {
  return a.in_bf16 ? launch_chunk_pipe(a, st) : launch_chunk_seq(a, st);
}

}  // namespace la
