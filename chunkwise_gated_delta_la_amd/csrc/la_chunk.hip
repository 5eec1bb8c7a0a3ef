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
//                       (delta modes) of K K^T on MFMA, with decay and mask
//   T        wave 0     the four 16 x 16 diagonal blocks of T by forward
//                       substitution (one lane per column)
//            waves 0-2  wave j: the blocks below the diagonal in column
//                       block j, T_ij = -T_ii sum_k A_ik T_kj, on MFMA
//   chain    wave 0     K S, R, U_new = T R, S update (MFMA)
//            waves 1-3  Q S for their row tiles (MFMA), from the entry
//                       state that wave 0 published in LDS
//   output   waves 1-3  O = diag(gam) Q S + Aqk U_new; wave 0 publishes the
//                       new state for the next chunk's Q S
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

// Rows of the f32x4 accumulator `a` this lane holds: 4 g + i.
// Number of the lower-triangular tile job p (0..9) -> (ti, tj), ti >= tj.
__device__ __forceinline__ void tri_tile(int p, int& ti, int& tj) {
  ti = p >= 6 ? 3 : p >= 3 ? 2 : p >= 1 ? 1 : 0;
  tj = p - ti * (ti + 1) / 2;
}

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

template <typename T, int D, int MODE>
__global__ __launch_bounds__(kThreads) void chunk_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    const float* __restrict__ S0, void* __restrict__ out_, float* __restrict__ S_final,
    int L, int BH, int out_bf16) {
  constexpr bool kDelta = MODE != kModeLinear;
  constexpr bool kGated = MODE == kModeGatedDelta;
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
  constexpr int VPR = D / PE;                    // 16-byte vectors per row
  constexpr int NVQ = C * VPR / kThreads;        // Q (and K) vectors per thread
  static_assert(NVQ * kThreads == C * VPR, "tile split");

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
  const int nt = n * LDT;       // row n of a K^T / V^T / T / Aqk tile

  const size_t hbase = (size_t)bh * L;          // first token row of the head

  // T as the A operand of U_new = T R: bf16 copy (split inputs) or Tf.
  const T* Top;
  if constexpr (kDelta && kSplit) Top = Tb;
  else Top = reinterpret_cast<const T*>(Tf);
  constexpr int LDTop = kDelta && kSplit ? LDT : LDF;

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
  u32x4 pv;                 // threads < 2 * C: one half-row (8 or 4 columns) of V
  float pla = 0.f, pb = 0.f;
  constexpr int VVR = 16 / PE;                   // V vectors per tile row
  auto load_chunk = [&](int c) {
    const size_t row0 = hbase + (size_t)c * C;
#pragma unroll
    for (int m = 0; m < NVQ; ++m) {
      const int p = tid + kThreads * m;
      const int r = p / VPR, cv = p % VPR;
      pq[m] = *reinterpret_cast<const u32x4*>(q + (row0 + r) * D + cv * PE);
      pk[m] = *reinterpret_cast<const u32x4*>(k + (row0 + r) * D + cv * PE);
    }
    if (tid < C * VVR) {
      const int r = tid / VVR, h = tid % VVR;
      pv = *reinterpret_cast<const u32x4*>(v + (row0 + r) * D + col0 + h * PE);
    }
    if (wave == 0) {
      if (kGated) pla = log_alpha[row0 + lane];
      if (kDelta) pb = beta[row0 + lane];
    }
  };

  const int NC = L / C;
  load_chunk(0);

  for (int c = 0; c < NC; ++c) {
    const size_t row0 = hbase + (size_t)c * C;

    // ---------------- stage: registers -> LDS, then prefetch the next chunk
#pragma unroll
    for (int m = 0; m < NVQ; ++m) {
      const int p = tid + kThreads * m;
      const int r = p / VPR, cv = p % VPR;
      *reinterpret_cast<u32x4*>(Qs + r * LDQ + cv * PE) = pq[m];
      *reinterpret_cast<u32x4*>(Ks + r * LDQ + cv * PE) = pk[m];
      if constexpr (kKt) {
        const T* e = reinterpret_cast<const T*>(&pk[m]);
#pragma unroll
        for (int j = 0; j < PE; ++j) Kt[(cv * PE + j) * LDT + r] = e[j];
      }
    }
    if (tid < C * VVR) {
      const int r = tid / VVR, h = tid % VVR;
      const T* e = reinterpret_cast<const T*>(&pv);
#pragma unroll
      for (int j = 0; j < PE; ++j) Vt[(h * PE + j) * LDT + r] = e[j];
    }
    if (wave == 0) {
      if constexpr (kGated) gs[lane] = wave_inclusive_scan(pla);
      else gs[lane] = 0.f;
      bs[lane] = pb;
    }
    if (c + 1 < NC) load_chunk(c + 1);
    __syncthreads();

    // ---------------- scores: lower tiles of Q K^T (-> Aq) and K K^T (-> As)
    {
      constexpr int kJobs = kDelta ? 20 : 10;
      for (int job = wave; job < kJobs; job += kWaves) {
        int ti, tj;
        tri_tile(job % 10, ti, tj);
        const T* X = job < 10 ? Qs : Ks;
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          mma(frag_row(X + (16 * LDQ) * ti + nq + 32 * kb, g),
              frag_row(Ks + (16 * LDQ) * tj + nq + 32 * kb, g), acc);
        const int cc = 16 * tj + n;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * ti + 4 * g + i;
          float decay = 1.f;
          if constexpr (kGated) decay = __expf(r >= cc ? gs[r] - gs[cc] : 0.f);
          if (job < 10) {
            const float x = r >= cc ? acc[i] * decay : 0.f;
            const T h = from_f32<T>(x);
            Aq[r * LDT + cc] = h;
            if constexpr (kSplit) Aq[C * LDT + r * LDT + cc] = from_f32<T>(x - to_f32(h));
          } else {
            As[r * LDF + cc] = r > cc ? bs[r] * acc[i] * decay : 0.f;
          }
        }
      }
      // The output reads Aq in 32-column blocks: the upper tiles (0, 1) and
      // (2, 3) that share such a block with a lower tile must be zero.
      if (wave == kWaves - 1) {
#pragma unroll
        for (int p = 0; p < kPlanes; ++p)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            Aq[p * C * LDT + r * LDT + 16 + n] = from_f32<T>(0.f);
            Aq[p * C * LDT + (32 + r) * LDT + 48 + n] = from_f32<T>(0.f);
          }
      }
    }
    __syncthreads();

    if constexpr (kDelta) {
      // ---------------- T = (I + A)^{-1}: diagonal blocks (wave 0)
      // Lane (g, n) solves column n of diagonal block g:
      //   x_r = [r == n] - sum_{i < r} A[16g + r][16g + i] x_i.
      if (wave == 0) {
        float x[16];
        const float* Ab = As + (16 * g) * LDF + 16 * g;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float s = r == n ? 1.f : 0.f;
#pragma unroll
          for (int i4 = 0; i4 < r; i4 += 4) {
            const f32x4 a4 = *reinterpret_cast<const f32x4*>(Ab + r * LDF + i4);
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (i4 + j < r) s = fmaf(-a4[j], x[i4 + j], s);
          }
          x[r] = s;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          Tf[(16 * g + r) * LDF + 16 * g + n] = x[r];
          if constexpr (kSplit) Tb[(16 * g + r) * LDT + 16 * g + n] = from_f32<T>(x[r]);
        }
      }
      __syncthreads();

      // ---------------- T: blocks below the diagonal, column block j = wave
      //   T_ij = -T_ii (sum_{k=j}^{i-1} A_ik T_kj),  i = j+1 .. 3
      if (wave < 3) {
        if (wave == 0) tcol_solve<T, 0, LDF, LDT>(As, Tf, Tb, g, n);
        else if (wave == 1) tcol_solve<T, 1, LDF, LDT>(As, Tf, Tb, g, n);
        else tcol_solve<T, 2, LDF, LDT>(As, Tf, Tb, g, n);
      } else {
        // Zero the upper blocks (0, 1) and (2, 3) of T that U_new = T R
        // reads as part of a 32-column block.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * g + i;
          if constexpr (kSplit) {
            Tb[r * LDT + 16 + n] = from_f32<T>(0.f);
            Tb[(32 + r) * LDT + 48 + n] = from_f32<T>(0.f);
          } else {
            Tf[r * LDF + 16 + n] = 0.f;
            Tf[(32 + r) * LDF + 48 + n] = 0.f;
          }
        }
      }
      __syncthreads();
    }

    // ---------------- chain (wave 0) and Q S (waves 1-3)
    f32x4 qs[2];
    if (wave == 0) {
      f32x4 un[4];
      if constexpr (kDelta) {
        Frag2<T> sf[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) sf[kb] = frag2_from_acc<T>(S[2 * kb], S[2 * kb + 1]);
        // R = diag(beta) (V - diag(gam) K S), rows 16 ti + 4 g + i
        f32x4 rr[4];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
          f32x4 ks = zero4();
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
            mma_ab2(frag_row(Ks + (16 * LDQ) * ti + nq + 32 * kb, g), sf[kb], ks);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * ti + 4 * g + i;
            const float gam = kGated ? __expf(gs[r]) : 1.f;
            rr[ti][i] = bs[r] * (to_f32(Vt[nt + r]) - gam * ks[i]);
          }
        }
        // U_new = T R (T lower triangular: row tile ti needs blocks <= ti / 2)
        Frag2<T> rf[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) rf[kb] = frag2_from_acc<T>(rr[2 * kb], rr[2 * kb + 1]);
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
          un[ti] = zero4();
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            if (kb == 1 && ti < 2) continue;
            mma_ab2(frag_row(Top + (16 * LDTop) * ti + n * LDTop + 32 * kb, g), rf[kb], un[ti]);
          }
        }
        // publish U_new for the output, then S' = gam_C S + K^T diag(gam_C / gam) U_new
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const Frag2<T> f = frag2_from_acc<T>(un[2 * kb], un[2 * kb + 1]);
          Ux[(kPlanes * kb) * kWave + lane] = f.hi;
          if constexpr (kSplit) Ux[(2 * kb + 1) * kWave + lane] = f.lo;
        }
        Frag2<T> ut[2];
        if constexpr (kGated) {
          const float gC = gs[C - 1];
          float slo[2][4], shi[2][4];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              slo[kb][i] = __expf(gC - gs[32 * kb + 4 * g + i]);
              shi[kb][i] = __expf(gC - gs[32 * kb + 16 + 4 * g + i]);
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
        for (int tj = 0; tj < NKT; ++tj)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            Frag<T> kt;
            if constexpr (kKt) kt = frag_row(Kt + (16 * LDT) * tj + nt + 32 * kb, g);
            else kt = frag_col(Ks + 32 * kb * LDQ + 16 * tj + n, LDQ, g);
            mma_ab2(kt, ut[kb], S[tj]);
          }
      } else {
        // linear: S' = S + K^T V
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const Frag<T> vf = frag_row(Vt + nt + 32 * kb, g);
#pragma unroll
          for (int tj = 0; tj < NKT; ++tj) {
            Frag<T> kt;
            if constexpr (kKt) kt = frag_row(Kt + (16 * LDT) * tj + nt + 32 * kb, g);
            else kt = frag_col(Ks + 32 * kb * LDQ + 16 * tj + n, LDQ, g);
            mma(kt, vf, S[tj]);
          }
        }
      }
    } else {
      // Q S for row tiles: wave 1 -> 0 and 3, wave 2 -> 1, wave 3 -> 2
      Frag2<T> sx[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        sx[kb].hi = Sx[(kPlanes * kb) * kWave + lane];
        if constexpr (kSplit) sx[kb].lo = Sx[(2 * kb + 1) * kWave + lane];
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int ti = u == 0 ? wave - 1 : 3;
        qs[u] = zero4();
        if (u == 1 && wave != 1) continue;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          mma_ab2(frag_row(Qs + (16 * LDQ) * ti + nq + 32 * kb, g), sx[kb], qs[u]);
      }
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
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (u == 1 && wave != 1) continue;
        const int ti = u == 0 ? wave - 1 : 3;
        f32x4 o = qs[u];
        if constexpr (kGated) {
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] *= __expf(gs[16 * ti + 4 * g + i]);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (kb == 1 && ti < 2) continue;     // Aq is zero above the diagonal
          Frag2<T> a;
          a.hi = frag_row(Aq + (16 * LDT) * ti + nt + 32 * kb, g);
          if constexpr (kSplit) a.lo = frag_row(Aq + C * LDT + (16 * LDT) * ti + nt + 32 * kb, g);
          if constexpr (kDelta) {
            mma_a2b2(a, uf[kb], o);
          } else {
            // linear: V is exact in the input type
            if constexpr (kSplit) mma(a.lo, uf[kb].hi, o);
            mma(a.hi, uf[kb].hi, o);
          }
        }
        const size_t ob = (row0 + 16 * ti + 4 * g) * D + col;
        if (out_bf16) {
          __bf16* out = static_cast<__bf16*>(out_);
#pragma unroll
          for (int i = 0; i < 4; ++i) out[ob + (size_t)i * D] = (__bf16)o[i];
        } else {
          float* out = static_cast<float*>(out_);
#pragma unroll
          for (int i = 0; i < 4; ++i) out[ob + (size_t)i * D] = o[i];
        }
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
      a.log_alpha, a.beta, a.S0, a.out, a.S_final, a.L, BH, a.out_bf16 ? 1 : 0);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const ChunkArgs& a, hipStream_t st) {
  switch (a.mode) {
    case kModeLinear: return launch_one<T, D, kModeLinear>(a, st);
    case kModeDelta: return launch_one<T, D, kModeDelta>(a, st);
    default: return launch_one<T, D, kModeGatedDelta>(a, st);
  }
}

}  // namespace

hipError_t launch_chunk(const ChunkArgs& a, hipStream_t st) {
  if (a.in_bf16) return a.d == 64 ? launch_d<__bf16, 64>(a, st) : launch_d<__bf16, 128>(a, st);
  return a.d == 64 ? launch_d<float, 64>(a, st) : launch_d<float, 128>(a, st);
}

}  // namespace la
