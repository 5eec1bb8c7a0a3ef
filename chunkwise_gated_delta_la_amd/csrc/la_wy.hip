// Intra-chunk kernel: everything of a chunk that does not depend on the
// carried state, fully parallel over (batch, head, chunk).
//
// For one chunk of C = 64 rows with keys K, values V, queries Q (C x d),
// write strengths beta and log-decays log_alpha:
//
//   g_r     = sum_{i <= r} log_alpha_i            (in-chunk cumulative decay)
//   Aqk     = (Q K^T) * M * Gamma,  Gamma_ri = exp(g_r - g_i), M_ri = [i <= r]
//   A       = strict_lower(diag(beta) (K K^T) * Gamma)
//   T       = (I + A)^{-1}                        (unit lower-triangular)
//   W       = T diag(beta * exp(g)) K,   U = T diag(beta) V
//
// This is the inductive redefinition of the per-token update vectors
// ("重新定义降低内存占用") in its WY/UT form ("HouseHolder变换和WY表示"), both
// sections of the hybrid-attention notes "混合注意力学习(1): 线性注意力",
// with the scalar decay of "Gated DeltaNet" folded in through Gamma and
// exp(g).  For plain linear attention only Aqk = (Q K^T) * M is needed (the
// masked intra-chunk product of "FWP分块并行机制" in the same notes).
//
// Mapping to gfx950.  One 256-thread workgroup (4 waves) per chunk.  Q, K, V
// are staged in LDS with 16-byte loads.  The two C x C score products and
// the two C x d products with T run on MFMA, float accumulate; only the
// tiles on or below the diagonal are formed.  T is solved in float by
// blocked forward substitution in LDS: 16-row blocks; the off-diagonal part
// of a block row is one small product over the rows already solved, the
// 16 x 16 diagonal block a right-looking substitution held in registers
// (one lane per column), so the serial depth is 16 per block row, not 64.
//
// Precision (bf16 inputs).  Q, K, V are exact bf16 MFMA operands; the
// float matrices T diag(beta exp(g)) and T diag(beta) enter the W and U
// products split into bf16 hi + lo parts, so W and U carry float accuracy.
// U is stored as float, Aqk as two bf16 planes (hi, lo), W as bf16 (its
// rounding is the one intermediate rounding kept on this path).
#include "la_device.hpp"
#include "la_kernels.hpp"

namespace la {
namespace {

constexpr int C = 64;
constexpr int kThreads = 256;

template <typename T, int D, int MODE>
__global__ __launch_bounds__(kThreads) void wy_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    T* __restrict__ Wout, float* __restrict__ Uout, T* __restrict__ Aqk_out,
    float* __restrict__ Gout, int L) {
  constexpr bool kDelta = MODE != kModeLinear;
  constexpr bool kSplit = IsBf16<T>::value;
  constexpr int kPlanes = kSplit ? 2 : 1;      // Aqk planes: hi (, lo)
  constexpr int LD = D + 16 / sizeof(T);       // LDS row pitch (elements)
  constexpr int LDF = C + 4;                   // float matrices' row pitch
  constexpr int NDT = D / 16;                  // 16-wide column tiles of d
  constexpr int kWaves = kThreads / kWave;

  __shared__ __attribute__((aligned(16))) T Ks[C * LD];
  __shared__ __attribute__((aligned(16))) T Qs[C * LD];
  __shared__ __attribute__((aligned(16))) T Vs[kDelta ? C * LD : 8];
  __shared__ __attribute__((aligned(16))) float As[kDelta ? C * LDF : 4];
  __shared__ __attribute__((aligned(16))) float Ts[kDelta ? C * LDF : 4];
  __shared__ __attribute__((aligned(16))) float gs[C];
  __shared__ __attribute__((aligned(16))) float bs[C];    // beta_r
  __shared__ __attribute__((aligned(16))) float bgs[C];   // beta_r * exp(g_r)

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int g = lane / 16;
  const int n = lane % 16;

  const int NC = L / C;
  const size_t chunk = blockIdx.x;
  const size_t bh = chunk / NC;
  const size_t row0 = bh * (size_t)L + (chunk % NC) * (size_t)C;

  stage_tile<T, C, D, LD, kThreads>(Ks, k + row0 * D, D, tid);
  stage_tile<T, C, D, LD, kThreads>(Qs, q + row0 * D, D, tid);
  if (kDelta) stage_tile<T, C, D, LD, kThreads>(Vs, v + row0 * D, D, tid);
  if (wave == 0) {
    float la = 0.f;
    if (MODE == kModeGatedDelta) la = log_alpha[row0 + lane];
    const float gl = wave_inclusive_scan(la);
    gs[lane] = gl;
    if (kDelta) {
      const float b = beta[row0 + lane];
      bs[lane] = b;
      bgs[lane] = MODE == kModeGatedDelta ? b * __expf(gl) : b;
      Gout[row0 + lane] = gl;
    }
  }
  __syncthreads();

  // ---- score products: lower-triangle tiles (ti >= tj) of Q K^T and K K^T.
  // Job j < 10 is tile j of Q K^T, job 10 + j the same tile of K K^T.
  // The consumer reads Aqk in 32-column blocks, so the two upper tiles that
  // share such a block with a lower tile, (0, 1) and (2, 3), are written as
  // zeros; the other upper tiles are never read.
  constexpr int kJobs = kDelta ? 20 : 10;
  T* Aqk = Aqk_out + chunk * (size_t)(kPlanes * C * C);
  if (wave == kWaves - 1) {
#pragma unroll
    for (int p = 0; p < kPlanes; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;
        Aqk[p * C * C + r * C + 16 + n] = from_f32<T>(0.f);
        Aqk[p * C * C + (32 + r) * C + 48 + n] = from_f32<T>(0.f);
      }
  }
  for (int job = wave; job < kJobs; job += kWaves) {
    const int p = job % 10;
    const int ti = p >= 6 ? 3 : p >= 3 ? 2 : p >= 1 ? 1 : 0;
    const int tj = p - ti * (ti + 1) / 2;
    const T* X = job < 10 ? Qs : Ks;
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) {
      const Frag<T> a = frag_row(X + (16 * ti + n) * LD + 32 * kb, g);
      const Frag<T> b = frag_row(Ks + (16 * tj + n) * LD + 32 * kb, g);
      mma(a, b, acc);
    }
    const int col = 16 * tj + n;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * ti + 4 * g + i;
      float decay = 1.f;
      if (MODE == kModeGatedDelta) decay = __expf(r >= col ? gs[r] - gs[col] : 0.f);
      if (job < 10) {
        const float x = r >= col ? acc[i] * decay : 0.f;
        const T h = from_f32<T>(x);
        Aqk[r * C + col] = h;
        if (kSplit) Aqk[C * C + r * C + col] = from_f32<T>(x - to_f32(h));
      } else {
        As[r * LDF + col] = r > col ? bs[r] * acc[i] * decay : 0.f;
      }
    }
  }
  if (!kDelta) return;
  __syncthreads();

  // ---- T = (I + A)^{-1}, blocked forward substitution over 16-row blocks.
  for (int R = 0; R < 4; ++R) {
    {
      // Rows 16R..16R+15, all 64 columns: X = E - A[rows, :16R] T[:16R, :]
      const int rr = tid / 16, c4 = 4 * (tid % 16);
      const int r = 16 * R + rr;
      float x[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) x[c] = (r == c4 + c) ? 1.f : 0.f;
      for (int i = 0; i < 16 * R; ++i) {
        const float a = As[r * LDF + i];
        const f32x4 t4 = *reinterpret_cast<const f32x4*>(Ts + i * LDF + c4);
#pragma unroll
        for (int c = 0; c < 4; ++c) x[c] = fmaf(-a, t4[c], x[c]);
      }
      *reinterpret_cast<f32x4*>(Ts + r * LDF + c4) = f32x4{x[0], x[1], x[2], x[3]};
    }
    __syncthreads();
    if (wave == 0) {
      // Diagonal block: y_rr = X_rr - sum_{i<rr} A[16R+rr][16R+i] y_i, one
      // lane per column, right-looking so each y_i updates the later rows
      // as soon as it is final.
      float y[16];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) y[rr] = Ts[(16 * R + rr) * LDF + lane];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
#pragma unroll
        for (int rr = i + 1; rr < 16; ++rr)
          y[rr] = fmaf(-As[(16 * R + rr) * LDF + 16 * R + i], y[i], y[rr]);
      }
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) Ts[(16 * R + rr) * LDF + lane] = y[rr];
    }
    __syncthreads();
  }

  // ---- W = (T diag(beta exp(g))) K and U = (T diag(beta)) V.
  // The bracketed float matrices are split A operands; K and V columns are
  // exact B operands.  Wave w owns column tiles tj = w, w + 4, ...; T is
  // lower triangular, so row tile ti needs contraction block 1 only when
  // ti >= 2.
  constexpr int kTPW = (NDT + kWaves - 1) / kWaves;   // column tiles per wave
  Frag<T> bk[kTPW][2], bv[kTPW][2];
#pragma unroll
  for (int u = 0; u < kTPW; ++u) {
    const int col = 16 * (wave + kWaves * u) + n;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bk[u][kb] = frag_col(Ks + 32 * kb * LD + col, LD, g);
      bv[u][kb] = frag_col(Vs + 32 * kb * LD + col, LD, g);
    }
  }
#pragma unroll
  for (int ti = 0; ti < 4; ++ti) {
    f32x4 aw[kTPW], au[kTPW];
#pragma unroll
    for (int u = 0; u < kTPW; ++u) aw[u] = au[u] = zero4();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (kb == 1 && ti < 2) continue;
      const float* trow = Ts + (16 * ti + n) * LDF + 32 * kb;
      const Frag2<T> tw = frag2_row_scaled<T>(trow, g, bgs + 32 * kb);
      const Frag2<T> tu = frag2_row_scaled<T>(trow, g, bs + 32 * kb);
#pragma unroll
      for (int u = 0; u < kTPW; ++u) {
        if (wave + kWaves * u >= NDT) continue;
        mma_ab2(bk[u][kb], tw, aw[u]);   // W^T tile = K^T (T diag(beta e^g))^T
        mma_ab2(bv[u][kb], tu, au[u]);   // U^T tile = V^T (T diag(beta))^T
      }
    }
    // The products above are transposed (A = K^T columns, B = split T
    // rows), so lane (g, n) holds chunk row 16 ti + n, columns
    // 16 tj + 4 g .. + 3: one contiguous 4-element store per lane.
#pragma unroll
    for (int u = 0; u < kTPW; ++u) {
      if (wave + kWaves * u >= NDT) continue;
      const size_t off = (row0 + 16 * ti + n) * D + 16 * (wave + kWaves * u) + 4 * g;
      *reinterpret_cast<f32x4*>(Uout + off) = au[u];
      if constexpr (kSplit) {
        bf16x4 w4;
#pragma unroll
        for (int i = 0; i < 4; ++i) w4[i] = (__bf16)aw[u][i];
        *reinterpret_cast<bf16x4*>(Wout + off) = w4;
      } else {
        *reinterpret_cast<f32x4*>(Wout + off) = aw[u];
      }
    }
  }
}

template <typename T, int D>
hipError_t launch_td(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t st) {
  const dim3 grid((unsigned)((size_t)a.B * a.H * (a.L / C))), block(kThreads);
  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  T* W = static_cast<T*>(ws.W);
  T* A = static_cast<T*>(ws.Aqk);
  switch (a.mode) {
    case kModeLinear:
      wy_kernel<T, D, kModeLinear><<<grid, block, 0, st>>>(q, k, v, a.log_alpha, a.beta,
                                                           W, ws.U, A, ws.G, a.L);
      break;
    case kModeDelta:
      wy_kernel<T, D, kModeDelta><<<grid, block, 0, st>>>(q, k, v, a.log_alpha, a.beta,
                                                          W, ws.U, A, ws.G, a.L);
      break;
    default:
      wy_kernel<T, D, kModeGatedDelta><<<grid, block, 0, st>>>(q, k, v, a.log_alpha,
                                                               a.beta, W, ws.U, A, ws.G, a.L);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_wy(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t st) {
  if (a.in_bf16) return a.d == 64 ? launch_td<__bf16, 64>(a, ws, st)
                                  : launch_td<__bf16, 128>(a, ws, st);
  return a.d == 64 ? launch_td<float, 64>(a, ws, st) : launch_td<float, 128>(a, ws, st);
}

}  // namespace la
