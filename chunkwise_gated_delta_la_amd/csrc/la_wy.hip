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
// the two C x d products with T run on MFMA (bf16 in, float accumulate);
// only the tiles on or below the diagonal are formed.  T is solved in float
// by blocked forward substitution in LDS: 16-row blocks; the off-diagonal
// part of a block row is one small product over the rows already solved,
// the 16 x 16 diagonal block is a right-looking substitution held in
// registers (one lane per column), so the serial depth is 16 per block row
// rather than 64.
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
    T* __restrict__ Wout, T* __restrict__ Uout, T* __restrict__ Aqk_out,
    float* __restrict__ Gout, int L) {
  constexpr bool kDelta = MODE != kModeLinear;
  constexpr int LD = D + 16 / sizeof(T) * 1;   // LDS row pitch (elements)
  constexpr int LDF = C + 4;                   // float matrices' row pitch
  constexpr int NDT = D / 16;                  // 16-wide column tiles of d

  __shared__ __attribute__((aligned(16))) T Ks[C * LD];
  __shared__ __attribute__((aligned(16))) T Qs[C * LD];
  __shared__ __attribute__((aligned(16))) T Vs[kDelta ? C * LD : 8];
  __shared__ __attribute__((aligned(16))) float As[kDelta ? C * LDF : 4];
  __shared__ __attribute__((aligned(16))) float Ts[kDelta ? C * LDF : 4];
  __shared__ float gs[C];
  __shared__ float bs[C];    // beta_r
  __shared__ float bgs[C];   // beta_r * exp(g_r)

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
  constexpr int kJobs = kDelta ? 20 : 10;
  T* Aqk = Aqk_out + chunk * (size_t)(C * C);
  for (int job = wave; job < kJobs; job += kThreads / kWave) {
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
        Aqk[r * C + col] = from_f32<T>(r >= col ? acc[i] * decay : 0.f);
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

  // ---- W = T diag(beta exp(g)) K and U = T diag(beta) V.
  // Wave w owns column tiles tj = w, w + 4, ... of d; T is lower triangular
  // so row tile ti only needs contraction block 1 when ti >= 2.
  for (int tj = wave; tj < NDT; tj += kThreads / kWave) {
    const int col = 16 * tj + n;
    Frag<T> bk[2], bv[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bk[kb] = frag_col_scaled(Ks + 32 * kb * LD + col, LD, g, bgs + 32 * kb);
      bv[kb] = frag_col_scaled(Vs + 32 * kb * LD + col, LD, g, bs + 32 * kb);
    }
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      f32x4 aw = zero4(), au = zero4();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb == 1 && ti < 2) continue;
        const Frag<T> t = frag_row_cvt<T>(Ts + (16 * ti + n) * LDF + 32 * kb, g);
        mma(t, bk[kb], aw);
        mma(t, bv[kb], au);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const size_t r = row0 + 16 * ti + 4 * g + i;
        Wout[r * D + col] = from_f32<T>(aw[i]);
        Uout[r * D + col] = from_f32<T>(au[i]);
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
  T* U = static_cast<T*>(ws.U);
  T* A = static_cast<T*>(ws.Aqk);
  switch (a.mode) {
    case kModeLinear:
      wy_kernel<T, D, kModeLinear><<<grid, block, 0, st>>>(q, k, v, a.log_alpha, a.beta,
                                                           W, U, A, ws.G, a.L);
      break;
    case kModeDelta:
      wy_kernel<T, D, kModeDelta><<<grid, block, 0, st>>>(q, k, v, a.log_alpha, a.beta,
                                                          W, U, A, ws.G, a.L);
      break;
    default:
      wy_kernel<T, D, kModeGatedDelta><<<grid, block, 0, st>>>(q, k, v, a.log_alpha,
                                                               a.beta, W, U, A, ws.G, a.L);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_wy(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t st) {
  if (a.bf16) return a.d == 64 ? launch_td<__bf16, 64>(a, ws, st)
                               : launch_td<__bf16, 128>(a, ws, st);
  return a.d == 64 ? launch_td<float, 64>(a, ws, st) : launch_td<float, 128>(a, ws, st);
}

}  // namespace la
