// Inter-chunk kernel: carries the state across chunks and produces the
// output, sequential over the chunks of one sequence.
//
// For chunk t with entry state S (dk x dv) and the intra-chunk quantities
// made by the WY kernel (W, U, Aqk, g):
//
//   U_new = U - W S                                   (true update rows)
//   O     = diag(exp(g)) Q S + Aqk U_new
//   S'    = exp(g_C) S + (diag(exp(g_C - g)) K)^T U_new
//
// Plain linear attention uses U_new = V, g = 0 (no W):
//   O = Q S + ((Q K^T) * M) V,   S' = S + K^T V
// which is the chunkwise form of "FWP分块并行机制" in the hybrid-attention
// notes "混合注意力学习(1): 线性注意力" (and "FLASH" in "LinearAttention 概述").
// The delta modes follow "重新定义降低内存占用" of the same notes: only W and
// U of the chunk are needed, never a past per-token state.
//
// Mapping to gfx950.  Columns of the state are independent, so the state is
// split into 16-column tiles: one wave owns one tile (all dk rows) of one
// (batch, head) and keeps it in MFMA accumulator registers for the whole
// sequence.  A workgroup of NW waves owns NW adjacent tiles and stages the
// chunk's Q, W, K, Aqk and its U columns in LDS once for all its waves.  The
// accumulator layout doubles as the B-operand layout (see la_device.hpp), so
// S feeds W S and Q S, and U_new feeds Aqk U_new and K^T U_new, straight from
// registers; only a float -> bf16 conversion sits between the products.
#include "la_device.hpp"
#include "la_kernels.hpp"

namespace la {
namespace {

constexpr int C = 64;

template <typename T, int D, int MODE, int NW>
__global__ __launch_bounds__(64 * NW) void state_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ Win,
    const T* __restrict__ Uin, const T* __restrict__ Aqk, const float* __restrict__ G,
    const float* __restrict__ S0, T* __restrict__ out, float* __restrict__ S_final,
    int L) {
  constexpr bool kDelta = MODE != kModeLinear;
  constexpr bool kGated = MODE == kModeGatedDelta;
  constexpr int NT = 64 * NW;                 // threads
  constexpr int NCOL = 16 * NW;               // state columns per workgroup
  constexpr int LD = D + 16 / sizeof(T);      // LDS row pitch, d-wide tiles
  constexpr int LDA = C + 16 / sizeof(T);     // LDS row pitch, Aqk
  constexpr int LDU = NCOL + 16 / sizeof(T);  // LDS row pitch, U columns
  constexpr int NKT = D / 16;                 // 16-row tiles of dk
  constexpr int NKB = D / 32;                 // 32-deep blocks of dk

  __shared__ __attribute__((aligned(16))) T Qs[C * LD];
  __shared__ __attribute__((aligned(16))) T Ks[C * LD];
  __shared__ __attribute__((aligned(16))) T Ws[kDelta ? C * LD : 8];
  __shared__ __attribute__((aligned(16))) T As[C * LDA];
  __shared__ __attribute__((aligned(16))) T Us[C * LDU];
  __shared__ float gs[C];

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int g = lane / 16;
  const int n = lane % 16;

  constexpr int kBlocksPerHead = D / NCOL;
  const size_t bh = blockIdx.x / kBlocksPerHead;
  const int cb = blockIdx.x % kBlocksPerHead;
  const int col0 = cb * NCOL;                 // first column of the workgroup
  const int col = col0 + 16 * wave + n;       // this lane's column

  // State tile: S[tj][i] = S[16 tj + 4 g + i][col].
  f32x4 S[NKT];
  const size_t sbase = bh * (size_t)D * D;
#pragma unroll
  for (int tj = 0; tj < NKT; ++tj)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      S[tj][i] = S0 ? S0[sbase + (size_t)(16 * tj + 4 * g + i) * D + col] : 0.f;

  const int NC = L / C;
  for (int c = 0; c < NC; ++c) {
    const size_t row0 = bh * (size_t)L + (size_t)c * C;
    stage_tile<T, C, D, LD, NT>(Qs, q + row0 * D, D, tid);
    stage_tile<T, C, D, LD, NT>(Ks, k + row0 * D, D, tid);
    if (kDelta) stage_tile<T, C, D, LD, NT>(Ws, Win + row0 * D, D, tid);
    stage_tile<T, C, C, LDA, NT>(As, Aqk + (bh * (size_t)NC + c) * (C * C), C, tid);
    stage_tile<T, C, NCOL, LDU, NT>(Us, Uin + row0 * D + col0, D, tid);
    if (kGated && tid < C) gs[tid] = G[row0 + tid];
    __syncthreads();

    // S as the B operand of the products over dk.
    Frag<T> sf[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sf[kb] = frag_from_acc<T>(S[2 * kb], S[2 * kb + 1]);

    // U_new = U - W S  (linear: V), rows 16 ti + 4 g + i.
    f32x4 un[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      f32x4 ws = zero4();
      if (kDelta) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          mma(frag_row(Ws + (16 * ti + n) * LD + 32 * kb, g), sf[kb], ws);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        un[ti][i] = to_f32(Us[(16 * ti + 4 * g + i) * LDU + 16 * wave + n]) - ws[i];
    }

    // O = diag(exp(g)) Q S + Aqk U_new
    f32x4 o[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      o[ti] = zero4();
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        mma(frag_row(Qs + (16 * ti + n) * LD + 32 * kb, g), sf[kb], o[ti]);
      if (kGated) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[ti][i] *= __expf(gs[16 * ti + 4 * g + i]);
      }
    }
    Frag<T> uf[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) uf[kb] = frag_from_acc<T>(un[2 * kb], un[2 * kb + 1]);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb == 1 && ti < 2) continue;   // Aqk is zero above the diagonal
        mma(frag_row(As + (16 * ti + n) * LDA + 32 * kb, g), uf[kb], o[ti]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        out[(row0 + 16 * ti + 4 * g + i) * D + col] = from_f32<T>(o[ti][i]);
    }

    // S' = exp(g_C) S + K^T diag(exp(g_C - g)) U_new
    if (kGated) {
      const float gC = gs[C - 1];
      const float decC = __expf(gC);
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
        uf[kb] = frag_from_acc_scaled<T>(un[2 * kb], un[2 * kb + 1], slo[kb], shi[kb]);
#pragma unroll
      for (int tj = 0; tj < NKT; ++tj) S[tj] *= decC;
    }
#pragma unroll
    for (int tj = 0; tj < NKT; ++tj)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        mma(frag_col(Ks + 32 * kb * LD + 16 * tj + n, LD, g), uf[kb], S[tj]);
    __syncthreads();
  }

  if (S_final) {
#pragma unroll
    for (int tj = 0; tj < NKT; ++tj)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S_final[sbase + (size_t)(16 * tj + 4 * g + i) * D + col] = S[tj][i];
  }
}

template <typename T, int D, int MODE, int NW>
void launch_one(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t st) {
  const dim3 grid((unsigned)((size_t)a.B * a.H * (D / (16 * NW)))), block(64 * NW);
  const bool delta = MODE != kModeLinear;
  state_kernel<T, D, MODE, NW><<<grid, block, 0, st>>>(
      static_cast<const T*>(a.q), static_cast<const T*>(a.k),
      static_cast<const T*>(ws.W),
      static_cast<const T*>(delta ? ws.U : a.v), static_cast<const T*>(ws.Aqk), ws.G,
      a.S0, static_cast<T*>(a.out), a.S_final, a.L);
}

// Waves per workgroup: as many as keep at least one workgroup per CU busy
// (256 CUs), since fewer waves per workgroup means more redundant staging.
inline int pick_nw(const ChunkArgs& a) {
  const long heads = (long)a.B * a.H;
  const int tiles = a.d / 16;
  int nw = 4;
  while (nw > 1 && heads * (tiles / nw) < 256) nw /= 2;
  return nw;
}

template <typename T, int D, int MODE>
void launch_mode(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t st) {
  switch (pick_nw(a)) {
    case 4: launch_one<T, D, MODE, 4>(a, ws, st); break;
    case 2: launch_one<T, D, MODE, 2>(a, ws, st); break;
    default: launch_one<T, D, MODE, 1>(a, ws, st); break;
  }
}

template <typename T, int D>
void launch_td(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t st) {
  switch (a.mode) {
    case kModeLinear: launch_mode<T, D, kModeLinear>(a, ws, st); break;
    case kModeDelta: launch_mode<T, D, kModeDelta>(a, ws, st); break;
    default: launch_mode<T, D, kModeGatedDelta>(a, ws, st); break;
  }
}

}  // namespace

hipError_t launch_state(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t st) {
  if (a.bf16) {
    if (a.d == 64) launch_td<__bf16, 64>(a, ws, st);
    else launch_td<__bf16, 128>(a, ws, st);
  } else {
    if (a.d == 64) launch_td<float, 64>(a, ws, st);
    else launch_td<float, 128>(a, ws, st);
  }
  return hipGetLastError();
}

}  // namespace la
