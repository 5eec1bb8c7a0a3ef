// Inter-chunk kernel: carries the state across chunks and produces the
// output, sequential over the chunks of one sequence.
//
// For chunk t with entry state S (dk x dv) and the intra-chunk quantities
// made by the WY kernel (W, U, Aqk, g):
//
//   U_new = U - W S                                   (true update rows)
//   O     = diag(exp(g)) Q S + Aqk U_new
//   S'    = exp(g_C) S + K^T diag(exp(g_C - g)) U_new
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
// registers.
//
// Precision (bf16 inputs).  S and U_new are float accumulators; where they
// feed a product they are split into bf16 hi + lo operands, and Aqk arrives
// as hi + lo planes, so every product carries float accuracy except the
// bf16 rounding of W.  The output is rounded once, to the output type.
#include "la_device.hpp"
#include "la_kernels.hpp"

namespace la {
namespace {

constexpr int C = 64;

template <typename T, typename TO, int D, int MODE, int NW>
__global__ __launch_bounds__(64 * NW) void state_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ Win,
    const void* __restrict__ Uin_, const T* __restrict__ Aqk,
    const float* __restrict__ G, const float* __restrict__ S0, TO* __restrict__ out,
    float* __restrict__ S_final, int L) {
  constexpr bool kDelta = MODE != kModeLinear;
  constexpr bool kGated = MODE == kModeGatedDelta;
  constexpr bool kSplit = IsBf16<T>::value;
  constexpr int kPlanes = kSplit ? 2 : 1;
  // U columns: float update rows in the delta modes, the values themselves
  // (input type) in linear mode.
  using UT = typename std::conditional<kDelta, float, T>::type;
  constexpr int NT = 64 * NW;                 // threads
  constexpr int NCOL = 16 * NW;               // state columns per workgroup
  constexpr int LD = D + 16 / sizeof(T);      // LDS row pitch, d-wide tiles
  constexpr int LDA = C + 16 / sizeof(T);     // LDS row pitch, Aqk planes
  constexpr int LDU = NCOL + 16 / sizeof(UT); // LDS row pitch, U columns
  constexpr int NKT = D / 16;                 // 16-row tiles of dk
  constexpr int NKB = D / 32;                 // 32-deep blocks of dk

  __shared__ __attribute__((aligned(16))) T Qs[C * LD];
  __shared__ __attribute__((aligned(16))) T Ks[C * LD];
  __shared__ __attribute__((aligned(16))) T Ws[kDelta ? C * LD : 8];
  __shared__ __attribute__((aligned(16))) T As[kPlanes * C * LDA];
  __shared__ __attribute__((aligned(16))) UT Us[C * LDU];
  __shared__ __attribute__((aligned(16))) float gs[C];

  const UT* Uin = static_cast<const UT*>(Uin_);
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
    const T* ap = Aqk + (bh * (size_t)NC + c) * (size_t)(kPlanes * C * C);
#pragma unroll
    for (int p = 0; p < kPlanes; ++p)
      stage_tile<T, C, C, LDA, NT>(As + p * C * LDA, ap + p * C * C, C, tid);
    stage_tile<UT, C, NCOL, LDU, NT>(Us, Uin + row0 * D + col0, D, tid);
    if (kGated && tid < C) gs[tid] = G[row0 + tid];
    __syncthreads();

    // S as the (split) B operand of the products over dk.
    Frag2<T> sf[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sf[kb] = frag2_from_acc<T>(S[2 * kb], S[2 * kb + 1]);

    // U_new = U - W S  (linear: V), rows 16 ti + 4 g + i.
    f32x4 un[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      f32x4 ws = zero4();
      if constexpr (kDelta) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          mma_ab2(frag_row(Ws + (16 * ti + n) * LD + 32 * kb, g), sf[kb], ws);
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
        mma_ab2(frag_row(Qs + (16 * ti + n) * LD + 32 * kb, g), sf[kb], o[ti]);
      if constexpr (kGated) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[ti][i] *= __expf(gs[16 * ti + 4 * g + i]);
      }
    }
    Frag2<T> uf[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) uf[kb] = frag2_from_acc<T>(un[2 * kb], un[2 * kb + 1]);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb == 1 && ti < 2) continue;   // Aqk is zero above the diagonal
        Frag2<T> a;
        a.hi = frag_row(As + (16 * ti + n) * LDA + 32 * kb, g);
        if constexpr (kSplit) a.lo = frag_row(As + C * LDA + (16 * ti + n) * LDA + 32 * kb, g);
        if constexpr (kDelta) {
          mma_a2b2(a, uf[kb], o[ti]);
        } else {
          // linear mode: U_new = V is exact in the input type (uf.lo = 0)
          if constexpr (kSplit) mma(a.lo, uf[kb].hi, o[ti]);
          mma(a.hi, uf[kb].hi, o[ti]);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        out[(row0 + 16 * ti + 4 * g + i) * D + col] = from_f32<TO>(o[ti][i]);
    }

    // S' = exp(g_C) S + K^T diag(exp(g_C - g)) U_new
    if constexpr (kGated) {
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
        uf[kb] = frag2_from_acc_scaled<T>(un[2 * kb], un[2 * kb + 1], slo[kb], shi[kb]);
#pragma unroll
      for (int tj = 0; tj < NKT; ++tj) S[tj] *= decC;
    }
#pragma unroll
    for (int tj = 0; tj < NKT; ++tj)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const Frag<T> kt = frag_col(Ks + 32 * kb * LD + 16 * tj + n, LD, g);
        if constexpr (kDelta) mma_ab2(kt, uf[kb], S[tj]);
        else mma(kt, uf[kb].hi, S[tj]);
      }
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

template <typename T, typename TO, int D, int MODE, int NW>
void launch_one(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t st) {
  const dim3 grid((unsigned)((size_t)a.B * a.H * (D / (16 * NW)))), block(64 * NW);
  const bool delta = MODE != kModeLinear;
  state_kernel<T, TO, D, MODE, NW><<<grid, block, 0, st>>>(
      static_cast<const T*>(a.q), static_cast<const T*>(a.k),
      static_cast<const T*>(ws.W), delta ? static_cast<const void*>(ws.U) : a.v,
      static_cast<const T*>(ws.Aqk), ws.G, a.S0, static_cast<TO*>(a.out), a.S_final, a.L);
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

template <typename T, typename TO, int D, int MODE>
void launch_mode(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t st) {
  switch (pick_nw(a)) {
    case 4: launch_one<T, TO, D, MODE, 4>(a, ws, st); break;
    case 2: launch_one<T, TO, D, MODE, 2>(a, ws, st); break;
    default: launch_one<T, TO, D, MODE, 1>(a, ws, st); break;
  }
}

template <typename T, typename TO, int D>
void launch_td(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t st) {
  switch (a.mode) {
    case kModeLinear: launch_mode<T, TO, D, kModeLinear>(a, ws, st); break;
    case kModeDelta: launch_mode<T, TO, D, kModeDelta>(a, ws, st); break;
    default: launch_mode<T, TO, D, kModeGatedDelta>(a, ws, st); break;
  }
}

template <typename T, typename TO>
void launch_types(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t st) {
  if (a.d == 64) launch_td<T, TO, 64>(a, ws, st);
  else launch_td<T, TO, 128>(a, ws, st);
}

}  // namespace

hipError_t launch_state(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t st) {
  if (a.in_bf16) {
    if (a.out_bf16) launch_types<__bf16, __bf16>(a, ws, st);
    else launch_types<__bf16, float>(a, ws, st);
  } else {
    launch_types<float, float>(a, ws, st);
  }
  return hipGetLastError();
}

}  // namespace la
