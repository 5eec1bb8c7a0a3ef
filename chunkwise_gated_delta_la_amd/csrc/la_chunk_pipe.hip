// Chunkwise forward for bf16 inputs in two kernels: the same computation as
// the float kernel in la_chunk.hip (see there for the formulas and their
// sources), split along what does and does not depend on the carried state.
//
// 1. t_solve_kernel, parallel over every (batch, head, chunk): the chunk's
//    A = strict_lower(diag(beta) K K^T * Gamma) and T = (I + A)^-1.  T does
//    not depend on the state, so all chunks are solved at once, at full
//    occupancy, and written to a workspace as the exact MFMA operand
//    fragments the second kernel feeds to U_new = T R (6 KiB per chunk).
//
// 2. chunk_pipe_kernel, one 512-thread workgroup per 16-column tile of one
//    (batch, head) state, walking the chunks in order with a single barrier
//    per chunk: two waves carry the serial chain (K S, R, U_new = T R and
//    the state update, each on half of the state's rows), four form the
//    output of their row tiles from what the chain published, and two move
//    the inputs and build the decay tables (the roles are listed at the
//    kernel).  The chain waves only ever wait for their own products, and
//    do as little besides them as possible: every LDS address they use is
//    one add of a loop-invariant lane offset to the ring slot, and the
//    float to bf16 splits take two instructions per value.  Inputs go from
//    HBM straight into LDS rings (global_load_lds_dwordx4: lane l's 16 bytes
//    land at base + 16 l) without passing through registers, issued ahead
//    of the chunk that reads them and waited for before the barrier that
//    opens it.
//
// State rows.  The rows of the state (the dk index) are kept in the
// registers in a fixed permuted order: register row p = 32 kb + 16 h +
// 4 g + j holds dk index 32 kb + 8 g + 4 h + j.  Any order works as long as
// every product over dk uses the same one; this one makes the operand
// fragment of a Q or K row over dk block kb for lane group g the 8
// contiguous columns 32 kb + 8 g .. + 7, one 16-byte read, while the
// accumulator tiles of S are still directly the B operand of K S and Q S.
// Only loading S0 and storing S_final see the permutation.
//
// Q and K tiles are stored row-major with the 16-byte units of row r
// permuted by XOR with key(r), a bit permutation of r's low bits chosen so
// that both the operand-row reads and the transposed reads below are free
// of bank conflicts.  K^T and V^T operands are read transposed from the
// row-major tiles with ds_read_b64_tr_b16 (within each 16-lane group, lane i
// receives element i % 4 of the 4-element runs addressed by lanes
// i / 4 + 4 j, j = 0..3), so no transposed copy is ever stored.  The scores
// are computed transposed (K Q^T tiles): the accumulator layout of K Q^T is
// exactly the A-operand layout of Aqk = Q K^T * M * Gamma for O += Aqk
// U_new, so the scores never leave registers.
//
// Precision as in the float kernel's bf16 path: q, k, v exact, float
// operands split into bf16 hi + lo, T a single bf16, float accumulation and
// state.
#include <type_traits>

#include "la_device.hpp"
#include "la_index.hpp"
#include "la_kernels.hpp"

namespace la {
namespace {

constexpr int C = 64;
constexpr int kThreads = 256;
constexpr int LDT = C + 8;        // row pitch of the bf16 T tile
constexpr int LDB = 20;           // row pitch of a float 16 x 16 block
typedef __bf16 T16;
typedef short s16x4 __attribute__((ext_vector_type(4)));
#define LA_LDS __attribute__((address_space(3)))

// ---------------------------------------------------------------- LDS access

// Loads at a byte offset from an LDS array.
template <typename V>
__device__ __forceinline__ V lds_ld(const void* base, uint32_t off) {
  return *(const LA_LDS V*)((const LA_LDS char*)base + off);
}

template <typename V>
__device__ __forceinline__ void lds_st(void* base, uint32_t off, const V& x) {
  *(LA_LDS V*)((LA_LDS char*)base + off) = x;
}

__device__ __forceinline__ bf16x4 read_tr(const void* base, uint32_t off) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (LA_LDS s16x4*)((const LA_LDS char*)base + off));
  return __builtin_bit_cast(bf16x4, r);
}

// The tile swizzle (swz_key, unit_off), the state-row order (dk_of_row)
// and the transposed-read offsets are in la_index.hpp, shared with the host
// checker of the index maps.

// Operand row R over dk block kb: the unit 4 kb + g (the key depends only on
// R's low four bits, so 16-row steps are a constant 32 D bytes).
template <int D>
__device__ __forceinline__ Frag<T16> frag_row_at(const void* tile, uint32_t off) {
  Frag<T16> f;
  f.v = lds_ld<bf16x8>(tile, off);
  return f;
}

// Transposed K operand over token rows r0 + kidx(g, j) for state tile
// tj = 2 kbs + h: lane (g, n) gets K[r0 + kidx(g, j)][dk_of_row(16 tj + n)],
// kidx(g, j) = 4 g + j for j < 4 and 16 + 4 g + j - 4 above (the order in
// which an accumulator pair gives its rows).  Lane k of group g addresses
// row r0 + 4 g + k / 4 (+ 16) at the four columns 32 kbs + 8 (k % 4) + 4 h
// .. + 3 (tr_off), so lane n receives element n % 4 of the runs of lanes
// n / 4 + 4 j: column 32 kbs + 8 (n / 4) + 4 h + n % 4.
__device__ __forceinline__ Frag<T16> frag_tr_at(const void* tile, uint32_t off, uint32_t half) {
  Frag<T16> f;
  const bf16x4 a = read_tr(tile, off);
  const bf16x4 b = read_tr(tile, off + half);
  f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}

// Column n of a plain C x 16 bf16 tile (this workgroup's V columns) as an
// operand over rows r0 .. r0 + 31.
__device__ __forceinline__ Frag<T16> frag_col_tr_v(const void* tile, int r0, int g, int n) {
  return frag_tr_at(tile, col_tr_off(r0, g, n), 16 * 16 * 2);
}

// V in accumulator layout for rows 16 ti + 4 g + i, column n: off is the
// lane's byte offset for ti = 0 (vacc_off), ti adds 512 bytes.
__device__ __forceinline__ f32x4 v_acc_at(const void* tile, uint32_t off) {
  const bf16x4 a = read_tr(tile, off);
  return f32x4{(float)a[0], (float)a[1], (float)a[2], (float)a[3]};
}

// A 16 x 16 float block (row pitch LDB) as a 16-deep split operand row:
// p[4 g + j] in slots j < 4, zero above.
__device__ __forceinline__ Frag2<T16> frag2_blk16(const float* p, int g) {
  Frag2<T16> f;
  const f32x4 a = *reinterpret_cast<const f32x4*>(p + 4 * g);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f.set(i, a[i]);
    f.set(4 + i, 0.f);
  }
  return f;
}

// Two side-by-side 16 x 16 float blocks as one 32-deep split operand row.
__device__ __forceinline__ Frag2<T16> frag2_blk32(const float* p0, const float* p1, int g) {
  Frag2<T16> f;
  const f32x4 a = *reinterpret_cast<const f32x4*>(p0 + 4 * g);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p1 + 4 * g);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f.set(i, a[i]);
    f.set(4 + i, b[i]);
  }
  return f;
}


// ---------------------------------------------------------------- DMA loads
//
// global_load_lds moves `size` bytes per lane from global memory straight
// into LDS at M0 + lane * size.  It is issued through inline assembly so
// that the compiler does not track it: the loading waves wait for it
// explicitly (s_waitcnt vmcnt) before the barrier that publishes the data.
// Otherwise the compiler, unable to tell the ring slots apart, would wait
// for the transfer before every later LDS read of the issuing wave.  Vector
// memory loads complete in issue order, so waiting until at most N are
// outstanding retires everything but the last N issued.

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const LA_LDS void*)p;
}

// Issued from a wave-uniform base address plus a 32-bit lane offset
// (scalar-base addressing: no per-lane 64-bit address arithmetic).
__device__ __forceinline__ void dma16s(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(base), "s"(lds) : "memory", "m0");
}

__device__ __forceinline__ void dma4s(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(off), "s"(base), "s"(lds) : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// DMA of one C x D tile into the swizzled layout by one wave; each
// instruction moves 1 KiB = 512 elements.  Instruction m of lane l stores
// LDS bytes 1024 m + 16 l: row r, position ul, i.e. logical unit
// ul ^ key(r); off[m] is that unit's byte offset in the source rows.
//
// Rows at or past nrows (the end of the sequence in a partial last chunk)
// read the last valid row instead, so no load leaves the tensor.
template <int D>
__device__ __forceinline__ void dma_tile_offsets(uint32_t (&off)[C * 2 * D / 1024], int lane,
                                                 int nrows) {
#pragma unroll
  for (int m = 0; m < C * 2 * D / 1024; ++m) off[m] = dma_src_off<D>(m, lane, nrows);
}

template <int D>
__device__ __forceinline__ void dma_tile(T16* dst, const T16* src_rows,
                                         const uint32_t (&off)[C * 2 * D / 1024]) {
  const uint32_t base = lds_addr(dst);
#pragma unroll
  for (int m = 0; m < C * 2 * D / 1024; ++m)
    dma16s(src_rows, off[m], __builtin_amdgcn_readfirstlane(base + 1024 * m));
}

// ---------------------------------------------------------------- T solve

// A T record holds the kTFrags fragments of bf16(T), fragment tfi(ti, kb)
// for row tile ti and 32-deep block kb <= ti / 2 (la_index.hpp): T enters
// U_new = T R as a single bf16 (its rounding costs well under the
// tolerance; R is split).

// Diagonal blocks D_i = (I + A_ii)^-1, each written over A_ii: lane (g, n)
// solves column n of block g by forward substitution.  The block's rows are
// loaded first, by the one wave of the workgroup, so every read of A_ii
// precedes every write of D_i, and nothing reads A_ii afterwards.
__device__ __forceinline__ int dblk(int i) { return bid(i, i) * 16 * LDB; }
__device__ __forceinline__ void t_diag(float* Ab, int g, int n) {
  const float* A = Ab + dblk(g);
  f32x4 arow[16][4];
#pragma unroll
  for (int r = 1; r < 16; ++r)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4)
      if (4 * i4 < r) arow[r][i4] = *reinterpret_cast<const f32x4*>(A + r * LDB + 4 * i4);
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
  for (int r = 0; r < 16; ++r) Ab[dblk(g) + r * LDB + n] = x[r];
}

// Blocks of T below the diagonal from the diagonal blocks D_i (in the
// diagonal A blocks' place) and the A blocks below the diagonal:
//   T10 = -D1 A10 D0,  T32 = -D3 A32 D2,
//   [T20 T21; T30 T31] = -[[D2, 0], [T32, D3]] [A20 A21; A30 A31] [[D0, 0], [T10, D1]]
// (block inverse of a 2 x 2 block lower-triangular matrix, applied twice),
// four dependent product steps.  Products split both operands.  The six
// blocks come back in accumulator layout: tb[0..5] = T10, T32, T20, T21,
// T30, T31 (element (4 g + e, n) of each).
__device__ __forceinline__ void t_col(const float* Ab, float* T32f, f32x4 (&tb)[6], int g,
                                      int n) {
  auto blkA = [&](int i, int j) { return Ab + bid(i, j) * 16 * LDB; };
  auto blkD = [&](int i) { return Ab + dblk(i); };
  auto dacc = [&](int i) {     // D_i in accumulator layout
    f32x4 d;
#pragma unroll
    for (int e = 0; e < 4; ++e) d[e] = blkD(i)[(4 * g + e) * LDB + n];
    return d;
  };
  const f32x4 D0 = dacc(0), D1 = dacc(1), D2 = dacc(2);
  // level 1
  f32x4 x10 = zero4(), x32 = zero4(), t10 = zero4(), t32 = zero4();
  mma_a2b2(frag2_blk16(blkA(1, 0) + n * LDB, g), frag2_from_acc<T16>(D0, zero4()), x10);
  mma_a2b2(frag2_blk16(blkA(3, 2) + n * LDB, g), frag2_from_acc<T16>(D2, zero4()), x32);
  mma_a2b2(frag2_blk16(blkD(1) + n * LDB, g), frag2_from_acc<T16>(x10, zero4()), t10);
  mma_a2b2(frag2_blk16(blkD(3) + n * LDB, g), frag2_from_acc<T16>(x32, zero4()), t32);
  t10 = -t10;
  t32 = -t32;
  // T32 rows are needed as an A operand: through LDS
#pragma unroll
  for (int e = 0; e < 4; ++e) T32f[(4 * g + e) * LDB + n] = t32[e];
  __syncthreads();
  // level 2: X = [A20 A21; A30 A31] [[D0, 0], [T10, D1]]
  f32x4 x00 = zero4(), x10b = zero4(), x01 = zero4(), x11 = zero4();
  {
    const Frag2<T16> b0 = frag2_from_acc<T16>(D0, t10);
    const Frag2<T16> b1 = frag2_from_acc<T16>(D1, zero4());
    mma_a2b2(frag2_blk32(blkA(2, 0) + n * LDB, blkA(2, 1) + n * LDB, g), b0, x00);
    mma_a2b2(frag2_blk32(blkA(3, 0) + n * LDB, blkA(3, 1) + n * LDB, g), b0, x10b);
    mma_a2b2(frag2_blk16(blkA(2, 1) + n * LDB, g), b1, x01);
    mma_a2b2(frag2_blk16(blkA(3, 1) + n * LDB, g), b1, x11);
  }
  // Y = -[[D2, 0], [T32, D3]] X
  f32x4 y00 = zero4(), y01 = zero4(), y10 = zero4(), y11 = zero4();
  {
    const Frag2<T16> d2 = frag2_blk16(blkD(2) + n * LDB, g);
    mma_a2b2(d2, frag2_from_acc<T16>(x00, zero4()), y00);
    mma_a2b2(d2, frag2_from_acc<T16>(x01, zero4()), y01);
    const Frag2<T16> td = frag2_blk32(T32f + n * LDB, blkD(3) + n * LDB, g);
    mma_a2b2(td, frag2_from_acc<T16>(x00, x10b), y10);
    mma_a2b2(td, frag2_from_acc<T16>(x01, x11), y11);
  }
  tb[0] = t10;
  tb[1] = t32;
  tb[2] = -y00;
  tb[3] = -y01;
  tb[4] = -y10;
  tb[5] = -y11;
}

// Gate activations of the fused prologue, from their definitions: the
// logistic function, and softplus(x) = log(1 + e^x) written as max(x, 0) +
// log(1 + e^-|x|) so that no exponential overflows.
__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + __expf(-x)); }
__device__ __forceinline__ float softplus_f(float x) {
  return fmaxf(x, 0.f) + log1pf(__expf(-fabsf(x)));
}

// What the fused prologue reads and writes besides k and the gates.
struct ProIn {
  const T16* q;      // queries (their norms)
  ProArrays out;     // per-token gates and log inverse norms
  int flags;         // kProGates | kProQKNorm
  float gate_scale;
  bool erase, decay; // the call's mode reads beta / log alpha
};

// Sum over each 16-lane group's four copies (lane groups g = 0..3 hold the
// same rows): the row sums of squares of a chunk's fragments, then the one
// for the lane's own row 16 g + n (selected without indexing a register
// array by a lane-dependent value).
template <int NKB>
__device__ __forceinline__ float row_sumsq(const Frag<T16> (&f)[4][NKB], int g) {
  float ss[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    float a = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = (float)f[t][kb].v[j];
        a = fmaf(x, x, a);
      }
    a += __shfl_xor(a, 16);
    a += __shfl_xor(a, 32);
    ss[t] = a;
  }
  return g == 0 ? ss[0] : g == 1 ? ss[1] : g == 2 ? ss[2] : ss[3];
}

// One wave per T-factor slot (blocks numbered chunk-fastest within a head):
// T of the slot's chunk into tws[slot][f][lane], f = tfi(ti, kb), the
// operand fragment T[16 ti + n][32 kb + kidx(g, j)] of lane (g, n).  In the
// fixed-length layout slot = (batch * H + head) * ceil(L / C) + chunk; in a
// packed batch the slot of chunk j of sequence s is floor(cu[s] / C) + s + j
// within its head (see SeqMap), found here by a binary search over s, and
// slots no chunk maps to exit at once.
//
// PRO: the fused prologue of the chunk's tokens first -- the gates the op
// uses (raw scores through sigmoid / -gate_scale softplus when asked) and
// log(1 / |q_t|), log(1 / |k_t|) (q and k normalised as x / sqrt(|x|^2 +
// eps)), written per token for the chain kernels.  Normalised keys enter A
// as diag(r) K K^T diag(r): the logs of r are folded into the decay
// exponents (row g_r + log r_r, column g_i - log r_i).  TS = false: the
// prologue alone (modes without erase have no T).
template <int D, bool GATED, bool PRO, bool TS>
__global__ __launch_bounds__(kWave) void t_solve_kernel(const T16* __restrict__ k,
                                                        const float* __restrict__ log_alpha,
                                                        const float* __restrict__ beta,
                                                        u32x4* __restrict__ tws, SeqMap sm,
                                                        ProIn pro) {
  constexpr int NKB = D / 32;
  __shared__ __attribute__((aligned(16))) float Ab[TS ? 10 * 16 * LDB : 1];
  __shared__ __attribute__((aligned(16))) float T32f[TS ? 16 * LDB : 1];
  // The diagonal inverses take the diagonal A blocks' place, and the bf16 T
  // tile that the record is gathered from the A blocks' place once they have
  // been read for the last time: half the LDS of separate arrays (14.25
  // KiB), so eleven of these one-wave workgroups share a compute unit
  // instead of five.
  static_assert(!TS || C * LDT * sizeof(T16) <= sizeof(Ab), "T tile fits in the A blocks");
  T16* const Tb = reinterpret_cast<T16*>(Ab);
  __shared__ __attribute__((aligned(16))) float gsh[C];               // row exponents
  __shared__ __attribute__((aligned(16))) float gcsh[PRO ? C : 1];    // column exponents
  __shared__ __attribute__((aligned(16))) float bsh[C];

  const int lane = threadIdx.x;
  const int g = lane / 16, n = lane % 16;
  const size_t item = blockIdx.x;
  size_t row0;
  int nv;   // rows of this chunk inside its sequence
  if (!sm.cu) {
    const int NC = (sm.L + C - 1) / C;
    const size_t bh = item / NC;
    const int c = (int)(item % NC);
    row0 = bh * sm.L + (size_t)c * C;
    nv = min(C, sm.L - c * C);
  } else {
    const size_t sph = sm.slots_per_head();
    const int h = (int)(item / sph), j = (int)(item % sph);
    auto start = [&](int s) { return min(max(sm.cu[s], 0), sm.L); };
    auto first_slot = [&](int s) { return start(s) / C + s; };
    if (first_slot(0) > j) return;
    int lo = 0, hi = sm.N - 1;      // largest s with first_slot(s) <= j
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if (first_slot(mid) <= j) lo = mid;
      else hi = mid - 1;
    }
    const int a = start(lo), len = min(max(sm.cu[lo + 1], a), sm.L) - a;
    const int c = j - first_slot(lo);
    if (c * C >= len) return;       // no chunk in this slot
    row0 = (size_t)h * sm.L + a + (size_t)c * C;
    nv = min(C, len - c * C);
  }
  // rows past the sequence's end (a partial last chunk) read the last valid
  // row and carry beta = 0, log alpha = 0, which makes their rows of A zero
  // and of T the identity

  // K rows as operands of K K^T.  Both operands are rows of K, so any
  // assignment of the contraction index to (group, slot) works; here slot j
  // of group g is column 32 kb + 8 g + j, one 16-byte load per fragment.
  Frag<T16> kf[4][NKB];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      kf[t][kb].v = *reinterpret_cast<const bf16x8*>(
          k + (row0 + min(16 * t + n, nv - 1)) * D + 32 * kb + 8 * g);
  const int lr = min(lane, nv - 1);
  float bv = 0.f, av = 0.f, lkv = 0.f;
  if constexpr (PRO) {
    const bool act = pro.flags & kProGates;
    if (pro.erase && lane < nv) {
      const float b = beta[row0 + lr];
      bv = act ? sigmoid_f(b) : b;
    }
    if (pro.decay && lane < nv) {
      const float a = log_alpha[row0 + lr];
      av = act ? -pro.gate_scale * softplus_f(a) : a;
    }
    float lqv = 0.f;
    if (pro.flags & kProQKNorm) {
      Frag<T16> qf[4][NKB];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          qf[t][kb].v = *reinterpret_cast<const bf16x8*>(
              pro.q + (row0 + min(16 * t + n, nv - 1)) * D + 32 * kb + 8 * g);
      lkv = -0.5f * __logf(row_sumsq<NKB>(kf, g) + kQKNormEps);
      lqv = -0.5f * __logf(row_sumsq<NKB>(qf, g) + kQKNormEps);
    }
    if (lane < nv) {
      pro.out.beta[row0 + lane] = bv;
      pro.out.log_alpha[row0 + lane] = av;
      pro.out.lq[row0 + lane] = lqv;
      pro.out.lk[row0 + lane] = lkv;
    }
  } else {
    bv = lane < nv ? beta[row0 + lr] : 0.f;
    if constexpr (GATED) av = lane < nv ? log_alpha[row0 + lr] : 0.f;
  }
  if constexpr (TS) {
    float gv = 0.f;
    if constexpr (GATED) gv = wave_inclusive_scan(av);
    gsh[lane] = gv + lkv;
    if constexpr (PRO) gcsh[lane] = gv - lkv;
    bsh[lane] = bv;
    // A blocks (R, t), t <= R: element (4 g + e, n) is row 16 R + 4 g + e,
    // column 16 t + n
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      const f32x4 br = *reinterpret_cast<const f32x4*>(bsh + 16 * R + 4 * g);
      const f32x4 gr = *reinterpret_cast<const f32x4*>(gsh + 16 * R + 4 * g);
#pragma unroll
      for (int t = 0; t <= R; ++t) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) mma(kf[R][kb], kf[t][kb], acc);
        const float gc = (PRO ? gcsh : gsh)[16 * t + n];
        float* blk = Ab + bid(R, t) * 16 * LDB;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool keep = R > t || 4 * g + e > n;
          float decay = 1.f;
          if constexpr (GATED) decay = __expf(keep ? gr[e] - gc : 0.f);
          blk[(4 * g + e) * LDB + n] = keep ? br[e] * acc[e] * decay : 0.f;
        }
      }
    }
    __syncthreads();
    t_diag(Ab, g, n);
    __syncthreads();
    f32x4 tb[6];
    t_col(Ab, T32f, tb, g, n);
    __syncthreads();     // (the A blocks are read for the last time)
    // T into its bf16 tile over the A blocks: the diagonal blocks from the
    // inverses (lane (g, n): column n of block g; the tile covers three of
    // them, so all are read before the first write), the six blocks below
    // from t_col, and zeros for the upper blocks (0, 1) and (2, 3) that T's
    // operand fragments span
    float dcol[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) dcol[r] = Ab[dblk(g) + r * LDB + n];
#pragma unroll
    for (int r = 0; r < 16; ++r) Tb[(16 * g + r) * LDT + 16 * g + n] = (T16)dcol[r];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * g + e;
      Tb[(16 + r) * LDT + n] = (T16)tb[0][e];
      Tb[(48 + r) * LDT + 32 + n] = (T16)tb[1][e];
      Tb[(32 + r) * LDT + n] = (T16)tb[2][e];
      Tb[(32 + r) * LDT + 16 + n] = (T16)tb[3][e];
      Tb[(48 + r) * LDT + n] = (T16)tb[4][e];
      Tb[(48 + r) * LDT + 16 + n] = (T16)tb[5][e];
      Tb[r * LDT + 16 + n] = (T16)0.f;
      Tb[(32 + r) * LDT + 48 + n] = (T16)0.f;
    }
    __syncthreads();
    u32x4* dst = tws + item * (kTRecFrags * kWave);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int kb = 0; kb <= ti / 2; ++kb) {
        const Frag<T16> f = frag_row(Tb + (16 * ti + n) * LDT + 32 * kb, g);
        dst[tfi(ti, kb) * kWave + lane] = __builtin_bit_cast(u32x4, f.v);
      }
  }
}


// ---------------------------------------------------------------- output roles

// Q rows of row tile TI of a chunk straight from HBM as operand fragments:
// lane (g, n) holds row 16 TI + n, columns 32 kb + 8 g .. + 7 of each dk
// block (one 16-byte load per block) -- the same contraction order as the
// K rows in LDS and the permuted state rows.  Rows at or past nrows (the
// end of the sequence in a partial last chunk) read the last valid row.
template <int D, int TI>
__device__ __forceinline__ void load_q(Frag<T16> (&qf)[D / 32], const T16* q, size_t r0,
                                       int nrows, int g, int n) {
  const T16* row = q + (r0 + (size_t)min(16 * TI + n, nrows - 1)) * D + 8 * g;
#pragma unroll
  for (int kb = 0; kb < D / 32; ++kb) qf[kb].v = *reinterpret_cast<const bf16x8*>(row + 32 * kb);
}

// Scores and Q S of one chunk for row tile TI, kept in registers.  sc[t] is
// the K Q^T tile (t, TI): lane (g, n) holds Aqk[16 TI + n][16 t + 4 g + e]
// (decayed, masked).  The output is formed transposed, O^T = S^T Q^T +
// U_new^T Aqk^T: the same operand fragments with A and B swapped (an A and a
// B fragment have the same lane layout), so that lane (g, n) holds token
// 16 TI + n at the four adjacent columns 4 g + e and writes them with one
// store.  qs holds gam[16 TI + n] (Q S)[16 TI + n][4 g + e].  roff[kb] is
// the lane's byte offset of operand row n over dk block kb in a K tile.  The
// decay of score (r, i) is exp(gsc[r] - gkc[i]) and Q S row r is scaled by
// esc[r]: the exponents g and the factors exp(g), or with normalised q and k
// the same with the logs of the inverse norms folded in.  Below the diagonal
// tile (column tile t < TI) the decay is the product of a row factor ra[r] =
// exp(gsc[r] - g[16 TI]) and a column factor cb[i] = exp(g[16 TI] - gkc[i])
// (g does not increase along the chunk, so neither factor exceeds the
// inverse norm it carries): two products instead of an exponential.
template <int D, bool GATED, int TI>
__device__ __forceinline__ void scores_qs(const Frag<T16> (&qf)[D / 32], const T16* Kt,
                                          const float* gsc, const float* gkc, const float* esc,
                                          const float* ra, const float* cb,
                                          const Frag<T16>* Sx, const uint32_t (&roff)[D / 32],
                                          f32x4 (&sc)[4], f32x4& qs, int g, int n, int lane) {
  constexpr int NKB = D / 32;
  constexpr uint32_t kRows16 = 32 * D;          // bytes of 16 tile rows
  Frag<T16> kf[TI + 1][NKB];
  Frag2<T16> sx[NKB];
#pragma unroll
  for (int t = 0; t <= TI; ++t)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) kf[t][kb] = frag_row_at<D>(Kt, roff[kb] + kRows16 * t);
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    sx[kb].hi = Sx[(2 * kb) * kWave + lane];
    sx[kb].lo = Sx[(2 * kb + 1) * kWave + lane];
  }
  float gq = 0.f, eq = 1.f, rq = 1.f;
  f32x4 gk = zero4(), cf[TI + 1];
  if constexpr (GATED) {
    gq = gsc[16 * TI + n];
    eq = esc[16 * TI + n];
    gk = *reinterpret_cast<const f32x4*>(gkc + 16 * TI + 4 * g);
    if constexpr (TI > 0) {
      rq = ra[16 * TI + n];
#pragma unroll
      for (int t = 0; t < TI; ++t)
        cf[t] = *reinterpret_cast<const f32x4*>(cb + (TI - 1) * C + 16 * t + 4 * g);
    }
  }
  qs = zero4();
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    mma(sx[kb].lo, qf[kb], qs);
    mma(sx[kb].hi, qf[kb], qs);
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    sc[t] = zero4();
    if (t > TI) continue;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) mma(kf[t][kb], qf[kb], sc[t]);
    // element (K row 16 t + 4 g + e, Q row 16 TI + n) = Aqk[r][i]
    if (t < TI) {
      if constexpr (GATED) sc[t] = (sc[t] * rq) * cf[t];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool keep = 4 * g + e <= n;
        float decay = 1.f;
        if constexpr (GATED) decay = __expf(keep ? gq - gk[e] : 0.f);
        sc[t][e] = keep ? sc[t][e] * decay : 0.f;
      }
    }
  }
  if constexpr (GATED) qs *= eq;
}

// Output of row tile TI, transposed: O^T = qs + U_new^T Aqk^T (U_new = V in
// the modes without erase).  U_new arrives in float (Uf, accumulator tile ti
// at ti * 64 + lane) and is split here.
// DSKIP: plus the residual D * V at the lane's token and four columns
// (dcol4, and four adjacent values of the value tile's row).
template <int D, int MODE, bool DSKIP, int TI>
__device__ __forceinline__ void out_rows(const f32x4 (&sc)[4], const f32x4& qs,
                                         const f32x4* Uf, const T16* Vt, f32x4& o, int g,
                                         int n, int lane, const f32x4& dcol4) {
  constexpr bool kDelta = mode_erase(MODE);
  o = qs;
#pragma unroll
  for (int kb = 0; kb <= TI / 2; ++kb) {
    const Frag2<T16> a = frag2_from_acc<T16>(sc[2 * kb], sc[2 * kb + 1]);
    if constexpr (kDelta) {
      const Frag2<T16> u =
          frag2_from_acc<T16>(Uf[(2 * kb) * kWave + lane], Uf[(2 * kb + 1) * kWave + lane]);
      mma_a2b2(u, a, o);
    } else {
      const Frag<T16> u = frag_col_tr_v(Vt, 32 * kb, g, n);
      mma(u, a.lo, o);
      mma(u, a.hi, o);
    }
  }
  if constexpr (DSKIP) {
    const bf16x4 vr = lds_ld<bf16x4>(Vt, (uint32_t)(((16 * TI + n) * 16 + 4 * g) * 2));
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] += dcol4[e] * (float)vr[e];
  }
}

// Store of row tile TI: token 16 TI + n, columns 4 g .. 4 g + 3 of the tile
// (one 8-byte bf16 or 16-byte float store per lane); tokens at or past nrows
// (past the end of the sequence in a partial last chunk) are not written.
template <int D, int TI>
__device__ __forceinline__ void store_rows(const f32x4& o, void* out_, size_t ob0, int out_bf16,
                                           int g, int n, int nrows) {
  if (16 * TI + n >= nrows) return;
  const size_t ob = ob0 + (size_t)(16 * TI + n) * D + 4 * g;
  if (out_bf16) {
    const bf16x4 h = __builtin_convertvector(o, bf16x4);
    *reinterpret_cast<bf16x4*>(static_cast<T16*>(out_) + ob) = h;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out_) + ob) = o;
  }
}

// In-chunk cumulative log-decay of the 64 values at p, one per lane.
__device__ __forceinline__ float cumsum64(const float* p, int lane) {
  return wave_inclusive_scan(p[lane]);
}


// ---------------------------------------------------------------- chain kernel

// One workgroup per (stream, 16-column tile of the state); the dv columns of
// S evolve independently, so a stream's state is split into D / 16 tiles
// that walk the chunks in parallel.  Waves and their roles:
//
//   waves 0, 1   the serial chain, each on half of the state's rows (dk):
//                the whole K S (the other half's bf16 state read from the
//                split both publish for the output waves), R = diag(beta)(V -
//                diag(gam) K S) and U_new = T R (each publishes two of its
//                four row tiles for the output waves), then the update of
//                its half, S <- gam_C S + K^T diag(gam_C / gam) U_new, and
//                its half's split published.  The two never wait for each
//                other inside a chunk.  Without erase: S <- gam_C S + K^T
//                diag(f) V.
//   DMA K        K of chunk c+2 and the gates of chunk c+4 into LDS rings;
//                beta V (or f V) of chunk c+1 in the chain's accumulator
//                layout
//   DMA V        Q of chunk c+1 (where Q is staged in LDS), V of chunk
//                c+3 and the T record of chunk c+2; the decay tables of
//                chunk c+2; the zero rows of a partial V
//   output (4)   one row tile each: the output of chunk c-1 from the U_new
//                published at the last barrier (formed transposed: one
//                store per lane of four adjacent columns), then the masked
//                decayed scores and diag(gam) Q S of chunk c kept in
//                registers (Q from the LDS ring, or straight from HBM one
//                chunk ahead where staging it would halve the occupancy)
//
// OUT: 8 waves (chain 0, 1; output tiles 3, 2 on waves 2, 3 and 0, 1 on
// waves 6, 7; DMA K wave 4, DMA V wave 5).  The state pass (OUT = false)
// has no output waves: 4 waves (chain 0, 1; DMA K 2; DMA V 3).  Waves go to
// the four SIMDs round robin, so the two chain halves run on their own
// SIMDs, each beside a DMA wave, and the output waves pair the row tiles of
// most and least work on the other two.  One barrier per chunk.
//
// OUT = false is the state pass of the sequence-parallel forward: the chain
// alone, with no Q and no outputs.  FUSED: q and k are normalised inside the
// op -- with r_t = 1 / |x_t| per token, every product of the method sees
// diag(r) K and diag(r) Q only through per-row factors that the decay tables
// already apply, so the inverse norms (their logs lq, lk, from the prologue)
// are folded into the tables and no product changes:
//   scores  exp((g_r + lq_r) - (g_i - lk_i)),  Q S rows  exp(g + lq),
//   update  exp(g_C - g + lk),  erase  beta exp(g + lk)
// (MODE is then one of the decayed modes; log alpha = 0 stands for none).
// DSKIP: the output gains the residual D * v (Mamba's term in v), D [H, dv].
template <int D, int MODE, bool OUT, bool FUSED, bool DSKIP>
__global__ __launch_bounds__(OUT ? 512 : 256) void chunk_pipe_kernel(
    const T16* __restrict__ q, const T16* __restrict__ k, const T16* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    const u32x4* __restrict__ tws, void* __restrict__ out_, StreamMap smap, int NS,
    int out_bf16, ProArrays pro, const float* __restrict__ dskip) {
  constexpr bool kDelta = mode_erase(MODE);      // delta rule: beta, T, U_new
  constexpr bool kGated = mode_decay(MODE);      // scalar decay: log alpha
  static_assert(!FUSED || kGated, "normalised q, k ride in the decay tables");
  static_assert(!DSKIP || OUT, "the residual is part of the output");
  constexpr int NKT = D / 16;                    // 16-row tiles of the state
  constexpr int NKB = D / 32;                    // 32-deep blocks over dk
  constexpr int HT = NKT / 2, HB = NKB / 2;      // of one chain half
  constexpr int NCT = D / 16;                    // column tiles per head
  constexpr int TILE = C * D;                    // elements of a K tile
  constexpr uint32_t kTileB = 2 * TILE;          // bytes of a K tile
  constexpr uint32_t kRows16 = 32 * D;           // bytes of 16 tile rows
  constexpr int NTILE = TILE * 2 / 1024;         // DMA instructions per tile
  constexpr int NG = 5;                          // gate rings (DMA 4 ahead)
  // The state pass keeps its LDS within 80 KiB, so that two of its
  // workgroups share a compute unit: K one chunk ahead (two slots), V three
  // ahead (four slots), and only the high part of the published state split
  // (no output waves read the low part).
  constexpr int KR = OUT ? 3 : 2;                // K ring (DMA KR - 1 ahead)
  constexpr int NV = OUT ? 5 : 4;                // value ring (DMA 3 ahead)
  constexpr int SXP = OUT ? 2 : 1;               // parts of the state split in Sx
  constexpr int kDmaK = OUT ? 4 : 2, kDmaV = OUT ? 5 : 3;
  constexpr bool kQSide = FUSED && OUT;          // (the state pass has no Q side: only lk)
  constexpr int NGATE = (kDelta ? 1 : 0) + (kGated ? 1 : 0) + (FUSED ? 1 : 0) + (kQSide ? 1 : 0);
  constexpr int NDMAK = NTILE + NGATE;           // per chunk of the DMA K wave
  constexpr int NDMAV = 2 + (kDelta ? kTRecFrags : 0);   // per chunk of the DMA V wave
  constexpr bool kBV = kDelta || MODE == kModeGatedLinear;  // beta V or f V for the chain

  __shared__ __attribute__((aligned(16))) T16 Ks[KR][TILE];
  __shared__ __attribute__((aligned(16))) T16 Vs[NV][C * 16];
  __shared__ __attribute__((aligned(16))) u32x4 Ts[kDelta ? 3 : 1][kDelta ? kTRecFrags * kWave : 1];
  __shared__ __attribute__((aligned(16))) float Ls[kGated ? NG : 1][C];  // log alpha
  __shared__ __attribute__((aligned(16))) float Bs[kDelta ? NG : 1][C];  // beta
  __shared__ __attribute__((aligned(16))) float Gs[kGated && OUT ? 3 : 1][C];   // g (in-chunk cumsum)
  __shared__ __attribute__((aligned(16))) float Es[kGated ? 3 : 1][C];   // exp(g)
  __shared__ __attribute__((aligned(16))) float Fs[kGated ? 3 : 1][C];   // exp(g_C - g)
  __shared__ __attribute__((aligned(16))) float BGs[kGated ? 3 : 1][C];  // beta exp(g)
  __shared__ __attribute__((aligned(16))) float LQs[kQSide ? NG : 1][C];  // log(1 / |q|)
  __shared__ __attribute__((aligned(16))) float LKs[FUSED ? NG : 1][C];   // log(1 / |k|)
  __shared__ __attribute__((aligned(16))) float Gk[kQSide ? 3 : 1][C];    // g - lk (score columns)
  __shared__ __attribute__((aligned(16))) float Eq[kQSide ? 3 : 1][C];    // exp(g + lq) (Q S rows)
  constexpr bool kFac = kGated && OUT;           // factored score decays below the diagonal
  __shared__ __attribute__((aligned(16))) float Ra[kFac ? 3 : 1][C];      // exp(gsc[r] - g[16 (r / 16)])
  __shared__ __attribute__((aligned(16))) float Cb[kFac ? 3 : 1][kFac ? 3 * C : 1];  // exp(g[16 t] - gkc[i]), t = 1..3
  __shared__ __attribute__((aligned(16))) Frag<T16> Sx[2][SXP * NKB * kWave];
  __shared__ __attribute__((aligned(16))) f32x4 Uf[kDelta && OUT ? 2 : 1][kDelta && OUT ? 4 * kWave : 1];
  __shared__ __attribute__((aligned(16))) f32x4 BVs[kBV ? 2 : 1][kBV ? 4 * kWave : 1];
  // Q: where the rest already holds more than half of the compute unit's
  // LDS (one workgroup per unit either way) or Q still fits under that
  // half, the DMA V wave stages Q in a ring of two tiles, one chunk ahead,
  // and the output waves read their rows from it; otherwise each output wave
  // loads its rows from HBM straight into registers, one chunk ahead.
  constexpr size_t kLdsRest =
      sizeof(Ks) + sizeof(Vs) + sizeof(Ts) + sizeof(Ls) + sizeof(Bs) + sizeof(Gs) + sizeof(Es) +
      sizeof(Fs) + sizeof(BGs) + sizeof(LQs) + sizeof(LKs) + sizeof(Gk) + sizeof(Eq) + sizeof(Ra) +
      sizeof(Cb) + sizeof(Sx) + sizeof(Uf) + sizeof(BVs);
  constexpr size_t kHalfLds = 80 * 1024;
  constexpr bool kQLds = OUT && (kLdsRest > kHalfLds || kLdsRest + 4 * TILE <= kHalfLds);
  __shared__ __attribute__((aligned(16))) T16 Qs[kQLds ? 2 : 1][kQLds ? TILE : 1];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int g = lane / 16;
  const int n = lane % 16;

  // stream (sequence or segment) and column tile; the column tiles of one
  // stream share an XCD (blocks go to XCDs round robin), so its K, Q and T
  // reads are shared in that XCD's L2
  int sidx, ct;
  {
    const int b = blockIdx.x;
    if (NS % 8 == 0) {
      const int x = b % 8, s = b / 8;
      ct = s % NCT;
      sidx = (s / NCT) * 8 + x;
    } else {
      sidx = b / NCT;
      ct = b % NCT;
    }
  }
  const int col0 = ct * 16;
  const int col = col0 + n;
  const StreamInfo si = stream_info(smap, sidx);
  const size_t hbase = si.row0;                 // first token row
  const int L = si.len;                         // tokens of this stream
  if (L == 0) {
    // empty sequence: the state passes through
    if (wave == 0 && si.sf) {
#pragma unroll
      for (int r = 0; r < D / 4; ++r) {
        const size_t e = (size_t)(4 * r + g) * D + col;
        si.sf[e] = si.s0 ? si.s0[e] : 0.f;
      }
    }
    return;
  }
  // Chunks; the last holds nlast rows (C unless L is not a multiple of C).
  // Rows past the sequence act as tokens that change nothing: beta = 0 and
  // log alpha = 0 (no erase, no write, no decay -- their rows of T are the
  // identity rows), V = 0 (no write in the modes without beta); their Q, K
  // and V reads are clamped to the last valid row and their outputs are not
  // stored.  Valid rows never see them: every product inside a chunk is
  // causal.
  const int NC = (L + C - 1) / C;
  const int nlast = L - (NC - 1) * C;
  const u32x4* tw = tws + si.slot0 * (kTRecFrags * kWave);
  const bool vzero = si.eye;          // a transition stream reads no V: its ring holds zeros

  // lane offsets of operand row n over each dk block in a K tile
  uint32_t roff[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) roff[kb] = unit_off<D>(n, 4 * kb + g);

  // Ring slot offsets go through readfirstlane: opaque to the loop
  // optimiser, which would otherwise turn each lane address into an
  // induction variable of its own plus a wrap correction (two adds per
  // address and a register each) instead of one add to a scalar.
  auto slot = [](int c, int depth, uint32_t bytes) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(c % depth) * bytes));
  };

  // DMA of K of chunk cc (the DMA K wave); rows past the sequence read the
  // last valid row
  auto issue_k = [&](int cc) {
    const size_t r0 = hbase + (size_t)cc * C;
    uint32_t po[NTILE];
    dma_tile_offsets<D>(po, lane, cc == NC - 1 ? nlast : C);
    dma_tile<D>(Ks[cc % KR], k + r0 * D, po);
  };
  // DMA of this tile's V columns (rows 32 m + l / 2, columns col0 + 8 (l % 2)
  // ..) and of the T record of chunk cc (the DMA V wave)
  auto issue_v = [&](int cc) {
    const size_t r0 = hbase + (size_t)cc * C;
    const int nr = cc == NC - 1 ? nlast : C;
    const uint32_t vb = lds_addr(Vs[cc % NV]);
#pragma unroll
    for (int m = 0; m < 2; ++m)
      dma16s(v + r0 * D + col0, (uint32_t)((min(32 * m + lane / 2, nr - 1) * D + 8 * (lane % 2)) * 2),
             __builtin_amdgcn_readfirstlane(vb + 1024 * m));
  };
  // DMA of Q of chunk cc (the DMA V wave), rows as for K
  auto issue_q = [&](int cc) {
    if constexpr (kQLds) {
      const size_t r0 = hbase + (size_t)cc * C;
      uint32_t po[NTILE];
      dma_tile_offsets<D>(po, lane, cc == NC - 1 ? nlast : C);
      dma_tile<D>(Qs[cc % 2], q + r0 * D, po);
    }
  };
  auto issue_t = [&](int cc) {
    const uint32_t tb = lds_addr(Ts[cc % 3]);
    const u32x4* src = tw + (size_t)cc * (kTRecFrags * kWave);
#pragma unroll
    for (int f = 0; f < kTRecFrags; ++f)
      dma16s(src, (uint32_t)((f * kWave + lane) * 16), __builtin_amdgcn_readfirstlane(tb + 1024 * f));
  };
  // DMA of the gates of chunk cc (the DMA K wave); lanes past the sequence
  // read the last valid token's gates (tables() zeroes them)
  auto issue_gates = [&](int cc) {
    const size_t r0 = hbase + (size_t)cc * C;
    const uint32_t go = (uint32_t)(cc == NC - 1 ? min(lane, nlast - 1) : lane) * 4;
    if constexpr (kDelta) dma4s(beta + r0, go, lds_addr(Bs[cc % NG]));
    if constexpr (kGated) dma4s(log_alpha + r0, go, lds_addr(Ls[cc % NG]));
    if constexpr (FUSED) dma4s(pro.lk + r0, go, lds_addr(LKs[cc % NG]));
    if constexpr (kQSide) dma4s(pro.lq + r0, go, lds_addr(LQs[cc % NG]));
  };
  // Gates of rows past the sequence set to zero, then the decay tables of
  // chunk cc from its gates (the DMA V wave, after the gates have landed)
  auto tables = [&](int cc) {
    if (cc == NC - 1 && lane >= nlast) {
      if constexpr (kDelta) Bs[cc % NG][lane] = 0.f;
      if constexpr (kGated) Ls[cc % NG][lane] = 0.f;
    }
    // the score decay's factors below the diagonal tile: row factor against
    // g at the start of the row's tile, column factors against g at the start
    // of each later tile (the unused ones, i >= 16 t, clamped: never read)
    auto factors = [&](float gv, float gsc, float gkc) {
      if constexpr (kFac) {
        const float g16 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), 16));
        const float g32 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), 32));
        const float g48 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), 48));
        const float g00 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), 0));
        const int tr = lane / 16;
        const float gt = tr == 0 ? g00 : tr == 1 ? g16 : tr == 2 ? g32 : g48;
        Ra[cc % 3][lane] = __expf(gsc - gt);
        Cb[cc % 3][0 * C + lane] = __expf(fminf(g16 - gkc, 80.f));
        Cb[cc % 3][1 * C + lane] = __expf(fminf(g32 - gkc, 80.f));
        Cb[cc % 3][2 * C + lane] = __expf(fminf(g48 - gkc, 80.f));
      }
    };
    if constexpr (FUSED) {
      const float gv = cumsum64(Ls[cc % NG], lane);
      const float gC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), kWave - 1));
      const float lk = LKs[cc % NG][lane];
      if constexpr (OUT) {
        const float lq = LQs[cc % NG][lane];
        Gs[cc % 3][lane] = gv + lq;
        Gk[cc % 3][lane] = gv - lk;
        Eq[cc % 3][lane] = __expf(gv + lq);
        factors(gv, gv + lq, gv - lk);
      }
      Es[cc % 3][lane] = __expf(gv);
      Fs[cc % 3][lane] = __expf(gC - gv + lk);
      if constexpr (kDelta) BGs[cc % 3][lane] = Bs[cc % NG][lane] * __expf(gv + lk);
    } else if constexpr (kGated) {
      const float gv = cumsum64(Ls[cc % NG], lane);
      const float gC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), kWave - 1));
      const float e = __expf(gv);
      if constexpr (OUT) Gs[cc % 3][lane] = gv;
      Es[cc % 3][lane] = e;
      Fs[cc % 3][lane] = __expf(gC - gv);
      if constexpr (kDelta) BGs[cc % 3][lane] = Bs[cc % NG][lane] * e;
      factors(gv, gv, gv);
    }
  };
  // beta V (erase) or f V (gated linear) of chunk cc in the chain's
  // accumulator layout (rows 16 ti + 4 g + e, column n), float
  auto make_bv = [&](int cc) {
    if constexpr (kBV) {
      const T16* Vt = Vs[cc % NV];
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        const f32x4 vv = v_acc_at(Vt, vacc_off(g, n) + 512 * ti);
        f32x4 s;
        if constexpr (kDelta) s = *reinterpret_cast<const f32x4*>(&Bs[cc % NG][16 * ti + 4 * g]);
        else s = *reinterpret_cast<const f32x4*>(&Fs[cc % 3][16 * ti + 4 * g]);
        BVs[cc % 2][ti * kWave + lane] = vv * s;
      }
    }
  };
  // V rows past the sequence set to zero once the last chunk's V has landed
  auto zero_v_tail = [&]() {
    if (nlast < C && lane >= nlast) {
      u32x4* row = reinterpret_cast<u32x4*>(Vs[(NC - 1) % NV] + lane * 16);
      row[0] = u32x4{0u, 0u, 0u, 0u};
      row[1] = u32x4{0u, 0u, 0u, 0u};
    }
  };

  // Each role runs its own loop with the same barriers (two in the
  // prologue, one per chunk), so the registers one role carries from chunk
  // to chunk are not live in the other's code.
  if (wave < 2) {
    // ================= chain: half h of the state's rows
    const int h = wave;
    f32x4 S[HT];
    Frag2<T16> sf[HB];            // bf16 split of this half of S, as published in Sx
    if (si.eye) {
#pragma unroll
      for (int j = 0; j < HT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          S[j][i] = dk_of_row(16 * (h * HT + j) + 4 * g + i) == col ? 1.f : 0.f;
    } else if (si.s0) {
#pragma unroll
      for (int j = 0; j < HT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          S[j][i] = si.s0[(size_t)dk_of_row(16 * (h * HT + j) + 4 * g + i) * D + col];
    } else {
#pragma unroll
      for (int j = 0; j < HT; ++j) S[j] = zero4();
    }
#pragma unroll
    for (int j = 0; j < HB; ++j) {
      const int kb = h * HB + j;
      sf[j] = frag2_from_acc<T16>(S[2 * j], S[2 * j + 1]);
      Sx[0][(SXP * kb) * kWave + lane] = sf[j].hi;
      if constexpr (OUT) Sx[0][(2 * kb + 1) * kWave + lane] = sf[j].lo;
    }
    __syncthreads();
    __syncthreads();
    // S is carried decayed by the coming chunk's gam_C: the accumulator of
    // that chunk's update, while sf (and Sx) hold the undecayed state.
    if constexpr (kGated) {
      const float g0 = Es[0][C - 1];
#pragma unroll
      for (int j = 0; j < HT; ++j) S[j] *= g0;
    }

    // loop-invariant lane offsets
    uint32_t ktr[HT / 2];
#pragma unroll
    for (int j = 0; j < HT / 2; ++j) ktr[j] = tr_off<D>(g, n, h * (HT / 2) + j);
    const uint32_t goff = (uint32_t)(4 * g) * 4;        // tables: row 16 ti + 4 g
    const uint32_t xoff = (uint32_t)lane * 16;          // Sx / Uf / BVs slots
    // The K rows of K S for chunk c+1 are loaded at the end of chunk c (the
    // DMA K wave lands each chunk's K within the step that issues it), so
    // that K S starts as soon as the barrier opens the chunk.  (The state
    // pass lands K one chunk ahead only: it loads them in the step.)
    constexpr bool kKPre = OUT && kDelta;
    Frag<T16> kfn[4][NKB];
    if constexpr (kKPre) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) kfn[ti][kb] = frag_row_at<D>(Ks, roff[kb] + kRows16 * ti);
    }

    for (int c = 0; c < NC; ++c) {
      const uint32_t kslot = slot(c, KR, kTileB);
      // gam_C of chunk c+1 (its tables are two chunks ahead), read first:
      // the split at the end of the chunk waits for it.  The load is
      // unconditional, from a clamped slot, so that no branch splits the
      // loop body.
      float gn = 1.f;
      if constexpr (kGated) {
        const float e = lds_ld<float>(Es, slot(c + 1 < NC ? c + 1 : c, 3, C * 4) + (C - 1) * 4);
        gn = c + 1 < NC ? e : 1.f;
      }
      Frag<T16> ktf[HT][2];
      if constexpr (kDelta) {
        const uint32_t tslot = slot(c, 3, C * 4);
        const uint32_t bvslot = slot(c, 2, 4 * kWave * 16);
        Frag<T16> kf[4][NKB], th[kTFrags], sh[NKB];
        f32x4 bv[4], bb[4], fr[4];
        // K S over the whole state: this half's bf16 S from registers, the
        // other half's from the split both halves published at the end of
        // the last chunk (the state enters K S as one bf16: its rounding
        // stays well inside the tolerance, the split being kept everywhere
        // else).  Both halves form the same products in the same order, so
        // they hold the same K S and need no exchange.
        {
          const uint32_t a = slot(c, 2, SXP * NKB * kWave * 16) + xoff;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            // (register arrays only ever indexed by compile-time values)
            if (kb / HB == h) sh[kb] = sf[kb % HB].hi;
            else sh[kb].v = lds_ld<bf16x8>(Sx, a + (SXP * kb) * kWave * 16);
          }
        }
        if constexpr (kKPre) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) kf[ti][kb] = kfn[ti][kb];
        } else {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            const uint32_t a = kslot + roff[kb];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) kf[ti][kb] = frag_row_at<D>(Ks, a + kRows16 * ti);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x4 ks[4];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
          ks[ti] = zero4();
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) mma(kf[ti][kb], sh[kb], ks[ti]);
        }
        // the other operands under the products
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) bv[ti] = lds_ld<f32x4>(BVs, bvslot + xoff + ti * kWave * 16);
        if constexpr (kGated) {
#pragma unroll
          for (int ti = 0; ti < 4; ++ti) {
            bb[ti] = lds_ld<f32x4>(BGs, tslot + goff + 64 * ti);
            fr[ti] = lds_ld<f32x4>(Fs, tslot + goff + 64 * ti);
          }
        } else {
          const uint32_t gslot = slot(c, NG, C * 4);
#pragma unroll
          for (int ti = 0; ti < 4; ++ti) bb[ti] = lds_ld<f32x4>(Bs, gslot + goff + 64 * ti);
        }
        {
          const uint32_t a = slot(c, 3, kTRecFrags * kWave * 16) + xoff;
#pragma unroll
          for (int f = 0; f < kTFrags; ++f) th[f].v = lds_ld<bf16x8>(Ts, a + f * kWave * 16);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < HT; ++j)
            ktf[j][kb] = frag_tr_at(Ks, kslot + ktr[j / 2] + 8 * (j % 2) + 64 * D * kb, kRows16);
        // R = diag(beta) V - diag(beta gam) K S
        f32x4 rr[4], un[4];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
          for (int i = 0; i < 4; ++i) rr[ti][i] = fmaf(-bb[ti][i], ks[ti][i], bv[ti][i]);
        Frag2<T16> rf[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) rf[kb] = frag2_from_acc<T16>(rr[2 * kb], rr[2 * kb + 1]);
        // U_new = T R, R split
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
          un[ti] = zero4();
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            if (kb <= ti / 2) mma_ab2(th[tfi(ti, kb)], rf[kb], un[ti]);
        }
        // U_new in float for the output waves (which split it); both halves
        // hold all of it, each publishes two of its row tiles
        if constexpr (OUT) {
          const uint32_t a = slot(c, 2, 4 * kWave * 16) + xoff;
          if (h == 0) {
            lds_st<f32x4>(Uf, a + 0 * kWave * 16, un[0]);
            lds_st<f32x4>(Uf, a + 1 * kWave * 16, un[1]);
          } else {
            lds_st<f32x4>(Uf, a + 2 * kWave * 16, un[2]);
            lds_st<f32x4>(Uf, a + 3 * kWave * 16, un[3]);
          }
        }
        // operand of the state update: diag(gam_C / gam) U_new (gated), U_new
        Frag2<T16> ut[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if constexpr (kGated) {
            const f32x4 flo = fr[2 * kb], fhi = fr[2 * kb + 1];
            const float slo[4] = {flo[0], flo[1], flo[2], flo[3]};
            const float shi[4] = {fhi[0], fhi[1], fhi[2], fhi[3]};
            ut[kb] = frag2_from_acc_scaled<T16>(un[2 * kb], un[2 * kb + 1], slo, shi);
          } else {
            ut[kb] = frag2_from_acc<T16>(un[2 * kb], un[2 * kb + 1]);
          }
        }
        // S += K^T ut on this half (S is already decayed by gam_C)
#pragma unroll
        for (int j = 0; j < HT; ++j)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) mma_ab2(ktf[j][kb], ut[kb], S[j]);
        if constexpr (kKPre) {
          const uint32_t ns = slot(c + 1 < NC ? c + 1 : c, KR, kTileB);
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
              kfn[ti][kb] = frag_row_at<D>(Ks, ns + roff[kb] + kRows16 * ti);
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < HT; ++j)
            ktf[j][kb] = frag_tr_at(Ks, kslot + ktr[j / 2] + 8 * (j % 2) + 64 * D * kb, kRows16);
        if constexpr (kGated) {
          // S += K^T diag(gam_C / gam) V (S is already decayed by gam_C):
          // f V in float from the DMA V wave, split here
          const uint32_t bvslot = slot(c, 2, 4 * kWave * 16);
          Frag2<T16> ut[2];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            ut[kb] = frag2_from_acc<T16>(lds_ld<f32x4>(BVs, bvslot + xoff + (2 * kb) * kWave * 16),
                                         lds_ld<f32x4>(BVs, bvslot + xoff + (2 * kb + 1) * kWave * 16));
#pragma unroll
          for (int j = 0; j < HT; ++j)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) mma_ab2(ktf[j][kb], ut[kb], S[j]);
        } else {
          // S <- S + K^T V (V exact)
          const uint32_t vslot = slot(c, NV, C * 16 * 2);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const Frag<T16> vf = frag_col_tr_v((const char*)Vs + vslot, 32 * kb, g, n);
#pragma unroll
            for (int j = 0; j < HT; ++j) mma(ktf[j][kb], vf, S[j]);
          }
        }
      }
      // publish the split of this half of S_{c+1}; in gated mode the split
      // consumes S and the state carried on is S_{c+1} decayed by gam_C of
      // chunk c+1
      {
        const uint32_t a = slot(c + 1, 2, SXP * NKB * kWave * 16) + xoff;
#pragma unroll
        for (int j = 0; j < HB; ++j) {
          const int kb = h * HB + j;
          if constexpr (kGated) {
            const f32x4 d0 = S[2 * j] * gn, d1 = S[2 * j + 1] * gn;
            sf[j] = frag2_from_acc<T16>(S[2 * j], S[2 * j + 1]);
            S[2 * j] = d0;
            S[2 * j + 1] = d1;
          } else {
            sf[j] = frag2_from_acc<T16>(S[2 * j], S[2 * j + 1]);
          }
          lds_st<bf16x8>(Sx, a + (SXP * kb) * kWave * 16, sf[j].hi.v);
          if constexpr (OUT) lds_st<bf16x8>(Sx, a + (2 * kb + 1) * kWave * 16, sf[j].lo.v);
        }
      }
      __syncthreads();
    }
    if (si.sf) {
#pragma unroll
      for (int j = 0; j < HT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          si.sf[(size_t)dk_of_row(16 * (h * HT + j) + 4 * g + i) * D + col] = S[j][i];
    }
  } else if (wave == kDmaK) {
    // ================= DMA of K and the gates
    for (int cc = 0; cc < KR - 1 && cc < NC; ++cc) issue_k(cc);
    for (int cc = 0; cc < NG - 1 && cc < NC; ++cc) issue_gates(cc);
    vm_wait<0>();
    __syncthreads();
    __syncthreads();
    for (int c = 0; c < NC; ++c) {
      // the slots these fill held chunk c-1, last read before the barrier
      // that opened this chunk
      if (c + KR - 1 < NC) issue_k(c + KR - 1);
      if (c + NG - 1 < NC) issue_gates(c + NG - 1);
      if (c + 1 < NC) make_bv(c + 1);
      // Everything issued before this chunk has landed, and this chunk's K
      // too where it is issued one chunk ahead (the state pass) or the chain
      // reads it early (the delta modes' output pass): it is issued before
      // the gates.  Loads complete in issue order, so while any earlier
      // transfer is outstanding all N of this chunk's are too.
      if constexpr (KR == 3 && !(OUT && kDelta)) {
        if (c + NG - 1 < NC) vm_wait<NDMAK>();
        else vm_wait<0>();
      } else {
        if (c + NG - 1 < NC) vm_wait<NGATE>();
        else vm_wait<0>();
      }
      __syncthreads();
    }
  } else if (wave == kDmaV) {
    // ================= DMA of V and T; tables; beta V
    if (vzero) {
      // the V ring of a transition stream: zero once, never loaded
      u32x4* vr = reinterpret_cast<u32x4*>(&Vs[0][0]);
#pragma unroll
      for (int i = 0; i < NV * C * 16 * 2 / 16 / kWave; ++i) vr[i * kWave + lane] = u32x4{0u, 0u, 0u, 0u};
    }
    issue_q(0);
    for (int cc = 0; cc < 3 && cc < NC; ++cc)
      if (!vzero) issue_v(cc);
    if constexpr (kDelta) {
      issue_t(0);
      if (NC > 1) issue_t(1);
    }
    vm_wait<0>();
    if (NC <= 3) zero_v_tail();
    __syncthreads();        // (the DMA K wave's gates have landed)
    tables(0);
    if (NC > 1) tables(1);
    make_bv(0);
    __syncthreads();
    for (int c = 0; c < NC; ++c) {
      // Q of the next chunk first (its slot held chunk c-1, last read before
      // the barrier that opened this chunk): the wait below leaves only this
      // chunk's V and T transfers outstanding
      if (c + 1 < NC) issue_q(c + 1);
      if (c + 3 < NC && !vzero) issue_v(c + 3);
      if constexpr (kDelta)
        if (c + 2 < NC) issue_t(c + 2);
      if (c + 2 < NC) tables(c + 2);
      if (c + 3 < NC) vm_wait<NDMAV>();
      else vm_wait<0>();
      // the last chunk's V landed at the latest in the wait above at c = NC - 3
      if (c == NC - 3) zero_v_tail();
      __syncthreads();
    }
  } else {
    // ================= output waves, one row tile each
    if constexpr (OUT) {
      const f32x4 dcol4 = DSKIP ? *reinterpret_cast<const f32x4*>(dskip + (size_t)si.head * D + col0 + 4 * g)
                                : zero4();
      auto run = [&](auto ti_c) {
        constexpr int TI = decltype(ti_c)::value;
        Frag<T16> qc[NKB], qn[NKB];
        if constexpr (!kQLds) load_q<D, TI>(qc, q, hbase, NC == 1 ? nlast : C, g, n);
        __syncthreads();
        __syncthreads();
        f32x4 sc[4], qs, ot;
        for (int c = 0; c < NC; ++c) {
          if constexpr (kQLds) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
              qc[kb] = frag_row_at<D>(Qs, slot(c, 2, kTileB) + roff[kb] + kRows16 * TI);
          } else {
            // Q of the next chunk (the last chunk's again at the end: the
            // load is unconditional)
            const int cn = c + 1 < NC ? c + 1 : c;
            load_q<D, TI>(qn, q, hbase + (size_t)cn * C, cn == NC - 1 ? nlast : C, g, n);
          }
          if (c > 0) {
            out_rows<D, MODE, DSKIP, TI>(sc, qs, Uf[kDelta ? (c - 1) % 2 : 0], Vs[(c - 1) % NV], ot,
                                         g, n, lane, dcol4);
            store_rows<D, TI>(ot, out_, (hbase + (size_t)(c - 1) * C) * D + col0, out_bf16, g, n, C);
          }
          const T16* Kc = Ks[c % KR];
          const float* gc = Gs[kGated ? c % 3 : 0];
          const float* gk = kQSide ? Gk[c % 3] : gc;
          const float* ec = kQSide ? Eq[c % 3] : Es[kGated ? c % 3 : 0];
          scores_qs<D, kGated, TI>(qc, Kc, gc, gk, ec, Ra[kFac ? c % 3 : 0], Cb[kFac ? c % 3 : 0],
                                   Sx[c % 2], roff, sc, qs, g, n, lane);
          if constexpr (!kQLds) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) qc[kb] = qn[kb];
          }
          __syncthreads();
        }
        const int c = NC - 1;
        out_rows<D, MODE, DSKIP, TI>(sc, qs, Uf[kDelta ? c % 2 : 0], Vs[c % NV], ot, g, n, lane,
                                     dcol4);
        store_rows<D, TI>(ot, out_, (hbase + (size_t)c * C) * D + col0, out_bf16, g, n, nlast);
      };
      if (wave == 2) run(std::integral_constant<int, 3>{});
      else if (wave == 3) run(std::integral_constant<int, 2>{});
      else if (wave == 6) run(std::integral_constant<int, 0>{});
      else run(std::integral_constant<int, 1>{});
    }
  }
}

// ---------------------------------------------------------------- wide kernel (no erase)
//
// The modes without erase carry no per-chunk solve, and their chain is one
// product per chunk (S <- gam_C S + K^T diag(f) V), so a chunk step is
// mostly the output: scores, Q S and Aqk V.  The chain kernel above repeats
// the scores and the staging of Q and K in each of a head's D / 16 column
// tiles.  This kernel gives one workgroup 64 state columns of a stream, one
// wave per 16-column tile, so the four tiles share one copy of the chunk's
// Q, K and masked decayed scores:
//
//   every wave   issues a quarter of the DMA of chunk c+2 (Q, K: rings of
//                three swizzled tiles) and its own tile's V columns; forms
//                its share of the ten lower score tiles of chunk c+1
//                (Aqk^T tiles K Q^T, packed as the split operand blocks
//                (TI, kb) the output reads: wave 0 blocks (3,0), (0,0);
//                wave 1 (3,1), (2,1); wave 2 (2,0); wave 3 (1,0)) into a
//                double buffer; then, for chunk c, O^T = S^T Q^T diag(gam)
//                + V^T Aqk^T for its 16 columns and all 64 rows (S split,
//                V exact, the scores split), and S <- gam_C S + K^T diag(f) V
//                (V exact, or f V split with decay).
//
// One barrier per chunk.  The state tile stays in the wave's accumulators
// in the permuted row order of the chain kernel; the output is stored
// transposed (one 8- or 16-byte store per lane and row tile).  The gates
// arrive by DMA (wave 0) and each wave forms the chunk's cumulative decay
// in registers, exchanging values across lanes with ds_bpermute.
template <int D, bool GATED>
__global__ __launch_bounds__(256) void lin_wide_kernel(
    const T16* __restrict__ q, const T16* __restrict__ k, const T16* __restrict__ v,
    const float* __restrict__ log_alpha, void* __restrict__ out_, StreamMap smap, int NS,
    int out_bf16) {
  constexpr int NKB = D / 32;
  constexpr int NST = D / 16;              // state row tiles (dk)
  constexpr int NCG = D / 64;              // 64-column groups per stream
  constexpr int TILE = C * D;
  constexpr uint32_t kTileB = 2 * TILE;
  constexpr uint32_t kRows16 = 32 * D;
  constexpr int NTILE = TILE * 2 / 1024;   // DMA instructions per Q or K tile
  constexpr int NTW = NTILE / 4;           // of them per wave
  constexpr int NR = 3;                    // Q, K, V rings: DMA two chunks ahead
  constexpr int NAB = 6;                   // score blocks (TI, kb), kb <= TI / 2
  constexpr int NDMA = 2 * NTW + 2;        // per wave and chunk (+1 gates on wave 0)
  static_assert(NTILE % 4 == 0, "the tile DMA splits over four waves");

  __shared__ __attribute__((aligned(16))) T16 Qs[NR][TILE];
  __shared__ __attribute__((aligned(16))) T16 Ks[NR][TILE];
  __shared__ __attribute__((aligned(16))) T16 Vs[NR][4][C * 16];
  __shared__ __attribute__((aligned(16))) Frag<T16> Ab[2 * NAB * kWave];
  __shared__ __attribute__((aligned(16))) float Ls[GATED ? NR : 1][C];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int g = lane / 16;
  const int n = lane % 16;

  // stream and column group; the groups of one stream share an XCD
  int sidx, cg;
  {
    const int b = blockIdx.x;
    if (NCG > 1 && NS % 8 == 0) {
      const int x = b % 8, s = b / 8;
      cg = s % NCG;
      sidx = (s / NCG) * 8 + x;
    } else {
      sidx = b / NCG;
      cg = b % NCG;
    }
  }
  const int col0 = 64 * cg + 16 * wave;       // this wave's state columns
  const int col = col0 + n;
  const StreamInfo si = stream_info(smap, sidx);
  const size_t hbase = si.row0;
  const int L = si.len;
  if (L == 0) {
    if (si.sf) {
#pragma unroll
      for (int r = 0; r < D / 4; ++r) {
        const size_t e = (size_t)(4 * r + g) * D + col;
        si.sf[e] = si.s0 ? si.s0[e] : 0.f;
      }
    }
    return;
  }
  // chunks; rows past the sequence read the last valid row, have log alpha
  // = 0 and V = 0, and are not stored (as in the chain kernel)
  const int NC = (L + C - 1) / C;
  const int nlast = L - (NC - 1) * C;

  uint32_t roff[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) roff[kb] = unit_off<D>(n, 4 * kb + g);
  auto slot = [](int c, int depth, uint32_t bytes) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(c % depth) * bytes));
  };

  // this wave's part of the DMA of chunk cc
  auto issue = [&](int cc) {
    const size_t r0 = hbase + (size_t)cc * C;
    const int nr = cc == NC - 1 ? nlast : C;
    // source offset of lane l's unit of DMA instruction m (the swizzled
    // layout of dma_tile_offsets), computed per instruction: m depends on
    // the wave, and a register array indexed by it would go to scratch
    auto toff = [&](int m) {
      constexpr int RB = 2 * D;
      const int byte = 1024 * m + 16 * lane;
      const int r = byte / RB, ul = (byte % RB) / 16;
      return (uint32_t)(min(r, nr - 1) * RB + ((ul ^ swz_key<D>(r)) << 4));
    };
    const uint32_t qb = lds_addr(Qs[cc % NR]), kb_ = lds_addr(Ks[cc % NR]);
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
      const int m = wave * NTW + i;
      const uint32_t o = toff(m);
      dma16s(q + r0 * D, o, __builtin_amdgcn_readfirstlane(qb + 1024 * m));
      dma16s(k + r0 * D, o, __builtin_amdgcn_readfirstlane(kb_ + 1024 * m));
    }
    const uint32_t vb = lds_addr(Vs[cc % NR][wave]);
#pragma unroll
    for (int m = 0; m < 2; ++m)
      dma16s(v + r0 * D + col0,
             (uint32_t)((min(32 * m + lane / 2, nr - 1) * D + 8 * (lane % 2)) * 2),
             __builtin_amdgcn_readfirstlane(vb + 1024 * m));
    if constexpr (GATED)
      if (wave == 0)
        dma4s(log_alpha + r0, (uint32_t)min(lane, nr - 1) * 4, lds_addr(Ls[cc % NR]));
  };
  // V rows past the sequence set to zero once the last chunk's V has landed
  auto zero_v_tail = [&]() {
    if (nlast < C && lane >= nlast) {
      u32x4* row = reinterpret_cast<u32x4*>(Vs[(NC - 1) % NR][wave] + lane * 16);
      row[0] = u32x4{0u, 0u, 0u, 0u};
      row[1] = u32x4{0u, 0u, 0u, 0u};
    }
  };
  // the chunk's cumulative log decay g (lane = token), 0 past the sequence
  auto gates = [&](int cc) {
    const float la = lane < (cc == NC - 1 ? nlast : C) ? Ls[cc % NR][lane] : 0.f;
    return wave_inclusive_scan(la);
  };
  auto lane_val = [](float x, int src) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x)));
  };

  // score tile (TI, t) of chunk cc, t <= TI: K rows 16 t .. against Q rows
  // 16 TI .., masked on the diagonal, decayed by exp(g_r - g_i)
  auto score_tile = [&](int cc, int TI, int t, float gv) {
    const uint32_t ks = slot(cc, NR, kTileB), qs = ks;
    f32x4 s = zero4();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const Frag<T16> kf = frag_row_at<D>(Ks, ks + roff[kb] + kRows16 * t);
      const Frag<T16> qf = frag_row_at<D>(Qs, qs + roff[kb] + kRows16 * TI);
      mma(kf, qf, s);
    }
    // element (K row i = 16 t + 4 g + e, Q row r = 16 TI + n)
    float gr = 0.f;
    if constexpr (GATED) gr = lane_val(gv, 16 * TI + n);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * t + 4 * g + e, r = 16 * TI + n;
      float d = 1.f;
      if constexpr (GATED) d = __expf(fminf(gr - lane_val(gv, i), 0.f));
      s[e] = i <= r ? s[e] * d : 0.f;
    }
    return s;
  };
  auto put_block = [&](int bi, const f32x4& a, const f32x4& b) {
    const Frag2<T16> f = frag2_from_acc<T16>(a, b);
    const uint32_t o = (uint32_t)lane * 16;
    lds_st<bf16x8>(Ab, o + (2 * bi) * kWave * 16, f.hi.v);
    lds_st<bf16x8>(Ab, o + (2 * bi + 1) * kWave * 16, f.lo.v);
  };
  // this wave's blocks of chunk cc (block index tfi(TI, kb))
  auto scores = [&](int cc) {
    float gv = 0.f;
    if constexpr (GATED) gv = gates(cc);
    if (wave == 0) {
      put_block(tfi(3, 0), score_tile(cc, 3, 0, gv), score_tile(cc, 3, 1, gv));
      put_block(tfi(0, 0), score_tile(cc, 0, 0, gv), zero4());
    } else if (wave == 1) {
      put_block(tfi(3, 1), score_tile(cc, 3, 2, gv), score_tile(cc, 3, 3, gv));
      put_block(tfi(2, 1), score_tile(cc, 2, 2, gv), zero4());
    } else if (wave == 2) {
      put_block(tfi(2, 0), score_tile(cc, 2, 0, gv), score_tile(cc, 2, 1, gv));
    } else {
      put_block(tfi(1, 0), score_tile(cc, 1, 0, gv), score_tile(cc, 1, 1, gv));
    }
  };

  // the state tile: register row p of tile j holds dk index dk_of_row(p)
  f32x4 S[NST];
  if (si.s0) {
#pragma unroll
    for (int j = 0; j < NST; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[j][i] = si.s0[(size_t)dk_of_row(16 * j + 4 * g + i) * D + col];
  } else {
#pragma unroll
    for (int j = 0; j < NST; ++j) S[j] = zero4();
  }
  // K^T operand offsets of state tile j (token block 0)
  uint32_t ktr[NST];
#pragma unroll
  for (int j = 0; j < NST; ++j) ktr[j] = tr_off<D>(g, n, j / 2) + 8 * (j % 2);

  // Everything but the last issued chunk has landed: each wave waits for its
  // own transfers (vector-memory operations retire in issue order; stores
  // issued after the chunk's DMA only make the wait stricter).
  auto wait_but_last = [&]() {
    if constexpr (GATED) {
      if (wave == 0) vm_wait<NDMA + 1>();
      else vm_wait<NDMA>();
    } else {
      vm_wait<NDMA>();
    }
  };

  issue(0);
  if (NC > 1) {
    issue(1);
    wait_but_last();
  } else {
    vm_wait<0>();
    zero_v_tail();
  }
  __syncthreads();

  for (int c = 0; c < NC; ++c) {
    // chunk c landed before the barrier that opened this step; c+2 goes to
    // the slot chunk c-1 held, read for the last time before that barrier
    if (c + 2 < NC) issue(c + 2);
    scores(c);
    __syncthreads();
    const uint32_t ts = slot(c, NR, kTileB);
    const uint32_t as = (uint32_t)lane * 16;
    const T16* Vt = Vs[c % NR][wave];
    float gv = 0.f, gC = 0.f;
    if constexpr (GATED) {
      gv = gates(c);
      gC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), kWave - 1));
    }
    // V columns of this tile over the two token blocks (exact)
    Frag<T16> vf[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) vf[kb] = frag_col_tr_v(Vt, 32 * kb, g, n);
    // S split (the entering state) as the A operand of S^T Q^T
    Frag2<T16> sx[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sx[kb] = frag2_from_acc<T16>(S[2 * kb], S[2 * kb + 1]);
    const int nrows = c == NC - 1 ? nlast : C;
    const size_t ob0 = (hbase + (size_t)c * C) * D + col0;
    auto out_tile = [&](auto ti_c) {
      constexpr int TI = decltype(ti_c)::value;
      f32x4 o = zero4();
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const Frag<T16> qf = frag_row_at<D>(Qs, ts + roff[kb] + kRows16 * TI);
        mma(sx[kb].lo, qf, o);
        mma(sx[kb].hi, qf, o);
      }
      if constexpr (GATED) o *= __expf(lane_val(gv, 16 * TI + n));
#pragma unroll
      for (int kb = 0; kb <= TI / 2; ++kb) {
        Frag<T16> ah, al;
        ah.v = lds_ld<bf16x8>(Ab, as + (2 * tfi(TI, kb)) * kWave * 16);
        al.v = lds_ld<bf16x8>(Ab, as + (2 * tfi(TI, kb) + 1) * kWave * 16);
        mma(vf[kb], al, o);
        mma(vf[kb], ah, o);
      }
      store_rows<D, TI>(o, out_, ob0, out_bf16, g, n, nrows);
    };
    out_tile(std::integral_constant<int, 0>{});
    out_tile(std::integral_constant<int, 1>{});
    out_tile(std::integral_constant<int, 2>{});
    out_tile(std::integral_constant<int, 3>{});
    // S <- gam_C S + K^T diag(f) V
    if constexpr (GATED) {
      const float dC = __expf(gC);
#pragma unroll
      for (int j = 0; j < NST; ++j) S[j] *= dC;
      // f V, split: slot j of block kb is token 32 kb + kidx(g, j)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        Frag2<T16> fv;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float f = __expf(gC - lane_val(gv, 32 * kb + kidx(g, j)));
          fv.set(j, (float)vf[kb].v[j] * f);
        }
#pragma unroll
        for (int j = 0; j < NST; ++j) {
          const Frag<T16> kt = frag_tr_at(Ks, ts + ktr[j] + 64 * D * kb, kRows16);
          mma_ab2(kt, fv, S[j]);
        }
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < NST; ++j) {
          const Frag<T16> kt = frag_tr_at(Ks, ts + ktr[j] + 64 * D * kb, kRows16);
          mma(kt, vf[kb], S[j]);
        }
    }
    // chunk c+1 lands before the barrier (the one issued at this step's top
    // may stay in flight: it is read two steps on)
    if (c + 2 < NC) wait_but_last();
    else vm_wait<0>();
    // the last chunk's V, issued at c = NC - 3, has landed in the full wait
    // of c = NC - 2 and is read at c = NC - 1
    if (c == NC - 2) zero_v_tail();
    __syncthreads();
  }
  if (si.sf) {
#pragma unroll
    for (int j = 0; j < NST; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) si.sf[(size_t)dk_of_row(16 * j + 4 * g + i) * D + col] = S[j][i];
  }
}

// ---------------------------------------------------------------- segment scan

constexpr int kScanThreads = 512;
constexpr int kScanCols = 8;         // state columns per workgroup
constexpr int kScanGroup = 8;        // threads per segment of the log-alpha sums

// States entering the segments of the sequence-parallel forward, from the
// state pass's X_p and M_p: S_in(0) = S0, S_in(1) = X_0 and S_in(p+1) =
// M_p S_in(p) + X_p, with M_p = exp(G_p) I, G_p the sum of log alpha over
// segment p, in the modes without erase.  One workgroup per 8-column tile
// of one sequence's state (M acts on the rows, so column tiles are
// independent; narrow tiles shorten each step of the serial chain), float
// FMA throughout, in a fixed order.
//
// Thread (r, u) (TPR threads per state row r) owns columns u CPT .. + CPT - 1
// of the tile.  With erase, each step is an 8-column product over the D
// rows of S_in(p) held in LDS: the thread sums the 4-row blocks b = u +
// TPR j of its row of M_p (registers, loaded one step ahead), and the TPR
// partial sums of a row are added across the adjacent lanes.  Without
// erase there is no product: every segment's G_p is summed first, then each
// thread runs the scalar recursion on its own elements.
template <int D, bool ERASE, bool GATED>
__global__ __launch_bounds__(kScanThreads) void seg_scan_kernel(
    StreamMap m, const float* __restrict__ log_alpha) {
  constexpr int SC = kScanCols;
  constexpr int NCT = D / SC;
  constexpr int TPR = kScanThreads / D;  // threads per state row: 4 or 8
  constexpr int CPT = SC / TPR;          // columns per thread: 2 or 1
  constexpr int NBT = D / 4 / TPR;       // 4-row blocks of the sums per thread
  constexpr int LDS_P = 12;              // row pitch of the S_in tile (floats)
  __shared__ __attribute__((aligned(16))) float Sc[ERASE ? D : 1][LDS_P];
  __shared__ float G[GATED && !ERASE ? 1024 : 1];
  const int bh = blockIdx.x / NCT, ct = blockIdx.x % NCT;
  const int t = threadIdx.x, r = t / TPR, u = t % TPR;
  const size_t e0 = (size_t)r * D + ct * SC + u * CPT;   // this thread's first element
  const int nc = (m.sm.L + m.sm.C - 1) / m.sm.C;
  const int P = m.P;
  auto state = [&](const float* base, int p) { return base + ((size_t)bh * P + p) * m.dd; };

  float cur[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) cur[j] = m.S0 ? m.S0[(size_t)bh * m.dd + e0 + j] : 0.f;
  auto put = [&](int p) {
    float* out = m.sin + ((size_t)bh * P + p) * m.dd + e0;
#pragma unroll
    for (int j = 0; j < CPT; ++j) out[j] = cur[j];
  };
  put(0);
  {
    const float* X = state(m.xs, 0) + e0;
#pragma unroll
    for (int j = 0; j < CPT; ++j) cur[j] = X[j];
  }
  put(1);

  if constexpr (ERASE) {
    f32x4 mv[NBT], mn[NBT];
    float xv[CPT], xn[CPT];
    auto fetch = [&](int p, f32x4 (&mr)[NBT], float (&xr)[CPT]) {
      const float* M = state(m.ms, p) + (size_t)r * D;
#pragma unroll
      for (int j = 0; j < NBT; ++j) mr[j] = *reinterpret_cast<const f32x4*>(M + 4 * (u + TPR * j));
      const float* X = state(m.xs, p) + e0;
#pragma unroll
      for (int j = 0; j < CPT; ++j) xr[j] = X[j];
    };
    if (P > 2) fetch(1, mv, xv);
    for (int p = 2; p < P; ++p) {
      __syncthreads();                   // the last step's reads of Sc are done
#pragma unroll
      for (int j = 0; j < CPT; ++j) Sc[r][u * CPT + j] = cur[j];
      __syncthreads();
      if (p + 1 < P) fetch(p, mn, xn);   // next step's operands, in flight meanwhile
      float a[SC];
#pragma unroll
      for (int c = 0; c < SC; ++c) a[c] = 0.f;
#pragma unroll
      for (int j = 0; j < NBT; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float* row = Sc[4 * (u + TPR * j) + e];
#pragma unroll
          for (int c4 = 0; c4 < SC / 4; ++c4) {
            const f32x4 sv = *reinterpret_cast<const f32x4*>(row + 4 * c4);
#pragma unroll
            for (int i = 0; i < 4; ++i) a[4 * c4 + i] = fmaf(mv[j][e], sv[i], a[4 * c4 + i]);
          }
        }
#pragma unroll
      for (int o = 1; o < TPR; o *= 2)
#pragma unroll
        for (int c = 0; c < SC; ++c) a[c] += __shfl_xor(a[c], o);
#pragma unroll
      for (int j = 0; j < CPT; ++j) cur[j] = a[u * CPT + j] + xv[j];
      put(p);
#pragma unroll
      for (int j = 0; j < NBT; ++j) mv[j] = mn[j];
#pragma unroll
      for (int j = 0; j < CPT; ++j) xv[j] = xn[j];
    }
  } else {
    if constexpr (GATED) {
      // G_p for p = 1 .. P - 2: kScanGroup threads per segment, a fixed
      // strided order and a butterfly within the group
      const float* la = log_alpha + (size_t)bh * m.sm.L;
      constexpr int NSEG = kScanThreads / kScanGroup;
      for (int p0 = 1; p0 < P - 1; p0 += NSEG) {
        const int p = p0 + t / kScanGroup;
        float sum = 0.f;
        if (p < P - 1) {
          const int t0 = seg_chunk0(p, P, nc) * m.sm.C;
          const int t1 = min(seg_chunk0(p + 1, P, nc) * m.sm.C, m.sm.L);
          for (int i = t0 + t % kScanGroup; i < t1; i += kScanGroup) sum += la[i];
        }
#pragma unroll
        for (int o = 1; o < kScanGroup; o *= 2) sum += __shfl_xor(sum, o);
        if (p < P - 1 && t % kScanGroup == 0) G[p] = sum;
      }
      __syncthreads();
    }
    // eight steps' X loads ahead of their stores (which the compiler must
    // otherwise assume they depend on)
    constexpr int kBatch = 8;
    for (int p0 = 2; p0 < P; p0 += kBatch) {
      float xb[kBatch][CPT];
#pragma unroll
      for (int k = 0; k < kBatch; ++k)
        if (p0 + k < P) {
          const float* X = state(m.xs, p0 + k - 1) + e0;
#pragma unroll
          for (int j = 0; j < CPT; ++j) xb[k][j] = X[j];
        }
#pragma unroll
      for (int k = 0; k < kBatch; ++k)
        if (p0 + k < P) {
          const float d = GATED ? __expf(G[p0 + k - 1]) : 1.f;
#pragma unroll
          for (int j = 0; j < CPT; ++j) cur[j] = fmaf(d, cur[j], xb[k][j]);
          put(p0 + k);
        }
    }
  }
}

// ---------------------------------------------------------------- output norm

// Output normalisation of the fused epilogue: each (token, head) row of out
// becomes o / sqrt(mean(o^2) + eps) times w[h] (ones without w) -- the norm
// that takes the place of linear attention's dropped denominator ("The
// Devil in Linear Transformer" in "LinearAttention 概述").  HBM-bound, in
// place.  Grid y walks the (b, h) sequences (L token rows of [B, H, L, dv],
// or the H heads of [H, T, dv]), so a workgroup knows its head without any
// per-row division and keeps its lanes' weights in registers; grid x walks
// a sequence's rows.  Every lane moves 16 bytes (EPL elements) per access,
// D / EPL adjacent lanes hold one row and reduce its sum of squares among
// themselves, kOutNormU row groups' loads are in flight per wave (at eight
// waves per SIMD, 128 KiB per compute unit: what HBM's latency asks for).
constexpr int kOutNormU = 4;

template <typename TO, int D>
__global__ __launch_bounds__(256) void out_norm_kernel(TO* __restrict__ out, int L, int H,
                                                       unsigned nseq, const float* __restrict__ w,
                                                       float eps) {
  constexpr int EPL = 16 / (int)sizeof(TO);        // elements per lane
  constexpr int LPR = D / EPL;                     // lanes per row
  constexpr int RPW = kWave / LPR;                 // rows per wave and group
  typedef TO vec __attribute__((ext_vector_type(EPL)));
  const int lane = threadIdx.x % kWave;
  const int c0 = (lane % LPR) * EPL;
  for (unsigned sq = blockIdx.y; sq < nseq; sq += gridDim.y) {
  float wv[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) wv[j] = 1.f;
  if (w) {
    const f32x4* wp = reinterpret_cast<const f32x4*>(w + (size_t)(sq % H) * D + c0);
#pragma unroll
    for (int j = 0; j < EPL / 4; ++j) {
      const f32x4 t = wp[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[4 * j + i] = t[i];
    }
  }
  TO* seq = out + (size_t)sq * L * D;
  const int groups = (L + RPW - 1) / RPW;
  const int nwaves = gridDim.x * (256 / kWave);
  for (int gi = blockIdx.x * (256 / kWave) + threadIdx.x / kWave; gi < groups;
       gi += kOutNormU * nwaves) {
    int row[kOutNormU];
    bool live[kOutNormU];
    vec x[kOutNormU];
#pragma unroll
    for (int u = 0; u < kOutNormU; ++u) {
      row[u] = (gi + u * nwaves) * RPW + lane / LPR;
      live[u] = gi + u * nwaves < groups && row[u] < L;
      x[u] = live[u] ? *reinterpret_cast<const vec*>(seq + (size_t)row[u] * D + c0) : vec{};
    }
#pragma unroll
    for (int u = 0; u < kOutNormU; ++u) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < EPL; ++j) ss = fmaf((float)x[u][j], (float)x[u][j], ss);
#pragma unroll
      for (int off = LPR / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
      if (!live[u]) continue;
      const float r = rsqrtf(ss / D + eps);
      vec y;
#pragma unroll
      for (int j = 0; j < EPL; ++j) y[j] = (TO)((float)x[u][j] * r * wv[j]);
      *reinterpret_cast<vec*>(seq + (size_t)row[u] * D + c0) = y;
    }
  }
  }
}

// ---------------------------------------------------------------- non-causal form

// Partial K^T V of one block of tokens of one (b, h) sequence: the sum over
// its tokens of k_t v_t^T, a dk x dv float tile per workgroup.  The chunks
// of a sum are independent, so token blocks run in parallel and the partial
// states are added afterwards.  K and V chunks are DMA'd into LDS (double
// buffered, the chain kernel's swizzled tile layout); both MFMA operands
// are transposed reads of those tiles -- a K^T fragment (dk rows, token
// contraction) and a V fragment (token contraction, dv columns) have the
// same shape -- so the result arrives in the permuted state-row order on
// both sides, undone at the store.  Wave w owns output row tiles w * TMW ..;
// rows past the sequence's end read the last token and their V rows are
// zeroed, so they add nothing.
template <int D>
__global__ __launch_bounds__(kThreads) void kv_kernel(const T16* __restrict__ k,
                                                      const T16* __restrict__ v,
                                                      float* __restrict__ partial, int L,
                                                      int TB, int NB) {
  constexpr int NT = D / 16;                 // 16-wide tiles per side
  constexpr int TMW = NT / 4;                // output row tiles per wave
  constexpr int NTILE = C * 2 * D / 1024;    // DMA instructions per tile
  constexpr uint32_t kRows16 = 32 * D;
  __shared__ __attribute__((aligned(16))) T16 Ks[2][C * D];
  __shared__ __attribute__((aligned(16))) T16 Vs[2][C * D];
  const size_t bh = blockIdx.x / NB;
  const int t0 = (blockIdx.x % NB) * TB, t1 = min(t0 + TB, L);
  const int nch = (t1 - t0 + C - 1) / C;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int g = lane / 16, n = lane % 16;
  const T16* kb0 = k + (bh * L + t0) * D;
  const T16* vb0 = v + (bh * L + t0) * D;
  auto rows_of = [&](int c) { return min(C, t1 - t0 - c * C); };
  // each wave moves half of the K or the V tile of a chunk
  constexpr int NH = NTILE / 2;
  auto issue = [&](int c) {
    uint32_t off[NTILE];
    dma_tile_offsets<D>(off, lane, rows_of(c));
    const T16* src = (wave < 2 ? kb0 : vb0) + (size_t)c * C * D;
    const uint32_t base = lds_addr(wave < 2 ? Ks[c % 2] : Vs[c % 2]);
    const int m0 = (wave % 2) * NH;
#pragma unroll
    for (int m = 0; m < NH; ++m)
      dma16s(src, off[m0 + m], __builtin_amdgcn_readfirstlane(base + 1024 * (m0 + m)));
  };
  f32x4 acc[TMW][NT];
#pragma unroll
  for (int i = 0; i < TMW; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = zero4();
  issue(0);
  for (int c = 0; c < nch; ++c) {
    if (c + 1 < nch) {
      issue(c + 1);
      vm_wait<NH>();                 // this wave's part of chunk c has landed
    } else {
      vm_wait<0>();
    }
    __syncthreads();
    const int nr = rows_of(c);
    if (nr < C) {
      // V rows past the end of the block's tokens (the sequence's end) add
      // nothing: zeroed once the whole tile has landed
      if (wave == 2)
        for (int r = nr; r < C; ++r) {
          T16* row = Vs[c % 2] + r * D;
          for (int j = lane; j < D; j += kWave) row[j] = (T16)0.f;
        }
      __syncthreads();
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      Frag<T16> a[TMW];
#pragma unroll
      for (int i = 0; i < TMW; ++i) {
        const int tm = wave * TMW + i;
        a[i] = frag_tr_at(Ks[c % 2], tr_off<D>(g, n, tm / 2) + 8 * (tm % 2) + 64 * D * kb,
                          kRows16);
      }
#pragma unroll
      for (int tn = 0; tn < NT; ++tn) {
        const Frag<T16> b = frag_tr_at(Vs[c % 2],
                                       tr_off<D>(g, n, tn / 2) + 8 * (tn % 2) + 64 * D * kb,
                                       kRows16);
#pragma unroll
        for (int i = 0; i < TMW; ++i) mma(a[i], b, acc[i][tn]);
      }
    }
    __syncthreads();                 // buffer c % 2 is free for chunk c + 2
  }
  float* out = partial + (size_t)blockIdx.x * D * D;
#pragma unroll
  for (int i = 0; i < TMW; ++i)
#pragma unroll
    for (int tn = 0; tn < NT; ++tn)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        out[(size_t)dk_of_row(16 * (wave * TMW + i) + 4 * g + e) * D + dk_of_row(16 * tn + n)] =
            acc[i][tn][e];
}

// S = S0 + the sum of the partial states (fixed order): one thread per state
// element.  Written to the workspace's S slot and, if given, to S_final.
__global__ __launch_bounds__(256) void seg_sum_kernel(const float* __restrict__ xs,
                                                      const float* __restrict__ S0,
                                                      float* __restrict__ S,
                                                      float* __restrict__ S_final, int P,
                                                      size_t dd, size_t n) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  const size_t bh = e / dd, i = e % dd;
  const float* x = xs + bh * P * dd + i;
  float a = S0 ? S0[e] : 0.f;
  for (int p = 0; p < P; ++p) a += x[(size_t)p * dd];
  S[e] = a;
  if (S_final) S_final[e] = a;
}

// O = Q S for every token of a (b, h) sequence (the bidirectional form:
// each token reads the state after the whole sequence).  One workgroup per
// (b, h) and kQsRows tokens; S (float) is split once into bf16 hi + lo
// operand fragments in LDS.  The product is computed transposed, O^T = S^T
// Q^T, whose fragments are the same per-lane values as those of Q S (a
// 16 x 32 operand holds row n, contraction 8 g ..): the accumulator then
// gives each lane 4 consecutive columns of one token.  A float output
// stores them (16 bytes); a bf16 one regroups two column tiles over the
// four lane groups first (eight shuffles), so that each lane stores 8
// consecutive columns in one 16-byte write and each store instruction
// writes 64-byte pieces of its 16 rows instead of 32-byte ones (10% less
// time).  Wave w of 4 computes token rows 16 w .. + 15 of each 64-token
// block, all column tiles, the next block's Q fragments loaded (16-byte
// reads straight from HBM) before this block's products.
constexpr int kQsRows = 1024;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kQsThreads = 256;

template <int D>
__global__ __launch_bounds__(kQsThreads) void qs_kernel(const T16* __restrict__ q,
                                                      const float* __restrict__ S,
                                                      void* __restrict__ out_, int L,
                                                      int out_bf16) {
  constexpr int NKB = D / 32, NCT = D / 16;
  __shared__ __attribute__((aligned(16))) Frag2<T16> Sf[NKB][NCT][kWave];
  const int nblk = (L + kQsRows - 1) / kQsRows;
  const size_t bh = blockIdx.x / nblk;
  const int r0 = (blockIdx.x % nblk) * kQsRows;
  const int r1 = min(r0 + kQsRows, L);
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int g = lane / 16, n = lane % 16;
  const float* Sb = S + bh * D * D;
  for (int f = wave; f < NKB * NCT; f += kQsThreads / kWave) {
    const int kb = f / NCT, ct = f % NCT;
    Frag2<T16> x;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const float a0 = Sb[(size_t)(32 * kb + 8 * g + j) * D + 16 * ct + n];
      const float a1 = Sb[(size_t)(32 * kb + 8 * g + j + 1) * D + 16 * ct + n];
      uint32_t hi, lo;
      split_pair(a0, a1, hi, lo);
      const bf16x2 h = __builtin_bit_cast(bf16x2, hi), l = __builtin_bit_cast(bf16x2, lo);
      x.hi.v[j] = h[0];
      x.hi.v[j + 1] = h[1];
      x.lo.v[j] = l[0];
      x.lo.v[j + 1] = l[1];
    }
    Sf[kb][ct][lane] = x;
  }
  __syncthreads();
  constexpr int kStep = 16 * kQsThreads / kWave;     // token rows per block
  const T16* qb = q + bh * (size_t)L * D;
  auto load_q = [&](int rt, Frag<T16> (&qf)[NKB]) {
    const int rr = min(rt + n, L - 1);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      qf[kb].v = *reinterpret_cast<const bf16x8*>(qb + (size_t)rr * D + 32 * kb + 8 * g);
  };
  Frag<T16> qf[NKB], qn[NKB];
  int rt = r0 + 16 * wave;                       // this wave's first token row
  if (rt < r1) load_q(rt, qf);
  for (; rt < r1; rt += kStep) {
    if (rt + kStep < r1) load_q(rt + kStep, qn);
    const int tok = rt + n;                      // this lane's token
    if (out_bf16) {
#pragma unroll
      for (int p = 0; p < NCT / 2; ++p) {
        // tiles 2 p and 2 p + 1 as packed bf16 pairs: lane (g, n) holds
        // columns 32 p + 16 h + 4 g .. + 3 of token n in w[h]
        uint32_t w[2][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          f32x4 acc = zero4();
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            mma(Sf[kb][2 * p + h][lane].hi, qf[kb], acc);
            mma(Sf[kb][2 * p + h][lane].lo, qf[kb], acc);
          }
          const u32x2 y = __builtin_bit_cast(u32x2, __builtin_convertvector(acc, bf16x4));
          w[h][0] = y[0];
          w[h][1] = y[1];
        }
        // lane (g, n) gathers columns 32 p + 8 g .. + 7: tile 2 p + g / 2,
        // from lane groups 2 (g % 2) and 2 (g % 2) + 1 of the same token
        const int sa = 32 * (g & 1) + n, sb = sa + 16;
        const uint32_t a00 = __shfl(w[0][0], sa), a01 = __shfl(w[0][1], sa);
        const uint32_t a10 = __shfl(w[1][0], sa), a11 = __shfl(w[1][1], sa);
        const uint32_t b00 = __shfl(w[0][0], sb), b01 = __shfl(w[0][1], sb);
        const uint32_t b10 = __shfl(w[1][0], sb), b11 = __shfl(w[1][1], sb);
        const bool lo = g < 2;
        if (tok < r1) {
          const size_t o = (bh * (size_t)L + tok) * D + 32 * p + 8 * g;
          *reinterpret_cast<u32x4*>(static_cast<T16*>(out_) + o) =
              u32x4{lo ? a00 : a10, lo ? a01 : a11, lo ? b00 : b10, lo ? b01 : b11};
        }
      }
    } else {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          mma(Sf[kb][ct][lane].hi, qf[kb], acc);
          mma(Sf[kb][ct][lane].lo, qf[kb], acc);
        }
        if (tok < r1)
          *reinterpret_cast<f32x4*>(static_cast<float*>(out_) + (bh * (size_t)L + tok) * D +
                                    16 * ct + 4 * g) = acc;
      }
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) qf[kb] = qn[kb];
  }
}

// ---------------------------------------------------------------- launches

constexpr int kComputeUnits = 256;   // gfx950 (MI355X)
constexpr int kMinSegChunks = 4;     // shortest segment worth a pass
constexpr int kMaxSegments = 64;

// Workspace layout: the T fragments of every chunk (delta modes); then, for
// P > 1, X, M and S_in, [BH, P, D, D] float each; then, with the fused
// prologue, its four per-token arrays (beta, log alpha, lq, lk), each on a
// 256-byte boundary.
size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

size_t tsolve_bytes(const ChunkArgs& a) {
  return mode_erase(a.mode) ? chunk_slots(a) * kTRecFrags * kWave * sizeof(u32x4) : 0;
}

size_t seg_states_offset(const ChunkArgs& a) { return align256(tsolve_bytes(a)); }

size_t seg_states_end(const ChunkArgs& a) {
  if (a.P <= 1) return tsolve_bytes(a);
  return seg_states_offset(a) + 3 * (size_t)a.B * a.H * a.P * a.d * a.d * sizeof(float);
}

size_t token_rows(const ChunkArgs& a) { return (a.cu ? (size_t)a.H : (size_t)a.B * a.H) * a.L; }

size_t pro_stride(const ChunkArgs& a) { return align256(token_rows(a) * sizeof(float)); }

// The arguments the chain kernels run with: with the fused prologue, its
// gates and, for normalised q and k, the decayed kernel of the mode.
ChunkArgs kernel_args(const ChunkArgs& a) {
  ChunkArgs k = a;
  if (a.pro) {
    const ProArrays p = pro_arrays(a);
    k.mode = kernel_mode(a);
    k.log_alpha = p.log_alpha;
    k.beta = p.beta;
  }
  return k;
}

StreamMap stream_map(const ChunkArgs& a, int pass) {
  StreamMap m{seq_map(a), a.S0, a.S_final, pass, a.P, mode_erase(a.mode),
              (size_t)a.d * a.d, nullptr, nullptr, nullptr};
  if (pass != kPassWhole) {
    float* base = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + seg_states_offset(a));
    const size_t n = (size_t)a.B * a.H * a.P * m.dd;
    m.xs = base;
    m.ms = base + n;
    m.sin = base + 2 * n;
  }
  return m;
}

// a: the kernel arguments (kernel_args of the call)
template <int D, int MODE, bool OUT, bool FUSED, bool DSKIP>
hipError_t launch_one(const ChunkArgs& a, int pass, hipStream_t st) {
  const StreamMap m = stream_map(a, pass);
  const size_t ns = (size_t)a.B * a.H * m.per_seq();
  const dim3 grid((unsigned)(ns * (D / 16))), block(OUT ? 512 : 256);
  const ProArrays pro = FUSED ? pro_arrays(a) : ProArrays{};
  chunk_pipe_kernel<D, MODE, OUT, FUSED, DSKIP><<<grid, block, 0, st>>>(
      static_cast<const T16*>(a.q), static_cast<const T16*>(a.k), static_cast<const T16*>(a.v),
      a.log_alpha, a.beta, static_cast<const u32x4*>(a.workspace), a.out, m, (int)ns,
      a.out_bf16 ? 1 : 0, pro, a.dskip);
  return hipGetLastError();
}

// the residual in v only where outputs are written
template <int D, int MODE, bool OUT, bool FUSED>
hipError_t launch_ep(const ChunkArgs& a, int pass, hipStream_t st) {
  if constexpr (OUT)
    if (a.dskip) return launch_one<D, MODE, OUT, FUSED, true>(a, pass, st);
  return launch_one<D, MODE, OUT, FUSED, false>(a, pass, st);
}

// a: the call's arguments (raw gates when the prologue activates them)
template <int D, bool GATED, bool PRO, bool TS>
hipError_t launch_t(const ChunkArgs& a, hipStream_t st) {
  const size_t items = chunk_slots(a);
  ProIn pro{};
  if (PRO)
    pro = ProIn{static_cast<const T16*>(a.q), pro_arrays(a), a.pro, a.gate_scale,
                mode_erase(a.mode), mode_decay(a.mode)};
  t_solve_kernel<D, GATED, PRO, TS><<<dim3((unsigned)items), dim3(kWave), 0, st>>>(
      static_cast<const T16*>(a.k), a.log_alpha, a.beta, static_cast<u32x4*>(a.workspace),
      seq_map(a), pro);
  return hipGetLastError();
}

template <int D, bool OUT>
hipError_t launch_d(const ChunkArgs& call, int pass, hipStream_t st) {
  const ChunkArgs a = kernel_args(call);
  const bool fused = call.pro & kProQKNorm;
  switch (a.mode) {
    case kModeLinear: return launch_ep<D, kModeLinear, OUT, false>(a, pass, st);
    case kModeDelta: return launch_ep<D, kModeDelta, OUT, false>(a, pass, st);
    case kModeGatedLinear:
      return fused ? launch_ep<D, kModeGatedLinear, OUT, true>(a, pass, st)
                   : launch_ep<D, kModeGatedLinear, OUT, false>(a, pass, st);
    default:
      return fused ? launch_ep<D, kModeGatedDelta, OUT, true>(a, pass, st)
                   : launch_ep<D, kModeGatedDelta, OUT, false>(a, pass, st);
  }
}

template <int D>
hipError_t launch_scan_d(const ChunkArgs& call, hipStream_t st) {
  const ChunkArgs a = kernel_args(call);
  const StreamMap m = stream_map(a, kPassOut);
  const dim3 grid((unsigned)((size_t)a.B * a.H * (D / kScanCols))), block(kScanThreads);
  if (mode_erase(a.mode))
    seg_scan_kernel<D, true, false><<<grid, block, 0, st>>>(m, a.log_alpha);
  else if (mode_decay(a.mode))
    seg_scan_kernel<D, false, true><<<grid, block, 0, st>>>(m, a.log_alpha);
  else
    seg_scan_kernel<D, false, false><<<grid, block, 0, st>>>(m, a.log_alpha);
  return hipGetLastError();
}

}  // namespace

size_t chunk_pipe_workspace_bytes(const ChunkArgs& a) {
  if (!a.pro) return seg_states_end(a);
  return align256(seg_states_end(a)) + 4 * pro_stride(a);
}

// Token blocks per sequence of the non-causal K^T V: about four workgroups
// per compute unit in all (each streams its block's K and V once), each
// block whole chunks and non-empty; every block adds one partial state to
// write and sum.
int plan_sum_segments(const ChunkArgs& a) {
  const long seqs = (long)a.B * a.H;
  const int nc = (a.L + C - 1) / C;
  // one round of kv_kernel: two of its workgroups (64 KiB of LDS each) per
  // compute unit.  More blocks add rounds, and each writes a d x d partial
  // that seg_sum_kernel reads back (at B8 H16 L4096 d128, four blocks per
  // sequence instead of eight: 68 + 11 instead of 73 + 18 us).
  long P = (2L * kComputeUnits + seqs - 1) / seqs;
  P = std::max(1L, std::min({P, (long)nc, (long)kMaxSegments}));
  // the balanced block size, then the blocks it takes (none empty)
  const int per = (int)((nc + P - 1) / P);
  return (nc + per - 1) / per;
}

// X (P per sequence), an unused M block and S (slot 0 of S_in): the state
// layout of the sequence-parallel passes.
size_t noncausal_workspace_bytes(const ChunkArgs& a) {
  return 3 * (size_t)a.B * a.H * a.P * a.d * a.d * sizeof(float);
}

ProArrays pro_arrays(const ChunkArgs& a) {
  char* base = static_cast<char*>(a.workspace) + align256(seg_states_end(a));
  const size_t s = pro_stride(a);
  return ProArrays{reinterpret_cast<float*>(base), reinterpret_cast<float*>(base + s),
                   reinterpret_cast<float*>(base + 2 * s), reinterpret_cast<float*>(base + 3 * s)};
}

// Rough cost, in chunk steps of the whole-sequence walk, of P segments,
// fitted to measured step times (gated delta rule, dk = dv = 128, L = 65536,
// one to sixteen heads):
// * state pass: two of its workgroups fit on a compute unit, but two sharing
//   one run slower: 0.8 of a walk step while every workgroup has a unit of
//   its own, 1.35 per round of two per unit beyond that;
// * output pass: one workgroup per unit, 1.05 of a walk step per round;
// * each pass fills and drains its pipeline (about 3 steps), and the scan
//   adds about 2 steps per segment with erase (a dk x dk by dk x 8 product
//   per workgroup), 0.3 without.
// Segments are used when they save at least 5% on this estimate.
int plan_segments(const ChunkArgs& a) {
  if (!a.in_bf16 || a.cu) return 1;
  const long chains = (long)a.B * a.H * (a.d / 16);
  const long nc = ((long)a.L + C - 1) / C;
  const long cus = kComputeUnits;
  const double whole = (double)((chains + cus - 1) / cus) * nc;
  double best = whole;
  int best_p = 1;
  for (int P = 2; P <= nc / kMinSegChunks && P <= kMaxSegments; ++P) {
    const long n1 = chains * ((P - 1) + (mode_erase(a.mode) ? P - 2 : 0));
    const long n3 = chains * P;
    const double steps = (double)((nc + P - 1) / P) + 3.0;
    const double state = n1 <= cus ? 0.8 : 1.35 * (double)((n1 + 2 * cus - 1) / (2 * cus));
    const double out = 1.05 * (double)((n3 + cus - 1) / cus);
    const double scan = (mode_erase(a.mode) ? 2.0 : 0.3) * P;
    const double cost = (state + out) * steps + scan;
    if (cost < best) {
      best = cost;
      best_p = P;
    }
  }
  return best < 0.95 * whole ? best_p : 1;
}

hipError_t launch_tsolve(const ChunkArgs& a, hipStream_t st) {
  if (a.pro) {
    // the prologue, and T in the delta modes (with the decay exponents of
    // the prologue's gates, zero where the mode has none)
    if (mode_erase(a.mode))
      return a.d == 64 ? launch_t<64, true, true, true>(a, st) : launch_t<128, true, true, true>(a, st);
    return a.d == 64 ? launch_t<64, true, true, false>(a, st) : launch_t<128, true, true, false>(a, st);
  }
  const bool gated = mode_decay(a.mode);
  if (a.d == 64)
    return gated ? launch_t<64, true, false, true>(a, st) : launch_t<64, false, false, true>(a, st);
  return gated ? launch_t<128, true, false, true>(a, st) : launch_t<128, false, false, true>(a, st);
}

hipError_t launch_out_norm(const ChunkArgs& a, hipStream_t st) {
  const unsigned nseq = (unsigned)(a.cu ? a.H : a.B * a.H);
  // rows per workgroup pass: 4 waves of kWave * EPL / D rows, kOutNormU
  // passes in flight; about 8 workgroups per compute unit in all
  const int per = 4 * kOutNormU * kWave * (a.out_bf16 ? 8 : 4) / a.d;
  const unsigned gx = (unsigned)std::max<long>(
      1, std::min<long>((a.L + per - 1) / per, (8L * kComputeUnits + nseq - 1) / nseq));
  const dim3 grid(gx, std::min(nseq, 65535u)), block(256);
  if (a.out_bf16) {
    if (a.d == 64)
      out_norm_kernel<T16, 64><<<grid, block, 0, st>>>(static_cast<T16*>(a.out), a.L, a.H,
                                                        nseq, a.norm_w, a.norm_eps);
    else
      out_norm_kernel<T16, 128><<<grid, block, 0, st>>>(static_cast<T16*>(a.out), a.L, a.H,
                                                         nseq, a.norm_w, a.norm_eps);
  } else {
    if (a.d == 64)
      out_norm_kernel<float, 64><<<grid, block, 0, st>>>(static_cast<float*>(a.out), a.L, a.H,
                                                          nseq, a.norm_w, a.norm_eps);
    else
      out_norm_kernel<float, 128><<<grid, block, 0, st>>>(static_cast<float*>(a.out), a.L, a.H,
                                                           nseq, a.norm_w, a.norm_eps);
  }
  return hipGetLastError();
}

// Non-causal form: partial K^T V of a.P token blocks per sequence (chunk-
// aligned, kv_kernel), S = S0 + their sum, then O = Q S.  a.mode is LINEAR;
// the workspace holds the partials (P per sequence) and S.
hipError_t launch_noncausal(const ChunkArgs& a, hipStream_t st) {
  const StreamMap m = stream_map(a, kPassOut);    // the state arrays' layout
  const size_t n = (size_t)a.B * a.H * m.dd;
  float* S = m.sin;                       // slot 0 of S_in holds S
  const int nc = (a.L + C - 1) / C;
  const int TB = (nc + a.P - 1) / a.P * C;  // tokens per block; every block is non-empty
  const dim3 kvgrid((unsigned)((size_t)a.B * a.H * a.P)), block(kThreads);
  if (a.d == 64)
    kv_kernel<64><<<kvgrid, block, 0, st>>>(static_cast<const T16*>(a.k),
                                            static_cast<const T16*>(a.v), m.xs, a.L, TB, a.P);
  else
    kv_kernel<128><<<kvgrid, block, 0, st>>>(static_cast<const T16*>(a.k),
                                             static_cast<const T16*>(a.v), m.xs, a.L, TB, a.P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  seg_sum_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st>>>(m.xs, a.S0, S,
                                                                         a.S_final, a.P, m.dd, n);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t wgs = (size_t)a.B * a.H * ((a.L + kQsRows - 1) / kQsRows);
  if (a.d == 64)
    qs_kernel<64><<<dim3((unsigned)wgs), dim3(kQsThreads), 0, st>>>(
        static_cast<const T16*>(a.q), S, a.out, a.L, a.out_bf16 ? 1 : 0);
  else
    qs_kernel<128><<<dim3((unsigned)wgs), dim3(kQsThreads), 0, st>>>(
        static_cast<const T16*>(a.q), S, a.out, a.L, a.out_bf16 ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_chunk_state(const ChunkArgs& a, hipStream_t st) {
  return a.d == 64 ? launch_d<64, false>(a, kPassState, st)
                   : launch_d<128, false>(a, kPassState, st);
}

hipError_t launch_seg_scan(const ChunkArgs& a, hipStream_t st) {
  return a.d == 64 ? launch_scan_d<64>(a, st) : launch_scan_d<128>(a, st);
}

// The wide kernel serves the whole-sequence walk of the modes without erase
// (not the segment passes, nor the fused q, k norms or residual, which the
// chain kernel's tables and output waves carry) where its workgroups (one
// per stream and 64 columns) fill the compute units: per column tile and
// chunk it is faster, but it has a quarter of the chain kernel's
// workgroups, each with a chain as long.
bool use_wide(const ChunkArgs& a) {
  const long wgs = (long)a.B * a.H * (a.d / 64);
  return !mode_erase(a.mode) && a.P <= 1 && !(a.pro & kProQKNorm) && !a.dskip &&
         wgs >= kComputeUnits;
}

template <int D>
hipError_t launch_wide_d(const ChunkArgs& call, hipStream_t st) {
  const ChunkArgs a = kernel_args(call);
  const StreamMap m = stream_map(a, kPassWhole);
  const size_t ns = (size_t)a.B * a.H;
  const dim3 grid((unsigned)(ns * (D / 64))), block(256);
  if (mode_decay(a.mode))
    lin_wide_kernel<D, true><<<grid, block, 0, st>>>(
        static_cast<const T16*>(a.q), static_cast<const T16*>(a.k), static_cast<const T16*>(a.v),
        a.log_alpha, a.out, m, (int)ns, a.out_bf16 ? 1 : 0);
  else
    lin_wide_kernel<D, false><<<grid, block, 0, st>>>(
        static_cast<const T16*>(a.q), static_cast<const T16*>(a.k), static_cast<const T16*>(a.v),
        a.log_alpha, a.out, m, (int)ns, a.out_bf16 ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_chunk_pipe(const ChunkArgs& a, hipStream_t st) {
  if (use_wide(a)) return a.d == 64 ? launch_wide_d<64>(a, st) : launch_wide_d<128>(a, st);
  const int pass = a.P > 1 ? kPassOut : kPassWhole;
  return a.d == 64 ? launch_d<64, true>(a, pass, st) : launch_d<128, true>(a, pass, st);
}

}  // namespace la
