// Device-side helpers shared by the gfx950 kernels of liblachunk.
//
// Element types: q, k, v and outputs are either float or __bf16 (bfloat16,
// round-to-nearest-even on conversion from float); everything is accumulated
// in float.
//
// MFMA fragments.  The dense contractions use v_mfma_f32_16x16x32_bf16 (bf16
// inputs) or eight v_mfma_f32_16x16x4_f32 (float inputs) per 32-deep block of
// the contraction.  For a 16 x 16 output tile and a 32-deep block:
//
//   * lane l (0..63) holds, for the A operand, 8 values of row (l % 16) and,
//     for the B operand, 8 values of column (l % 16); the 8 values are the
//     contraction indices kidx(l / 16, j), j = 0..7, of the block;
//   * the float accumulator holds, in lane l, column (l % 16) and rows
//     4 * (l / 16) + i, i = 0..3.
//
// Because a contraction is a plain sum, any assignment of contraction
// indices to (lane group, slot) works as long as A and B use the same one.
// We use
//
//     kidx(g, j) = 4 g + j         for j < 4
//     kidx(g, j) = 16 + 4 g + j - 4 for j >= 4
//
// which is exactly the set of rows an accumulator lane holds in two
// vertically stacked 16 x 16 tiles.  A tile produced by one product can
// therefore feed the next product as its B operand straight from registers
// (convert and pack, no data movement), which keeps the carried state and
// the per-chunk update vectors on chip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace la {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// Contraction index held in slot j of lane group g (see the file comment).
__device__ __forceinline__ constexpr int kidx(int g, int j) {
  return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4);
}

// Eight operand values of one lane for one 32-deep block.
template <typename T>
struct Frag;

template <>
struct Frag<__bf16> {
  bf16x8 v;
  __device__ __forceinline__ void set(int j, float x) { v[j] = (__bf16)x; }
};

template <>
struct Frag<float> {
  float v[8];
  __device__ __forceinline__ void set(int j, float x) { v[j] = x; }
};

// acc += A(16 x 32) * B(32 x 16) over one 32-deep block.
__device__ __forceinline__ void mma(const Frag<__bf16>& a, const Frag<__bf16>& b,
                                    f32x4& acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}

__device__ __forceinline__ void mma(const Frag<float>& a, const Frag<float>& b,
                                    f32x4& acc) {
  // Each 16x16x4 step consumes one value per lane: lane group g supplies
  // contraction index kidx(g, j) in step j, so the 8 steps cover the block.
#pragma unroll
  for (int j = 0; j < 8; ++j)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], acc, 0, 0, 0);
}

// B operand built from two stacked accumulator tiles (rows 0-15 in `lo`,
// rows 16-31 in `hi`), each scaled per row.  scale_lo[i] / scale_hi[i] apply
// to the rows this lane holds (4 * g + i and 16 + 4 * g + i).
template <typename T>
__device__ __forceinline__ Frag<T> frag_from_acc(const f32x4& lo, const f32x4& hi) {
  Frag<T> f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f.set(i, lo[i]);
    f.set(4 + i, hi[i]);
  }
  return f;
}

template <typename T>
__device__ __forceinline__ Frag<T> frag_from_acc_scaled(const f32x4& lo, const f32x4& hi,
                                                        const float* slo,
                                                        const float* shi) {
  Frag<T> f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f.set(i, lo[i] * slo[i]);
    f.set(4 + i, hi[i] * shi[i]);
  }
  return f;
}

// Operand row of a row-major matrix in LDS or global memory: 8 values
// m[row][k0 + kidx(g, j)], i.e. two runs of 4 contiguous elements.
__device__ __forceinline__ Frag<__bf16> frag_row(const __bf16* p, int g) {
  Frag<__bf16> f;
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(p + 4 * g);
  const bf16x4 b = *reinterpret_cast<const bf16x4*>(p + 16 + 4 * g);
  f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}

__device__ __forceinline__ Frag<float> frag_row(const float* p, int g) {
  Frag<float> f;
  const f32x4 a = *reinterpret_cast<const f32x4*>(p + 4 * g);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 16 + 4 * g);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f.v[i] = a[i];
    f.v[4 + i] = b[i];
  }
  return f;
}

// Operand column of a row-major matrix with row pitch `ld` (elements):
// 8 values m[k0 + kidx(g, j)][col], gathered one by one.
template <typename T>
__device__ __forceinline__ Frag<T> frag_col(const T* p, int ld, int g) {
  Frag<T> f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f.set(j, to_f32(p[kidx(g, j) * ld]));
  return f;
}

// Same, scaling element j by s[kidx(g, j)] before the conversion.
template <typename T>
__device__ __forceinline__ Frag<T> frag_col_scaled(const T* p, int ld, int g,
                                                   const float* s) {
  Frag<T> f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f.set(j, to_f32(p[kidx(g, j) * ld]) * s[kidx(g, j)]);
  return f;
}


// Operand row read from a float matrix and converted to the MFMA input type:
// 8 values p[kidx(g, j)].  Used for the float UT matrix T feeding bf16 MFMAs.
template <typename T>
__device__ __forceinline__ Frag<T> frag_row_cvt(const float* p, int g) {
  Frag<T> f;
  const f32x4 a = *reinterpret_cast<const f32x4*>(p + 4 * g);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 16 + 4 * g);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f.set(i, a[i]);
    f.set(4 + i, b[i]);
  }
  return f;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Cooperative copy of a ROWS x COLS tile from global memory (row pitch gld
// elements) into LDS (row pitch LLD elements) with 16-byte vectors.
template <typename T, int ROWS, int COLS, int LLD, int NTHREADS>
__device__ __forceinline__ void stage_tile(T* lds, const T* __restrict__ src, size_t gld,
                                           int tid) {
  constexpr int VE = 16 / sizeof(T);
  constexpr int VPR = COLS / VE;
  constexpr int NV = ROWS * VPR;
  static_assert(COLS % VE == 0 && (LLD * sizeof(T)) % 16 == 0, "16-byte rows");
#pragma unroll
  for (int it = 0; it < (NV + NTHREADS - 1) / NTHREADS; ++it) {
    const int p = tid + it * NTHREADS;
    if (NV % NTHREADS == 0 || p < NV) {
      const int r = p / VPR, cv = p % VPR;
      *reinterpret_cast<u32x4*>(lds + r * LLD + cv * VE) =
          *reinterpret_cast<const u32x4*>(src + r * gld + cv * VE);
    }
  }
}

// Lanes of x moved by a DPP pattern; lanes without a source (or outside
// row_mask) read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or_zero(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, true));
}

// Inclusive prefix sum across the 64 lanes of a wave, in registers: a
// Hillis-Steele scan inside each row of 16 lanes (row_shr 1, 2, 4, 8), then
// lane 15 of rows 0 and 2 added to rows 1 and 3 (row_bcast:15) and lane 31
// added to rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ float wave_inclusive_scan(float x) {
  x += dpp_or_zero<0x111, 0xf>(x);
  x += dpp_or_zero<0x112, 0xf>(x);
  x += dpp_or_zero<0x114, 0xf>(x);
  x += dpp_or_zero<0x118, 0xf>(x);
  x += dpp_or_zero<0x142, 0xa>(x);
  x += dpp_or_zero<0x143, 0xc>(x);
  return x;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------------------
// Split operands.  A float value x feeding a bf16 MFMA is carried as
// hi = bf16(x) and lo = bf16(x - hi); a product with an exact bf16 operand a
// is then a*hi + a*lo, accurate to about 2^-16 relative instead of 2^-8.
// Two split operands multiply as a.hi*b.hi + a.hi*b.lo + a.lo*b.hi (the
// a.lo*b.lo term is below float rounding).  For float inputs the MFMA is
// already float and nothing is split: `lo` is unused and all lo products
// compile away.
template <typename T>
struct IsBf16 {
  static constexpr bool value = false;
};
template <>
struct IsBf16<__bf16> {
  static constexpr bool value = true;
};

template <typename T>
struct Frag2 {
  Frag<T> hi, lo;
  __device__ __forceinline__ void set(int j, float x) {
    if constexpr (IsBf16<T>::value) {
      const __bf16 h = (__bf16)x;
      hi.v[j] = h;
      lo.v[j] = (__bf16)(x - (float)h);
    } else {
      hi.set(j, x);
    }
  }
};

// acc += a * b with b split
template <typename T>
__device__ __forceinline__ void mma_ab2(const Frag<T>& a, const Frag2<T>& b, f32x4& acc) {
  if constexpr (IsBf16<T>::value) mma(a, b.lo, acc);
  mma(a, b.hi, acc);
}

// acc += a * b with both split
template <typename T>
__device__ __forceinline__ void mma_a2b2(const Frag2<T>& a, const Frag2<T>& b, f32x4& acc) {
  if constexpr (IsBf16<T>::value) {
    mma(a.lo, b.hi, acc);
    mma(a.hi, b.lo, acc);
  }
  mma(a.hi, b.hi, acc);
}

// Split B operand from two stacked accumulator tiles (see frag_from_acc).
template <typename T>
__device__ __forceinline__ Frag2<T> frag2_from_acc(const f32x4& lo, const f32x4& hi) {
  Frag2<T> f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f.set(i, lo[i]);
    f.set(4 + i, hi[i]);
  }
  return f;
}

template <typename T>
__device__ __forceinline__ Frag2<T> frag2_from_acc_scaled(const f32x4& lo, const f32x4& hi,
                                                          const float* slo,
                                                          const float* shi) {
  Frag2<T> f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f.set(i, lo[i] * slo[i]);
    f.set(4 + i, hi[i] * shi[i]);
  }
  return f;
}

// bf16 specialisations: two values are rounded per instruction
// (v_cvt_pk_bf16_f32), and each remainder x - hi is one bf16 dot product
// of the packed pair with (-1, 0) or (0, -1) accumulated onto x
// (v_dot2c_f32_bf16): the product is exact and x - hi is representable, so
// the remainder is exact, 2 instructions per value in all.  Same roundings
// as Frag2::set.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// The two selector pairs, held in scalar registers.  Written as constants,
// (-1, 0) would be folded into the inline constant -1.0, which the
// instruction reads as the 32-bit pattern 0xbf800000, i.e. the pair (0, -1).
struct SplitSel {
  uint32_t lo_half, hi_half;
};
__device__ __forceinline__ SplitSel split_sel() {
  uint32_t a = 0x0000bf80u, b = 0xbf800000u;
  asm("" : "+s"(a), "+s"(b));
  return SplitSel{a, b};
}

__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const SplitSel s = split_sel();
  const bf16x2 h = __builtin_convertvector(f32x2{x0, x1}, bf16x2);
  const float r0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, s.lo_half), h, x0, false);
  const float r1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, s.hi_half), h, x1, false);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r0, r1}, bf16x2));
  hi = __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ Frag2<__bf16> frag2_pack(float a0, float a1, float a2, float a3,
                                                    float b0, float b1, float b2, float b3) {
  uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
  split_pair(a0, a1, h0, l0);
  split_pair(a2, a3, h1, l1);
  split_pair(b0, b1, h2, l2);
  split_pair(b2, b3, h3, l3);
  Frag2<__bf16> f;
  f.hi.v = __builtin_bit_cast(bf16x8, u32x4{h0, h1, h2, h3});
  f.lo.v = __builtin_bit_cast(bf16x8, u32x4{l0, l1, l2, l3});
  return f;
}

template <>
__device__ __forceinline__ Frag2<__bf16> frag2_from_acc<__bf16>(const f32x4& lo, const f32x4& hi) {
  return frag2_pack(lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]);
}

template <>
__device__ __forceinline__ Frag2<__bf16> frag2_from_acc_scaled<__bf16>(const f32x4& lo,
                                                                      const f32x4& hi,
                                                                      const float* slo,
                                                                      const float* shi) {
  return frag2_pack(lo[0] * slo[0], lo[1] * slo[1], lo[2] * slo[2], lo[3] * slo[3],
                    hi[0] * shi[0], hi[1] * shi[1], hi[2] * shi[2], hi[3] * shi[3]);
}

// Split operand from a float row p[kidx(g, j)] (a row of a float matrix
// as the A operand, or a column stored contiguously as the B operand).
template <typename T>
__device__ __forceinline__ Frag2<T> frag2_row(const float* p, int g) {
  Frag2<T> f;
  const f32x4 a = *reinterpret_cast<const f32x4*>(p + 4 * g);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 16 + 4 * g);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f.set(i, a[i]);
    f.set(4 + i, b[i]);
  }
  return f;
}

// Split A operand from a float row p[kidx(g, j)], each value scaled by
// s[kidx(g, j)] first (a matrix times a diagonal on the right).
template <typename T>
__device__ __forceinline__ Frag2<T> frag2_row_scaled(const float* p, int g, const float* s) {
  Frag2<T> f;
  const f32x4 a = *reinterpret_cast<const f32x4*>(p + 4 * g);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 16 + 4 * g);
  const f32x4 sa = *reinterpret_cast<const f32x4*>(s + 4 * g);
  const f32x4 sb = *reinterpret_cast<const f32x4*>(s + 16 + 4 * g);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f.set(i, a[i] * sa[i]);
    f.set(4 + i, b[i] * sb[i]);
  }
  return f;
}

}  // namespace la
