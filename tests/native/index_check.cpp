// Host check of the chunk kernels' index maps (la_index.hpp): every transfer
// and read the kernels make through them is simulated on byte images of the
// LDS tiles, and each lane's result is compared with the element the
// kernels' layout assigns it.  Built by tests/test_sanitize_cpu.py under
// AddressSanitizer, so an offset outside a simulated array fails too.
//
// Hardware behaviour the simulation assumes (as the kernels do):
//  * global_load_lds_dwordx4: lane l of the instruction writes its 16
//    source bytes to LDS at the instruction's base + 16 l;
//  * ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives
//    element i % 4 of the 4-element runs read at the addresses of lanes
//    i / 4 + 4 j of its group, j = 0..3 (element j of its result);
//  * MFMA 16x16x32 operands: lane 16 g + n holds k = 8 g .. 8 g + 7 of row
//    (A) or column (B) n; an accumulator tile holds rows 4 g + i of column n.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "la_index.hpp"

namespace {

using la::kTileC;
constexpr int C = kTileC;
int g_fail = 0;
long g_checks = 0;

#define CHECK(cond, ...)                                 \
  do {                                                   \
    ++g_checks;                                          \
    if (!(cond)) {                                       \
      if (g_fail < 20) {                                 \
        std::fprintf(stderr, "%s:%d: ", __FILE__, __LINE__); \
        std::fprintf(stderr, __VA_ARGS__);               \
        std::fprintf(stderr, "\n");                      \
      }                                                  \
      ++g_fail;                                          \
    }                                                    \
  } while (0)

// Element id of a source tile: row r, column c (fits 16 bits for C x 128).
uint16_t id(int r, int c) { return (uint16_t)(r * 256 + c); }

// ds_read_b64_tr_b16 over one wave: addr[l] is lane l's byte address into
// img; returns the four elements each lane receives.
std::vector<uint16_t> read_tr(const std::vector<uint16_t>& img, const uint32_t* addr) {
  std::vector<uint16_t> out(64 * 4);
  for (int l = 0; l < 64; ++l) {
    const int grp = l / 16, i = l % 16;
    for (int j = 0; j < 4; ++j) {
      const uint32_t a = addr[16 * grp + i / 4 + 4 * j];
      CHECK(a % 8 == 0 && a / 2 + 4 <= img.size(), "read_tr address %u out of the image", a);
      out[4 * l + j] = a / 2 + 4 <= img.size() ? img[a / 2 + i % 4] : 0xffff;
    }
  }
  return out;
}

// Row of the B (or A) operand element j of lane group g when the operand is
// formed from an accumulator pair (tiles 2 kb, 2 kb + 1): 4 g + j, then 16 +
// 4 g + j - 4.
int kidx(int g, int j) { return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4); }

// A C x D tile moved by the DMA of one wave (C * 2 D / 1024 instructions)
// from a source of nrows valid rows; returns the LDS image.
template <int D>
std::vector<uint16_t> dma_tile(int nrows, std::vector<int>* writes) {
  std::vector<uint16_t> img(C * D, 0xffff);
  writes->assign(C * D / 8, 0);
  constexpr int NI = C * 2 * D / 1024;
  for (int m = 0; m < NI; ++m)
    for (int lane = 0; lane < 64; ++lane) {
      const uint32_t src = la::dma_src_off<D>(m, lane, nrows);
      CHECK(src % 16 == 0, "D=%d m=%d lane=%d: unaligned source %u", D, m, lane, src);
      CHECK(src + 16 <= (uint32_t)nrows * 2 * D, "D=%d nrows=%d m=%d lane=%d: source %u past the "
            "valid rows", D, nrows, m, lane, src);
      const uint32_t dst = 1024 * m + 16 * lane;
      CHECK(dst + 16 <= (uint32_t)C * 2 * D, "D=%d: LDS byte %u past the tile", D, dst);
      const int r = src / (2 * D), c0 = (src % (2 * D)) / 2;
      for (int e = 0; e < 8; ++e) img[dst / 2 + e] = id(r, c0 + e);
      ++(*writes)[dst / 16];
    }
  return img;
}

template <int D>
void check_tile() {
  constexpr int NKB = D / 32, NU = D / 8;
  // the swizzle permutes the units of every row
  for (int r = 0; r < C; ++r) {
    std::vector<int> seen(NU, 0);
    for (int u = 0; u < NU; ++u) {
      const int p = u ^ la::swz_key<D>(r);
      CHECK(p >= 0 && p < NU, "D=%d row %d unit %d: position %d", D, r, u, p);
      if (p >= 0 && p < NU) ++seen[p];
    }
    for (int p = 0; p < NU; ++p) CHECK(seen[p] == 1, "D=%d row %d: position %d used %d times", D, r, p, seen[p]);
  }
  std::vector<int> writes;
  for (int nrows : {1, 17, 63, C}) {
    const std::vector<uint16_t> img = dma_tile<D>(nrows, &writes);
    for (int u = 0; u < C * D / 8; ++u) CHECK(writes[u] == 1, "D=%d: LDS unit %d written %d times", D, u, writes[u]);
    // operand-row reads: logical unit 4 kb + g of row R is K[R][32 kb + 8 g ..]
    for (int R = 0; R < C; ++R)
      for (int kb = 0; kb < NKB; ++kb)
        for (int g = 0; g < 4; ++g) {
          const uint32_t off = la::unit_off<D>(R, 4 * kb + g);
          CHECK(off % 16 == 0 && off + 16 <= (uint32_t)C * 2 * D, "D=%d: unit_off(%d, %d) = %u", D, R,
                4 * kb + g, off);
          const int rs = R < nrows ? R : nrows - 1;
          for (int j = 0; j < 8; ++j)
            CHECK(img[off / 2 + j] == id(rs, 32 * kb + 8 * g + j),
                  "D=%d nrows=%d: row %d kb %d g %d element %d", D, nrows, R, kb, g, j);
        }
    if (nrows != C) continue;
    // transposed K^T operand of the state update: state tile tj = 2 kbs + h,
    // token block kb; lane (g, n) element j must be
    // K[32 kb + kidx(g, j)][dk_of_row(16 tj + n)]
    for (int kbs = 0; kbs < NKB; ++kbs)
      for (int h = 0; h < 2; ++h)
        for (int kb = 0; kb < 2; ++kb) {
          uint32_t a0[64], a1[64];
          for (int l = 0; l < 64; ++l) {
            a0[l] = la::tr_off<D>(l / 16, l % 16, kbs) + 8 * h + 64 * D * kb;
            a1[l] = a0[l] + 32 * D;          // 16 rows further
          }
          const std::vector<uint16_t> lo = read_tr(img, a0), hi = read_tr(img, a1);
          const int tj = 2 * kbs + h;
          for (int l = 0; l < 64; ++l) {
            const int g = l / 16, n = l % 16;
            for (int j = 0; j < 8; ++j) {
              const uint16_t got = j < 4 ? lo[4 * l + j] : hi[4 * l + j - 4];
              CHECK(got == id(32 * kb + kidx(g, j), la::dk_of_row(16 * tj + n)),
                    "D=%d K^T tile %d kb %d lane %d element %d", D, tj, kb, l, j);
            }
          }
        }
  }
}

// The V tile of one workgroup's 16 columns: plain C x 16 bf16, moved by two
// DMA instructions (lane l: row 32 m + l / 2, columns 8 (l % 2) ..), read as
// the accumulator layout (v_acc_at) and as a transposed operand
// (frag_col_tr_v).
void check_v_tile() {
  for (int nr : {1, 40, C}) {
    std::vector<uint16_t> img(C * 16, 0xffff);
    std::vector<int> w(C * 16 / 8, 0);
    for (int m = 0; m < 2; ++m)
      for (int l = 0; l < 64; ++l) {
        const int r = 32 * m + l / 2, rs = r < nr - 1 ? r : nr - 1;
        const uint32_t dst = 1024 * m + 16 * l;
        CHECK(dst + 16 <= (uint32_t)C * 32, "V tile: LDS byte %u", dst);
        for (int e = 0; e < 8; ++e) img[dst / 2 + e] = id(rs, 8 * (l % 2) + e);
        ++w[dst / 16];
      }
    for (int u = 0; u < C * 2; ++u) CHECK(w[u] == 1, "V tile unit %d written %d times", u, w[u]);
    auto vrow = [&](int r) { return r < nr ? r : nr - 1; };
    for (int ti = 0; ti < 4; ++ti) {
      uint32_t a[64];
      for (int l = 0; l < 64; ++l) a[l] = la::vacc_off(l / 16, l % 16) + 512 * ti;
      const std::vector<uint16_t> v = read_tr(img, a);
      for (int l = 0; l < 64; ++l)
        for (int i = 0; i < 4; ++i)
          CHECK(v[4 * l + i] == id(vrow(16 * ti + 4 * (l / 16) + i), l % 16),
                "V accumulator layout: tile %d lane %d row %d", ti, l, i);
    }
    for (int kb = 0; kb < 2; ++kb) {
      uint32_t a0[64], a1[64];
      for (int l = 0; l < 64; ++l) {
        a0[l] = la::col_tr_off(32 * kb, l / 16, l % 16);
        a1[l] = a0[l] + 16 * 16 * 2;
      }
      const std::vector<uint16_t> lo = read_tr(img, a0), hi = read_tr(img, a1);
      for (int l = 0; l < 64; ++l)
        for (int j = 0; j < 8; ++j) {
          const uint16_t got = j < 4 ? lo[4 * l + j] : hi[4 * l + j - 4];
          CHECK(got == id(vrow(32 * kb + kidx(l / 16, j)), l % 16), "V^T operand kb %d lane %d element %d",
                kb, l, j);
        }
    }
  }
}

void check_small_maps() {
  // state rows: a permutation of dk, of the documented form
  for (int D : {64, 128}) {
    std::vector<int> seen(D, 0);
    for (int p = 0; p < D; ++p) {
      const int dk = la::dk_of_row(p);
      CHECK(dk >= 0 && dk < D, "dk_of_row(%d) = %d", p, dk);
      if (dk >= 0 && dk < D) ++seen[dk];
      const int kb = p / 32, h = (p / 16) % 2, g = (p / 4) % 4, j = p % 4;
      CHECK(dk == 32 * kb + 8 * g + 4 * h + j, "dk_of_row(%d) = %d", p, dk);
    }
    for (int d = 0; d < D; ++d) CHECK(seen[d] == 1, "dk %d held by %d rows", d, seen[d]);
  }
  // T fragments: (ti, kb <= ti / 2) onto 0..kTFrags-1
  std::vector<int> tf(la::kTFrags, 0);
  for (int ti = 0; ti < 4; ++ti)
    for (int kb = 0; kb <= ti / 2; ++kb) {
      const int f = la::tfi(ti, kb);
      CHECK(f >= 0 && f < la::kTFrags, "tfi(%d, %d) = %d", ti, kb, f);
      if (f >= 0 && f < la::kTFrags) ++tf[f];
    }
  for (int f = 0; f < la::kTFrags; ++f) CHECK(tf[f] == 1, "T fragment %d used %d times", f, tf[f]);
  // lower blocks of a 4 x 4 block matrix onto 0..9
  std::vector<int> bb(10, 0);
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j <= i; ++j) {
      const int b = la::bid(i, j);
      CHECK(b >= 0 && b < 10, "bid(%d, %d) = %d", i, j, b);
      if (b >= 0 && b < 10) ++bb[b];
    }
  for (int b = 0; b < 10; ++b) CHECK(bb[b] == 1, "block slot %d used %d times", b, bb[b]);
}

// Bank-conflict freedom of the operand-row reads under gfx950's rule for
// 16-byte LDS reads (64 four-byte banks; the 16 lanes of one cycle are the
// lane quads q = l / 4 of a half-wave with equal parity of q's three low
// bits, tests/lds_probe): no two lanes of one cycle may hit the same
// 16-byte bank unit at different addresses.
int b128_cycle(int l) { return 2 * ((l >> 5) & 1) + (((l >> 2) ^ (l >> 3) ^ (l >> 4)) & 1); }

template <int D>
void check_row_read_banks() {
  for (int t = 0; t < C / 16; ++t)
    for (int kb = 0; kb < D / 32; ++kb) {
      uint32_t addr[64];
      for (int l = 0; l < 64; ++l) addr[l] = la::unit_off<D>(16 * t + l % 16, 4 * kb + l / 16);
      for (int a = 0; a < 64; ++a)
        for (int b = a + 1; b < 64; ++b)
          if (b128_cycle(a) == b128_cycle(b) && addr[a] != addr[b])
            CHECK(((addr[a] >> 4) & 15) != ((addr[b] >> 4) & 15),
                  "D=%d: row reads of lanes %d and %d share bank unit %u (t %d, kb %d)", D, a, b,
                  (addr[a] >> 4) & 15, t, kb);
    }
}

}  // namespace

int main() {
  check_tile<64>();
  check_tile<128>();
  check_v_tile();
  check_small_maps();
  check_row_read_banks<64>();
  check_row_read_banks<128>();
  std::printf("%ld checks, %d failures\n", g_checks, g_fail);
  return g_fail == 0 ? 0 : 1;
}
