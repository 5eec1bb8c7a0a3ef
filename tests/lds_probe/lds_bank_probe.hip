// LDS bank-conflict probe for gfx950: one kernel dispatch per address
// pattern, each wave repeating four LDS reads whose per-lane addresses come
// from a host table.  Run it under rocprofv3 with the counters
// SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE and SQ_INSTS_LDS; the ratio
// IDX_ACTIVE / INSTS_LDS is the LDS cycles per instruction (about 4 for a
// conflict-free 16-byte read of 64 lanes, 2 for an 8-byte one) and
// BANK_CONFLICT / INSTS_LDS the cycles lost to conflicts.  The dispatches
// come in the order the patterns are printed (a table copy precedes each).
//
//   hipcc --offload-arch=gfx950 -O3 -std=c++17 -I chunkwise_gated_delta_la_amd/csrc \
//         -o /tmp/lds_bank_probe tests/lds_probe/lds_bank_probe.hip
//   cd /tmp && rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS \
//         GRBM_GUI_ACTIVE --output-format csv -d <out> -o p -- /tmp/lds_bank_probe
//
// The patterns establish the rule the chunk kernels' tile key is built for
// (la_index.hpp): 64 four-byte banks; a 16-byte read serves 16 lanes per
// cycle, two lane quads from each of two neighbouring 16-lane groups (the
// quads q = lane / 4 of a half-wave with equal parity of q's three low
// bits); an 8-byte transposed read serves 32 consecutive lanes per cycle.
#include <hip/hip_runtime.h>
#include <cstdint>
#include <cstdio>
#include <functional>
#include <string>
#include <vector>

#include "la_index.hpp"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
constexpr int kLds = 65536;
constexpr int kIters = 512;

// W = 16: ds_read_b128, W = 1: ds_read_b64_tr_b16
template <int W>
__global__ __launch_bounds__(256) void probe(const uint32_t* tab, uint32_t* out, uint32_t zero) {
  __shared__ __attribute__((aligned(16))) uint8_t buf[kLds];
  for (int i = threadIdx.x; i < kLds / 4; i += 256) reinterpret_cast<uint32_t*>(buf)[i] = i;
  const int lane = threadIdx.x % 64;
  uint32_t a[4];
  for (int j = 0; j < 4; ++j) a[j] = tab[j * 64 + lane];
  __syncthreads();
  u32x4 acc = u32x4{0u, 0u, 0u, 0u};
  // the addresses depend on the iteration through `zero` (0 at run time),
  // so the compiler can neither hoist the reads nor fold the sums
  for (int it = 0; it < kIters; ++it) {
    const uint32_t z = (uint32_t)it * zero;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (W == 16) {
        typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
        acc += *(const volatile lds_u32x4*)(buf + (a[j] ^ z));
      } else {
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(buf + (a[j] ^ z)));
        acc.x += (uint32_t)(uint16_t)x[0] | ((uint32_t)(uint16_t)x[1] << 16);
        acc.y += (uint32_t)(uint16_t)x[2] | ((uint32_t)(uint16_t)x[3] << 16);
      }
    }
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

struct Pattern {
  std::string name;
  int width;                                   // 16 or 1 (transposed)
  std::function<uint32_t(int lane, int j)> addr;
};

// the key the chunk kernels used before (16 consecutive lanes per cycle)
int old_key(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

}  // namespace

int main() {
  auto G = [](int l) { return l / 16; };
  auto N = [](int l) { return l % 16; };
  auto mpat = [&](int l, int j, int m1, int m2) {
    const int g = G(l), n = N(l);
    return (uint32_t)(256 * (n + 16 * g) + 16 * (n ^ (m1 * (g & 1)) ^ (m2 * (g >> 1)) ^ ((4 * j) % 16)));
  };
  std::vector<Pattern> pats = {
      {"b128 linear (64 lanes, 1 KiB)", 16, [](int l, int j) { return (uint32_t)(16 * l + 1024 * j); }},
      {"b128 row n, unit n ^ g", 16,
       [&](int l, int j) { return (uint32_t)(256 * N(l) + 16 * (N(l) ^ G(l) ^ (4 * j))); }},
      {"b128 row n, unit n ^ (g << 2)", 16,
       [&](int l, int j) { return (uint32_t)(256 * N(l) + 16 * (N(l) ^ (G(l) << 2) ^ j)); }},
      {"b128 row n, unit (n + g) % 16", 16,
       [&](int l, int j) { return (uint32_t)(256 * N(l) + 16 * ((N(l) + G(l) + j) % 16)); }},
      {"b128 128-byte rows n, unit (n + g) % 8", 16,
       [&](int l, int j) { return (uint32_t)(128 * N(l) + 16 * ((N(l) + G(l)) % 8) + 4096 * j); }},
      // unit n ^ (m1 (g & 1)) ^ (m2 (g >> 1)) on rows n + 16 g: patterns that
      // tell the candidate lane partitions apart
      {"b128 unit n ^ 4 (g & 1) ^ 5 (g >> 1)", 16, [&](int l, int j) { return mpat(l, j, 4, 5); }},
      {"b128 unit n ^ 15 (g & 1) ^ 4 (g >> 1)", 16, [&](int l, int j) { return mpat(l, j, 15, 4); }},
      {"b128 unit n ^ 8 (g & 1) ^ 15 (g >> 1)", 16, [&](int l, int j) { return mpat(l, j, 8, 15); }},
      {"b128 unit n ^ 7 (g & 1) ^ 15 (g >> 1)", 16, [&](int l, int j) { return mpat(l, j, 7, 15); }},
      {"b128 unit n ^ 5 (g & 1) ^ 2 (g >> 1)", 16, [&](int l, int j) { return mpat(l, j, 5, 2); }},
      {"b128 unit n ^ 11 (g >> 1)", 16, [&](int l, int j) { return mpat(l, j, 0, 11); }},
      {"b128 unit n ^ 3 (g & 1) ^ 9 (g >> 1)", 16, [&](int l, int j) { return mpat(l, j, 3, 9); }},
      {"b128 operand rows, old key", 16,
       [&](int l, int j) { const int r = 16 * j + N(l); return (uint32_t)(256 * r + 16 * ((4 * j + G(l)) ^ old_key(r))); }},
      {"b128 operand rows, current key (D = 128)", 16,
       [&](int l, int j) { const int r = 16 * j + N(l); return la::unit_off<128>(r, 4 * j + G(l)); }},
      {"b128 operand rows, current key (D = 64)", 16,
       [&](int l, int j) { const int r = 16 * j + N(l); return la::unit_off<64>(r, 4 * (j & 1) + G(l)); }},
      {"tr K^T reads, current key (D = 128), 8-byte half j & 1", 1,
       [&](int l, int j) { return la::tr_off<128>(G(l), N(l), j) + (uint32_t)(8 * (j & 1)); }},
      {"tr K^T reads, current key (D = 128), lower halves", 1,
       [&](int l, int j) { return la::tr_off<128>(G(l), N(l), j); }},
      {"tr K^T reads, current key, rows + 16 j", 1,
       [&](int l, int j) { return la::tr_off<128>(G(l), N(l), j) + (uint32_t)(16 * 256 * j); }},
      {"tr K^T reads, old key, lower halves", 1,
       [&](int l, int j) {
         const int r = 4 * G(l) + (N(l) >> 2);
         return (uint32_t)(256 * r + 16 * ((4 * j + (N(l) & 3)) ^ old_key(r)));
       }},
      {"tr K^T reads, odd groups in the other 8-byte half", 1,
       [&](int l, int j) { return la::tr_off<128>(G(l), N(l), j) + (uint32_t)(8 * (G(l) & 1)); }},
      {"tr reads of a 16-column tile (32-byte rows)", 1,
       [&](int l, int j) { return la::col_tr_off(16 * j, G(l), N(l)); }},
  };
  uint32_t *dtab = nullptr, *dout = nullptr;
  if (hipMalloc(&dtab, 4 * 64 * 4) != hipSuccess || hipMalloc(&dout, 512 * 256 * 4) != hipSuccess) {
    std::fprintf(stderr, "hipMalloc failed\n");
    return 1;
  }
  // 64 workgroups: one per compute unit; 512: two per unit (64 KiB of LDS
  // each), so that two workgroups' waves share each unit's LDS
  for (int grid : {64, 512})
  for (size_t p = 0; p < pats.size(); ++p) {
    std::vector<uint32_t> t(4 * 64);
    const uint32_t align = pats[p].width == 16 ? 16 : 8;
    for (int j = 0; j < 4; ++j)
      for (int l = 0; l < 64; ++l) {
        const uint32_t a = pats[p].addr(l, j);
        if (a % align != 0 || a + 16 > (uint32_t)kLds) {
          std::fprintf(stderr, "pattern %zu: address %u out of range\n", p, a);
          return 2;
        }
        t[j * 64 + l] = a;
      }
    if (hipMemcpy(dtab, t.data(), t.size() * 4, hipMemcpyHostToDevice) != hipSuccess) return 1;
    std::printf("pattern %zu: %s (%d workgroups)\n", p, pats[p].name.c_str(), grid);
    std::fflush(stdout);
    if (pats[p].width == 16) probe<16><<<grid, 256>>>(dtab, dout, 0u);
    else probe<1><<<grid, 256>>>(dtab, dout, 0u);
    if (hipDeviceSynchronize() != hipSuccess) return 1;
  }
  (void)hipFree(dtab);
  (void)hipFree(dout);
  return 0;
}
