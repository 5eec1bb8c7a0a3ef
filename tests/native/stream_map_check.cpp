// Host-side check of the chain kernel's stream decode (stream_info in
// la_kernels.hpp, compiled here for the CPU): for every pass of the
// sequence-parallel forward, over many (sequences, length, segments)
// shapes, every stream's token rows, T-factor slots and state pointers lie
// inside the tensors they index, segments start on chunk boundaries, the
// state pass runs the streams the scan reads, and the output pass covers
// every token row exactly once.  Pointers are fake bases: only offsets are
// compared, nothing is dereferenced.  Prints "ok <n> streams" or the first
// failure and exits non-zero.
#include "la_kernels.hpp"

#include <cstdio>
#include <vector>

using namespace la;

namespace {

int fail(const char* what, int BH, int L, int P, int pass, int s) {
  std::printf("FAIL %s: BH=%d L=%d P=%d pass=%d stream=%d\n", what, BH, L, P, pass, s);
  return 1;
}

}  // namespace

int main() {
  long checked = 0;
  const int C = 64;
  for (int BH : {1, 2, 3, 5})
    for (int L : {C * 2, C * 2 + 1, C * 9 + 23, C * 10, 4096 + 40, 65536})
      for (int P = 2; P <= 64; ++P) {
        const int nc = (L + C - 1) / C;
        if (P > nc) break;
        const size_t dd = 64 * 64;
        float* xs = reinterpret_cast<float*>(size_t(1) << 20);
        const float* S0 = reinterpret_cast<const float*>(size_t(1) << 40);
        float* Sf = reinterpret_cast<float*>(size_t(1) << 41);
        for (int erase = 0; erase < 2; ++erase)
          for (int pass : {kPassState, kPassOut}) {
            const SeqMap sm{nullptr, BH, 1, L, C};
            const StreamMap m{sm, S0, Sf, pass, P, erase != 0, dd, xs,
                              xs + (size_t)BH * P * dd, xs + 2 * (size_t)BH * P * dd};
            const int n = m.per_seq();
            if (pass == kPassState && n != (P - 1) + (erase ? P - 2 : 0))
              return fail("stream count", BH, L, P, pass, -1);
            std::vector<int> cover((size_t)BH * L, 0);
            std::vector<int> x_seen((size_t)BH * P, 0), m_seen((size_t)BH * P, 0);
            for (int s = 0; s < BH * n; ++s) {
              const StreamInfo si = stream_info(m, s);
              const int bh = s / n;
              const size_t lo = (size_t)bh * L;
              if (si.len < 1 || si.row0 < lo || si.row0 + si.len > lo + L)
                return fail("token rows", BH, L, P, pass, s);
              if ((si.row0 - lo) % C) return fail("chunk alignment", BH, L, P, pass, s);
              const size_t nch = (si.len + C - 1) / C;
              if (si.slot0 != (size_t)bh * nc + (si.row0 - lo) / C ||
                  si.slot0 + nch > (size_t)(bh + 1) * nc)
                return fail("T slots", BH, L, P, pass, s);
              auto index = [&](const float* p, const float* base) -> long {
                const long off = p - base - (long)((size_t)bh * P * dd);
                return (off >= 0 && off % (long)dd == 0 && off / (long)dd < P) ? off / (long)dd
                                                                                 : -1;
              };
              if (pass == kPassOut) {
                if (si.eye || index(si.s0, m.sin) < 0) return fail("S_in", BH, L, P, pass, s);
                const bool last = si.row0 + si.len == lo + L;
                if (last != (si.sf != nullptr) || (si.sf && si.sf != Sf + (size_t)bh * dd))
                  return fail("S_final", BH, L, P, pass, s);
                for (int t = 0; t < si.len; ++t) cover[si.row0 + t]++;
              } else if (si.eye) {
                const long p = index(si.sf, m.ms);
                if (!erase || si.s0 || p < 1 || p > P - 2) return fail("M_p", BH, L, P, pass, s);
                m_seen[(size_t)bh * P + p]++;
              } else {
                const long p = index(si.sf, m.xs);
                if (p < 0 || p > P - 2) return fail("X_p", BH, L, P, pass, s);
                if ((p == 0) != (si.s0 != nullptr) || (si.s0 && si.s0 != S0 + (size_t)bh * dd))
                  return fail("segment start state", BH, L, P, pass, s);
                x_seen[(size_t)bh * P + p]++;
              }
              ++checked;
            }
            if (pass == kPassOut) {
              for (int c : cover)
                if (c != 1) return fail("token coverage", BH, L, P, pass, -1);
            } else {
              for (int bh = 0; bh < BH; ++bh)
                for (int p = 0; p < P; ++p) {
                  if (x_seen[(size_t)bh * P + p] != (p <= P - 2 ? 1 : 0))
                    return fail("X_p coverage", BH, L, P, pass, -1);
                  if (m_seen[(size_t)bh * P + p] != (erase && p >= 1 && p <= P - 2 ? 1 : 0))
                    return fail("M_p coverage", BH, L, P, pass, -1);
                }
            }
          }
      }
  std::printf("ok %ld streams\n", checked);
  return 0;
}
