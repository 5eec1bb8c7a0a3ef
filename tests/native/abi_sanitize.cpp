// Argument validation of every C-ABI entry point under AddressSanitizer and
// UndefinedBehaviorSanitizer, on the host alone.
//
// Built by tests/test_sanitize_cpu.py from the library sources compiled for
// the host only (no device code: every call here must return before its
// first HIP call), with -fsanitize=address,undefined and
// -fno-sanitize-recover.  Each call passes NULL pointers, bad or extreme
// sizes (zero, negative, INT_MAX, products past 2^31 and 2^63), overlapping
// fake pointers that are never dereferenced, or too small and misaligned
// workspaces, and must return the expected error code with a message in
// la_last_error().  The size queries are swept over a grid that includes
// sizes whose byte counts overflow 32 and 64 bits.  A memory error, an
// integer overflow or a wrong code ends the program with a non-zero status.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "la.h"

namespace {

int g_fail = 0;
int g_calls = 0;

void expect(int got, int want, const char* what, int line) {
  ++g_calls;
  const char* msg = la_last_error();
  if (got != want) {
    std::fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", line, what, got, want,
                 msg ? msg : "(null)");
    ++g_fail;
    return;
  }
  if (want != LA_OK && (!msg || !msg[0] || std::strlen(msg) > 4096)) {
    std::fprintf(stderr, "line %d: %s: no message for code %d\n", line, what, got);
    ++g_fail;
  }
}

// any code but OK (the size sweeps, where several checks may fire first)
void expect_err(int got, const char* what, int line) {
  ++g_calls;
  if (got == LA_OK) {
    std::fprintf(stderr, "line %d: %s accepted invalid arguments\n", line, what);
    ++g_fail;
  }
}

#define EXPECT(call, code) expect((call), (code), #call, __LINE__)
#define EXPECT_ERR(call) expect_err((call), #call, __LINE__)

// Fake, well separated, 1 MiB-aligned pointers; never dereferenced.
constexpr uintptr_t P = uintptr_t(1) << 20;
void* fp(int i) { return reinterpret_cast<void*>(P * uintptr_t(i + 1)); }
float* ff(int i) { return reinterpret_cast<float*>(fp(i)); }
void* at(uintptr_t a) { return reinterpret_cast<void*>(a); }

const int kBadSizes[] = {0, -1, INT_MIN, INT_MAX};
const int kModes[] = {LA_MODE_LINEAR, LA_MODE_DELTA, LA_MODE_GATED_DELTA, LA_MODE_GATED_LINEAR};

struct Fwd {
  const void *q = fp(0), *k = fp(1), *v = fp(2);
  const float *la = ff(3), *be = ff(4), *s0 = ff(5);
  void* out = fp(6);
  float* sf = ff(7);
  int B = 1, H = 1, L = 64, dk = 64, dv = 64, C = 64, mode = 2, dtype = 1;
  void* ws = fp(8);
  size_t wsb = P;
  int call() const {
    return la_chunk_fwd(q, k, v, la, be, s0, out, sf, B, H, L, dk, dv, C, mode, dtype, ws, wsb,
                        nullptr);
  }
  int noalloc() const {
    return la_chunk_fwd_noalloc(q, k, v, la, be, s0, out, sf, B, H, L, dk, dv, C, mode, dtype,
                                nullptr);
  }
  int segmented(int P_) const {
    return la_chunk_fwd_segmented(q, k, v, la, be, s0, out, sf, B, H, L, dk, dv, C, mode, dtype,
                                  P_, ws, wsb, nullptr);
  }
  int fused(const la_fused_opts_t* o) const {
    return la_chunk_fwd_fused(q, k, v, la, be, s0, out, sf, B, H, L, dk, dv, C, mode, dtype, o,
                              ws, wsb, nullptr);
  }
};

void check_chunk_fwd() {
  {
    Fwd f; f.q = nullptr; EXPECT(f.call(), LA_ERR_NULL);
  }
  {
    Fwd f; f.out = nullptr; EXPECT(f.call(), LA_ERR_NULL);
  }
  {
    Fwd f; f.la = nullptr; EXPECT(f.call(), LA_ERR_NULL);
  }
  {
    Fwd f; f.be = nullptr; f.mode = LA_MODE_DELTA; EXPECT(f.call(), LA_ERR_NULL);
  }
  for (int bad : kBadSizes) {
    Fwd f;
    f.B = bad; EXPECT_ERR(f.call());
    f.B = 1; f.H = bad; EXPECT_ERR(f.call());
    f.H = 1; f.L = bad; EXPECT_ERR(f.call());
    f.L = 64; f.C = bad; EXPECT_ERR(f.call());
    f.C = 64; f.dk = bad; EXPECT_ERR(f.call());
    f.dk = 64; f.mode = bad; EXPECT_ERR(f.call());
    f.mode = 2; f.dtype = bad; EXPECT_ERR(f.call());
    EXPECT_ERR(f.noalloc());
  }
  {
    // sizes whose element counts pass 2^31 and 2^63
    Fwd f; f.B = 1 << 16; f.H = 1 << 16; f.L = 1 << 20; EXPECT_ERR(f.call());
    f.B = INT_MAX; f.H = INT_MAX; f.L = INT_MAX; EXPECT_ERR(f.call());
    EXPECT_ERR(f.noalloc());
  }
  {
    Fwd f; f.dk = 96; f.dv = 96; EXPECT(f.call(), LA_ERR_UNSUPPORTED);
  }
  {
    Fwd f; f.dk = 64; f.dv = 128; EXPECT(f.call(), LA_ERR_UNSUPPORTED);
  }
  {
    // out starting inside q (q spans 64 x 64 bf16 = 8 KiB)
    Fwd f; f.out = at(P + 128); EXPECT(f.call(), LA_ERR_ALIAS);
  }
  {
    // S_final partly over S0
    Fwd f; f.sf = reinterpret_cast<float*>(at(6 * P + 4)); EXPECT(f.call(), LA_ERR_ALIAS);
  }
  {
    // the workspace over k
    Fwd f; f.ws = at(2 * P - 1024); EXPECT(f.call(), LA_ERR_ALIAS);
  }
  {
    Fwd f; f.wsb = 1; EXPECT(f.call(), LA_ERR_WORKSPACE);
  }
  {
    Fwd f; f.ws = at(9 * P + 8); EXPECT(f.call(), LA_ERR_WORKSPACE);
  }
  {
    Fwd f; f.ws = nullptr; f.wsb = 0; EXPECT(f.call(), LA_ERR_WORKSPACE);
  }
  for (int P_ : {-1, 0, INT_MAX}) {
    Fwd f; EXPECT_ERR(f.segmented(P_));
  }
  {
    Fwd f; f.q = nullptr; EXPECT(f.segmented(2), LA_ERR_NULL);
  }
  {
    // fused: unknown flags, a non-positive gate scale, a non-positive norm eps
    Fwd f;
    la_fused_opts_t o{};
    o.flags = 1 << 10; EXPECT_ERR(f.fused(&o));
    o.flags = LA_PRO_GATES; o.gate_scale = 0.f; EXPECT_ERR(f.fused(&o));
    o.flags = LA_EPI_OUT_NORM; o.norm_eps = -1.f; EXPECT_ERR(f.fused(&o));
    o.flags = LA_EPI_DSKIP; o.dskip = nullptr; EXPECT_ERR(f.fused(&o));
    f.q = nullptr; o.flags = 0; EXPECT(f.fused(&o), LA_ERR_NULL);
  }
}

void check_varlen() {
  auto call = [](const int* cu, int N, int H, int T, int mode, void* out, void* ws, size_t wsb) {
    return la_chunk_fwd_varlen(fp(0), fp(1), fp(2), ff(3), ff(4), ff(5), out, ff(7), cu, N, H, T,
                               64, 64, 64, mode, 1, ws, wsb, nullptr);
  };
  const int* cu = reinterpret_cast<const int*>(fp(9));
  EXPECT(call(nullptr, 2, 1, 64, 2, fp(6), fp(8), P), LA_ERR_NULL);
  for (int bad : kBadSizes) {
    EXPECT_ERR(call(cu, bad, 1, 64, 2, fp(6), fp(8), P));
    EXPECT_ERR(call(cu, 2, bad, 64, 2, fp(6), fp(8), P));
    EXPECT_ERR(call(cu, 2, 1, bad == 0 ? -1 : bad, 2, fp(6), fp(8), P));
  }
  EXPECT_ERR(call(cu, INT_MAX, INT_MAX, INT_MAX, 2, fp(6), fp(8), P));
  EXPECT(call(cu, 2, 1, 64, 2, at(10 * P - 64), fp(8), P), LA_ERR_ALIAS);
  EXPECT(call(cu, 2, 1, 64, 2, fp(6), at(10 * P - 1024), P), LA_ERR_ALIAS);
  EXPECT(call(cu, 2, 1, 64, 2, fp(6), fp(8), 1), LA_ERR_WORKSPACE);
}

void check_noncausal() {
  auto call = [](int B, int H, int L, int dk, int dtype, void* out, size_t wsb) {
    return la_noncausal_fwd(fp(0), fp(1), fp(2), ff(5), out, ff(7), B, H, L, dk, dk, dtype, fp(8),
                            wsb, nullptr);
  };
  EXPECT(call(1, 1, 64, 64, 1, nullptr, P), LA_ERR_NULL);
  for (int bad : kBadSizes) {
    EXPECT_ERR(call(bad, 1, 64, 64, 1, fp(6), P));
    EXPECT_ERR(call(1, bad, 64, 64, 1, fp(6), P));
    EXPECT_ERR(call(1, 1, bad, 64, 1, fp(6), P));
    EXPECT_ERR(call(1, 1, 64, bad, 1, fp(6), P));
  }
  EXPECT_ERR(call(INT_MAX, INT_MAX, INT_MAX, 64, 1, fp(6), P));
  EXPECT(call(1, 1, 64, 64, 1, at(P + 64), P), LA_ERR_ALIAS);
  EXPECT(call(1, 1, 64, 64, 1, fp(6), 1), LA_ERR_WORKSPACE);
}

struct Bwd {
  const void *q = fp(0), *k = fp(1), *v = fp(2);
  const float *la = ff(3), *be = ff(4), *s0 = ff(5);
  const void* dout = fp(6);
  const float* dsf = ff(7);
  float *dq = ff(10), *dk_ = ff(11), *dv_ = ff(12), *dla = ff(13), *dbe = ff(14), *ds0 = ff(15);
  int B = 1, H = 1, L = 64, dk = 64, dv = 64, C = 64, mode = 2, dtype = 1;
  void* ws = fp(16);
  size_t wsb = 64 * P;
  int call() const {
    return la_chunk_bwd(q, k, v, la, be, s0, dout, dsf, dq, dk_, dv_, dla, dbe, ds0, B, H, L, dk,
                        dv, C, mode, dtype, ws, wsb, nullptr);
  }
  int varlen(const int* cu, int N) const {
    return la_chunk_bwd_varlen(q, k, v, la, be, s0, dout, dsf, cu, dq, dk_, dv_, dla, dbe, ds0, N,
                               H, L, dk, dv, C, mode, dtype, ws, wsb, nullptr);
  }
  int fused(const la_fused_opts_t* o) const {
    return la_chunk_bwd_fused(q, k, v, la, be, s0, dout, dsf, dq, dk_, dv_, dla, dbe, ds0, B, H,
                              L, dk, dv, C, mode, dtype, o, ws, wsb, nullptr);
  }
};

void check_bwd() {
  {
    Bwd b; b.q = nullptr; EXPECT(b.call(), LA_ERR_NULL);
  }
  {
    Bwd b; b.dout = nullptr; EXPECT(b.call(), LA_ERR_NULL);
  }
  {
    Bwd b; b.dq = nullptr; EXPECT(b.call(), LA_ERR_NULL);
  }
  for (int bad : kBadSizes) {
    Bwd b;
    b.B = bad; EXPECT_ERR(b.call());
    b.B = 1; b.L = bad; EXPECT_ERR(b.call());
    b.L = 64; b.mode = bad; EXPECT_ERR(b.call());
  }
  {
    Bwd b; b.B = INT_MAX; b.H = INT_MAX; b.L = INT_MAX; EXPECT_ERR(b.call());
  }
  {
    // grad_q over v
    Bwd b; b.dq = reinterpret_cast<float*>(at(3 * P - 64)); EXPECT(b.call(), LA_ERR_ALIAS);
  }
  {
    // two gradient outputs overlapping
    Bwd b; b.dk_ = reinterpret_cast<float*>(at(11 * P + 64)); EXPECT(b.call(), LA_ERR_ALIAS);
  }
  {
    Bwd b; b.wsb = 1; EXPECT(b.call(), LA_ERR_WORKSPACE);
  }
  {
    Bwd b;
    EXPECT(b.varlen(nullptr, 2), LA_ERR_NULL);
    EXPECT_ERR(b.varlen(reinterpret_cast<const int*>(fp(20)), 0));
    EXPECT_ERR(b.varlen(reinterpret_cast<const int*>(fp(20)), INT_MAX));
  }
  {
    Bwd b;
    la_fused_opts_t o{};
    o.flags = LA_EPI_OUT_NORM; o.norm_eps = 1e-6f; EXPECT_ERR(b.fused(&o));  // not supported
    o.flags = LA_PRO_GATES; o.gate_scale = -1.f; EXPECT_ERR(b.fused(&o));
    // v inside the prologue region of the workspace
    o.flags = LA_PRO_GATES | LA_PRO_QK_L2NORM; o.gate_scale = 1.f;
    b.v = at(17 * P + 256); EXPECT(b.fused(&o), LA_ERR_ALIAS);
  }
}

void check_decode() {
  auto call = [](const void* q, int B, int H, int dk, int dv, int mode, int dtype, void* out) {
    return la_decode_step(q, fp(1), fp(2), ff(3), ff(4), ff(5), out, B, H, dk, dv, mode, dtype,
                          nullptr);
  };
  EXPECT(call(nullptr, 1, 1, 64, 64, 2, 1, fp(6)), LA_ERR_NULL);
  EXPECT(call(fp(0), 1, 1, 64, 64, 2, 1, nullptr), LA_ERR_NULL);
  for (int bad : kBadSizes) {
    EXPECT_ERR(call(fp(0), bad, 1, 64, 64, 2, 1, fp(6)));
    EXPECT_ERR(call(fp(0), 1, bad, 64, 64, 2, 1, fp(6)));
    EXPECT_ERR(call(fp(0), 1, 1, bad, 64, 2, 1, fp(6)));
    EXPECT_ERR(call(fp(0), 1, 1, 64, 64, bad, 1, fp(6)));
    EXPECT_ERR(call(fp(0), 1, 1, 64, 64, 2, bad, fp(6)));
  }
  EXPECT_ERR(call(fp(0), INT_MAX, INT_MAX, 64, 64, 2, 1, fp(6)));
  EXPECT(call(fp(0), 1, 1, 64, 64, 2, 1, at(P + 32)), LA_ERR_ALIAS);
  la_fused_opts_t o{};
  o.flags = 1 << 12;
  EXPECT_ERR(la_decode_step_fused(fp(0), fp(1), fp(2), ff(3), ff(4), ff(5), fp(6), 1, 1, 64, 64,
                                  2, 1, &o, nullptr));
}

// The size queries over a grid of sizes, modes and dtypes, extreme ones
// included: each returns OK with a size, or an error; none may overflow.
void sweep_sizes() {
  const int sizes[] = {1, 63, 64, 65, 4096, 65536, 1 << 24, INT_MAX};
  const int ds[] = {64, 128};
  for (int mode : kModes)
    for (int dtype : {0, 1, 2})
      for (int d : ds)
        for (int B : sizes)
          for (int L : sizes) {
            size_t n = 0;
            int segs = 0;
            la_chunk_workspace_bytes(B, 32, L, d, d, 64, mode, dtype, &n);
            la_chunk_segmented_workspace_bytes(B, 32, L, d, d, 64, mode, dtype, 8, &n);
            la_chunk_segments(B, 32, L, d, d, 64, mode, dtype, &segs);
            la_chunk_varlen_workspace_bytes(B, 32, L, d, d, 64, mode, dtype, &n);
            la_noncausal_workspace_bytes(B, 32, L, d, d, dtype, &n);
            la_chunk_bwd_workspace_bytes(B, 32, L, d, d, 64, mode, dtype, &n);
            la_chunk_bwd_varlen_workspace_bytes(B, 32, L, d, d, 64, mode, dtype, &n);
            la_fused_opts_t o{};
            o.flags = LA_PRO_GATES | LA_PRO_QK_L2NORM;
            o.gate_scale = 1.f;
            la_chunk_fused_workspace_bytes(B, 32, L, d, d, 64, mode, dtype, &o, &n);
            la_chunk_bwd_fused_workspace_bytes(B, 32, L, d, d, 64, mode, dtype, &o, &n);
            g_calls += 9;
          }
  size_t n = 0;
  EXPECT(la_chunk_workspace_bytes(1, 1, 64, 64, 64, 64, 2, 1, nullptr), LA_ERR_NULL);
  EXPECT(la_chunk_workspace_bytes(1, 1, 64, 64, 64, 64, 2, 1, &n), LA_OK);
  EXPECT(la_chunk_workspace_bytes(1, 1, 64, 96, 96, 64, 2, 1, &n), LA_ERR_UNSUPPORTED);
  // 2^31 chunk-heads of 6 KiB overflow no size_t, but pass the grid limit
  EXPECT_ERR(la_chunk_workspace_bytes(INT_MAX, INT_MAX, INT_MAX, 128, 128, 64, 2, 1, &n));
  // the length limit: LA_MAX_TOKENS is taken, one more token is not
  int segs = 0;
  EXPECT(la_chunk_segments(1, 1, LA_MAX_TOKENS, 128, 128, 64, 2, 1, &segs), LA_OK);
  EXPECT(la_chunk_segments(1, 1, LA_MAX_TOKENS + 1, 128, 128, 64, 2, 1, &segs), LA_ERR_SHAPE);
  EXPECT(la_chunk_workspace_bytes(1, 1, LA_MAX_TOKENS, 128, 128, 64, 2, 1, &n), LA_OK);
  EXPECT(la_chunk_varlen_workspace_bytes(4, 1, LA_MAX_TOKENS + 1, 128, 128, 64, 2, 1, &n),
         LA_ERR_SHAPE);
  EXPECT(la_chunk_bwd_workspace_bytes(1, 1, LA_MAX_TOKENS + 1, 128, 128, 64, 2, 1, &n),
         LA_ERR_SHAPE);
}

void check_misc() {
  const char* v = la_version();
  if (!v || std::strncmp(v, "lachunk ", 8) != 0) {
    std::fprintf(stderr, "la_version: unexpected '%s'\n", v ? v : "(null)");
    ++g_fail;
  }
  // no recording in progress: nothing to report, no HIP call
  int count = -1;
  EXPECT(la_profile_end(nullptr, 0, nullptr), LA_ERR_NULL);
  EXPECT(la_profile_end(nullptr, 0, &count), LA_OK);
  if (count != 0) {
    std::fprintf(stderr, "la_profile_end: %d records without la_profile_begin\n", count);
    ++g_fail;
  }
}

}  // namespace

int main() {
  check_chunk_fwd();
  check_varlen();
  check_noncausal();
  check_bwd();
  check_decode();
  sweep_sizes();
  check_misc();
  std::printf("%d calls, %d failures\n", g_calls, g_fail);
  return g_fail == 0 ? 0 : 1;
}
