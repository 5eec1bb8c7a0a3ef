// C-ABI host layer of liblachunk: argument validation, dispatch to the
// gfx950 kernels, caller-provided workspace.  See include/la.h for the
// contract of every entry point.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>
#include <vector>
#include <map>
#include <cstring>
#include <algorithm>

#include "la.h"
#include "la_kernels.hpp"
#include "la_bwd.hpp"

// Scratch of la_chunk_fwd_noalloc: one array per GPU, in the library's code
// object.  Host code never uses this name as an address (on the host it is
// only a handle for the symbol lookup): the device address comes from
// hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[LA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int fail_hip(const char* what, hipError_t e) {
  return fail(LA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Half-open byte range of a tensor argument; empty when ptr is NULL.
struct Range {
  uintptr_t lo = 0, hi = 0;
  Range() = default;
  Range(const void* p, size_t bytes)
      : lo(reinterpret_cast<uintptr_t>(p)), hi(p ? lo + bytes : lo) {}
  bool empty() const { return lo == hi; }
  bool overlaps(const Range& o) const {
    return !empty() && !o.empty() && lo < o.hi && o.lo < hi;
  }
};

bool mul_ok(size_t a, size_t b, size_t* out) {
  if (a != 0 && b > SIZE_MAX / a) return false;
  *out = a * b;
  return true;
}

// Element count of a product of positive sizes, or false on overflow.
bool count(std::initializer_list<long> dims, size_t* out) {
  size_t n = 1;
  for (long d : dims)
    if (!mul_ok(n, (size_t)d, &n)) return false;
  *out = n;
  return true;
}

int check_mode_dtype(int mode, int dtype) {
  if (mode < LA_MODE_LINEAR || mode > LA_MODE_GATED_LINEAR)
    return fail(LA_ERR_UNSUPPORTED, "mode must be LA_MODE_LINEAR, LA_MODE_DELTA, "
                                    "LA_MODE_GATED_DELTA or LA_MODE_GATED_LINEAR, got " +
                                        std::to_string(mode));
  if (dtype != LA_DTYPE_F32 && dtype != LA_DTYPE_BF16 && dtype != LA_DTYPE_BF16_F32OUT)
    return fail(LA_ERR_UNSUPPORTED, "dtype must be LA_DTYPE_F32, LA_DTYPE_BF16 or "
                                    "LA_DTYPE_BF16_F32OUT, got " + std::to_string(dtype));
  return LA_OK;
}

int check_gates(int mode, const float* log_alpha, const float* beta) {
  if (la::mode_erase(mode) && !beta)
    return fail(LA_ERR_NULL, "beta is required for the delta modes");
  if (la::mode_decay(mode) && !log_alpha)
    return fail(LA_ERR_NULL, "log_alpha is required for the gated modes");
  return LA_OK;
}

// ---- kernel timing with HIP events (la_profile_begin / la_profile_end)
struct TimedLaunch {
  const char* name;
  hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<TimedLaunch> g_prof;

// Records an event on `st` if profiling is on; returns it (or nullptr).
hipEvent_t prof_mark(hipStream_t st) {
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_on) return nullptr;
  }
  hipEvent_t ev = nullptr;
  if (hipEventCreate(&ev) != hipSuccess) return nullptr;
  if (hipEventRecord(ev, st) != hipSuccess) {
    (void)hipEventDestroy(ev);
    return nullptr;
  }
  return ev;
}

void prof_add(const char* name, hipEvent_t a, hipEvent_t b) {
  if (!a || !b) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof.push_back({name, a, b});
}

// Shape, mode and dtype checks shared by la_chunk_fwd and
// la_chunk_workspace_bytes.
int check_chunk_shape(int B, int H, int L, int dk, int dv, int C, int mode, int dtype) {
  if (int e = check_mode_dtype(mode, dtype)) return e;
  if (B <= 0 || H <= 0 || L <= 0 || dk <= 0 || dv <= 0 || C <= 0)
    return fail(LA_ERR_SHAPE, "B, H, L, dk, dv and C must be positive");
  if (L > LA_MAX_TOKENS)
    return fail(LA_ERR_SHAPE, "L must be at most LA_MAX_TOKENS, got " + std::to_string(L));
  if (dk != dv || (dk != 64 && dk != 128))
    return fail(LA_ERR_UNSUPPORTED, "la_chunk_fwd supports dk == dv in {64, 128}, got dk=" +
                                        std::to_string(dk) + " dv=" + std::to_string(dv));
  if (C != 64)
    return fail(LA_ERR_UNSUPPORTED, "la_chunk_fwd supports C == 64, got " + std::to_string(C));
  size_t n_qk;
  if (!count({B, H, L, dk}, &n_qk) || n_qk > (SIZE_MAX >> 4))
    return fail(LA_ERR_SHAPE, "tensor sizes overflow size_t");
  const size_t nc = ((size_t)L + C - 1) / C;             // chunks, the last may be partial
  if ((size_t)B * H * (dv / 16) > 0x7fffffffu || (size_t)B * H * nc > 0x7fffffffu)
    return fail(LA_ERR_SHAPE, "B * H * dv / 16 or B * H * ceil(L / C) exceeds the launch grid");
  return LA_OK;
}

// Options of the fused entry points (NULL: none), reduced to what the mode
// uses (gate activations mean nothing in LINEAR mode): the effective flags.
struct Fused {
  int flags = 0;
  float gate_scale = 0.f;
  const float* dskip = nullptr;
  const float* norm_w = nullptr;
  float norm_eps = 0.f;
  int pro() const { return flags & (LA_PRO_GATES | LA_PRO_QK_L2NORM); }
};

int check_fused(const la_fused_opts_t* o, int mode, Fused* f) {
  *f = Fused{};
  if (!o) return LA_OK;
  const int all = LA_PRO_GATES | LA_PRO_QK_L2NORM | LA_EPI_DSKIP | LA_EPI_OUT_NORM;
  if (o->flags < 0 || (o->flags & ~all))
    return fail(LA_ERR_UNSUPPORTED, "fused flags must combine la_fused_flag_t values, got " +
                                        std::to_string(o->flags));
  const bool gates = la::mode_erase(mode) || la::mode_decay(mode);
  f->flags = gates ? o->flags : (o->flags & ~LA_PRO_GATES);
  if ((f->flags & LA_PRO_GATES) && la::mode_decay(mode)) {
    if (!(o->gate_scale > 0.f && o->gate_scale < 3.0e38f))
      return fail(LA_ERR_UNSUPPORTED, "gate_scale must be positive and finite");
    f->gate_scale = o->gate_scale;
  }
  if (f->flags & LA_EPI_DSKIP) {
    if (!o->dskip) return fail(LA_ERR_NULL, "LA_EPI_DSKIP needs dskip [H, dv]");
    f->dskip = o->dskip;
  }
  if (f->flags & LA_EPI_OUT_NORM) {
    if (!(o->norm_eps > 0.f && o->norm_eps < 3.0e38f))
      return fail(LA_ERR_UNSUPPORTED, "norm_eps must be positive and finite");
    f->norm_w = o->norm_weight;
    f->norm_eps = o->norm_eps;
  }
  return LA_OK;
}

void apply_fused(const Fused& f, la::ChunkArgs* a) {
  a->pro = f.pro();
  a->gate_scale = f.gate_scale;
  a->dskip = f.dskip;
  a->out_norm = (f.flags & LA_EPI_OUT_NORM) != 0;
  a->norm_w = f.norm_w;
  a->norm_eps = f.norm_eps;
}

// Shapes of the non-causal form: bf16 inputs, dk = dv in {64, 128}.
int check_noncausal(int B, int H, int L, int dk, int dv, int dtype) {
  if (dtype != LA_DTYPE_BF16 && dtype != LA_DTYPE_BF16_F32OUT)
    return fail(LA_ERR_UNSUPPORTED, "la_noncausal_fwd takes bf16 inputs (LA_DTYPE_BF16 or "
                                    "LA_DTYPE_BF16_F32OUT), got " + std::to_string(dtype));
  return check_chunk_shape(B, H, L, dk, dv, 64, LA_MODE_LINEAR, dtype);
}

// Segment count of la_chunk_fwd_segmented: 1 .. min(ceil(L / C), 1024);
// above 1 only for bf16 inputs.
int check_segments(int L, int C, int dtype, int segments) {
  const long nc = ((long)L + C - 1) / C;
  if (segments < 1 || segments > nc || segments > 1024)
    return fail(LA_ERR_SHAPE, "segments must be in [1, min(ceil(L / C), 1024)], got " +
                                  std::to_string(segments));
  if (segments > 1 && dtype == LA_DTYPE_F32)
    return fail(LA_ERR_UNSUPPORTED, "the sequence-parallel forward takes bf16 inputs");
  return LA_OK;
}

la::ChunkArgs chunk_args(const void* q, const void* k, const void* v, const float* log_alpha,
                         const float* beta, const float* S0, void* out, float* S_final, int B,
                         int H, int L, int dk, int C, int mode, int dtype, void* workspace,
                         const int* cu = nullptr) {
  return la::ChunkArgs{q, k, v, log_alpha, beta, S0, out, S_final, B, H, L, dk, C, mode,
                       dtype != LA_DTYPE_F32, dtype == LA_DTYPE_BF16, workspace, cu};
}

// Shape checks of a packed batch: N sequences of H heads over T tokens.
int check_varlen_shape(int N, int H, int T, int dk, int dv, int C, int mode, int dtype) {
  if (int e = check_mode_dtype(mode, dtype)) return e;
  if (N <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0 || C <= 0)
    return fail(LA_ERR_SHAPE, "N, H, dk, dv and C must be positive and T non-negative");
  if (T > LA_MAX_TOKENS)
    return fail(LA_ERR_SHAPE, "T must be at most LA_MAX_TOKENS, got " + std::to_string(T));
  if (dk != dv || (dk != 64 && dk != 128))
    return fail(LA_ERR_UNSUPPORTED, "la_chunk_fwd_varlen supports dk == dv in {64, 128}, got "
                                    "dk=" + std::to_string(dk) + " dv=" + std::to_string(dv));
  if (C != 64)
    return fail(LA_ERR_UNSUPPORTED, "la_chunk_fwd_varlen supports C == 64, got " +
                                        std::to_string(C));
  size_t n_qk;
  if (!count({H, T, dk}, &n_qk) || n_qk > (SIZE_MAX >> 4) || !count({N, H, dk, dv}, &n_qk))
    return fail(LA_ERR_SHAPE, "tensor sizes overflow size_t");
  const size_t slots = (size_t)H * (((size_t)T + C - 1) / C + (size_t)N);
  if ((size_t)N * H * (dv / 16) > 0x7fffffffu || slots > 0x7fffffffu)
    return fail(LA_ERR_SHAPE, "N * H * dv / 16 or H * (ceil(T / C) + N) exceeds the launch grid");
  return LA_OK;
}

// Workspace and alias checks, then the launches, shared by both forward
// entry points.  n_* are element counts of the tensors; cu (packed batches)
// is an input of cu_bytes bytes.
int run_chunk(const la::ChunkArgs& a, size_t n_qk, size_t n_v, size_t n_g, size_t n_s,
              int dtype, size_t workspace_bytes, size_t cu_bytes, void* stream,
              bool check_only = false) {
  const size_t need = la::chunk_workspace_bytes(a);
  if (need > 0 && !check_only) {
    if (!a.workspace)
      return fail(LA_ERR_WORKSPACE, "this call needs a workspace of " + std::to_string(need) +
                                        " bytes (la_chunk_workspace_bytes)");
    if (workspace_bytes < need)
      return fail(LA_ERR_WORKSPACE, "workspace has " + std::to_string(workspace_bytes) +
                                        " bytes, this call needs " + std::to_string(need));
    if (reinterpret_cast<uintptr_t>(a.workspace) % 16 != 0)
      return fail(LA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  }
  const size_t esz = dtype == LA_DTYPE_F32 ? 4 : 2;
  const size_t osz = dtype == LA_DTYPE_BF16 ? 2 : 4;
  const Range rq(a.q, n_qk * esz), rk(a.k, n_qk * esz), rv(a.v, n_v * esz);
  const Range rla(la::mode_decay(a.mode) ? a.log_alpha : nullptr, n_g * 4);
  const Range rb(la::mode_erase(a.mode) ? a.beta : nullptr, n_g * 4);
  const Range rs0(a.S0, n_s * 4), ro(a.out, n_v * osz), rsf(a.S_final, n_s * 4);
  const Range rws(need > 0 ? a.workspace : nullptr, need);
  const Range rcu(a.cu, cu_bytes);
  const size_t n_hd = (size_t)a.H * a.d * 4;             // an [H, dv] float parameter
  const Range rds(a.dskip, n_hd), rnw(a.out_norm ? a.norm_w : nullptr, n_hd);
  for (const Range* in : {&rq, &rk, &rv, &rla, &rb, &rs0, &rcu, &rds, &rnw})
    if (ro.overlaps(*in)) return fail(LA_ERR_ALIAS, "out overlaps an input");
  for (const Range* in : {&rq, &rk, &rv, &rla, &rb, &ro, &rcu, &rds, &rnw})
    if (rsf.overlaps(*in)) return fail(LA_ERR_ALIAS, "S_final overlaps an input or out");
  if (rsf.overlaps(rs0) && (a.S0 != a.S_final))
    return fail(LA_ERR_ALIAS, "S_final partially overlaps S0 (only S_final == S0 is allowed)");
  for (const Range* in : {&rq, &rk, &rv, &rla, &rb, &rs0, &ro, &rsf, &rcu, &rds, &rnw})
    if (rws.overlaps(*in)) return fail(LA_ERR_ALIAS, "workspace overlaps an input or output");
  if (check_only) return LA_OK;

  hipStream_t st = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = prof_mark(st);
  if (la::chunk_needs_tsolve(a)) {
    const hipError_t e = la::launch_tsolve(a, st);
    hipEvent_t e1 = prof_mark(st);
    prof_add("la_tsolve", e0, e1);
    if (e != hipSuccess) return fail_hip("launching the T-solve kernel", e);
    e0 = e1;
  }
  if (a.P > 1) {
    hipError_t e = la::launch_chunk_state(a, st);
    hipEvent_t e1 = prof_mark(st);
    prof_add("la_chunk_state", e0, e1);
    if (e != hipSuccess) return fail_hip("launching the state pass", e);
    e = la::launch_seg_scan(a, st);
    e0 = prof_mark(st);
    prof_add("la_seg_scan", e1, e0);
    if (e != hipSuccess) return fail_hip("launching the segment scan", e);
  }
  hipError_t e = la::launch_chunk(a, st);
  hipEvent_t e1 = prof_mark(st);
  prof_add("la_chunk", e0, e1);
  if (e != hipSuccess) return fail_hip("launching the chunk kernel", e);
  if (a.out_norm) {
    e = la::launch_out_norm(a, st);
    prof_add("la_out_norm", e1, prof_mark(st));
    if (e != hipSuccess) return fail_hip("launching the output norm", e);
  }
  return LA_OK;
}

// la_decode_step and la_decode_step_fused (flags 0: the inputs as given).
int decode_step(const void* q, const void* k, const void* v, const float* log_alpha,
                const float* beta, float* S, void* out, int B, int H, int dk, int dv, int mode,
                int dtype, const la_fused_opts_t* opts, void* stream) {
  if (!q || !k || !v || !S || !out) return fail(LA_ERR_NULL, "q, k, v, S and out are required");
  if (int e = check_mode_dtype(mode, dtype)) return e;
  if (int e = check_gates(mode, log_alpha, beta)) return e;
  Fused f;
  if (int e = check_fused(opts, mode, &f)) return e;
  if (B <= 0 || H <= 0 || dk <= 0 || dv <= 0)
    return fail(LA_ERR_SHAPE, "B, H, dk and dv must be positive");
  if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128))
    return fail(LA_ERR_UNSUPPORTED, "la_decode_step supports dk, dv in {64, 128}, got dk=" +
                                        std::to_string(dk) + " dv=" + std::to_string(dv));
  size_t n_k, n_v, n_g, n_s;
  if (!count({B, H, dk}, &n_k) || !count({B, H, dv}, &n_v) || !count({B, H}, &n_g) ||
      !count({B, H, dk, dv}, &n_s) || n_s > (SIZE_MAX >> 3))
    return fail(LA_ERR_SHAPE, "tensor sizes overflow size_t");
  if (n_g > 0x7fffffffu) return fail(LA_ERR_SHAPE, "B * H exceeds the launch grid");
  const size_t esz = dtype == LA_DTYPE_F32 ? 4 : 2;
  const size_t osz = dtype == LA_DTYPE_BF16 ? 2 : 4;
  const Range rq(q, n_k * esz), rk(k, n_k * esz), rv(v, n_v * esz);
  const Range rla(la::mode_decay(mode) ? log_alpha : nullptr, n_g * 4);
  const Range rb(la::mode_erase(mode) ? beta : nullptr, n_g * 4);
  const Range rs(S, n_s * 4), ro(out, n_v * osz);
  const Range rds(f.dskip, (size_t)H * dv * 4);
  const Range rnw((f.flags & LA_EPI_OUT_NORM) ? f.norm_w : nullptr, (size_t)H * dv * 4);
  for (const Range* in : {&rq, &rk, &rv, &rla, &rb, &rs, &rds, &rnw})
    if (ro.overlaps(*in)) return fail(LA_ERR_ALIAS, "out overlaps S or an input");
  for (const Range* in : {&rq, &rk, &rv, &rla, &rb, &rds, &rnw})
    if (rs.overlaps(*in)) return fail(LA_ERR_ALIAS, "S overlaps an input");

  la::DecodeArgs a{q, k, v, log_alpha, beta, S, out, B, H, dk, dv, mode,
                   dtype != LA_DTYPE_F32, dtype == LA_DTYPE_BF16, f.pro(), f.gate_scale};
  a.dskip = f.dskip;
  a.out_norm = (f.flags & LA_EPI_OUT_NORM) != 0;
  a.norm_w = f.norm_w;
  a.norm_eps = f.norm_eps;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = prof_mark(st);
  hipError_t e = la::launch_decode(a, st);
  prof_add("la_decode", e0, prof_mark(st));
  if (e != hipSuccess) return fail_hip("launching the decode kernel", e);
  return LA_OK;
}

// Shape checks of la_chunk_bwd: those of the forward, float32 or bf16
// inputs with gradients of the output in the same type.
int check_bwd_shape(int B, int H, int L, int dk, int dv, int C, int mode, int dtype) {
  if (dtype == LA_DTYPE_BF16_F32OUT)
    return fail(LA_ERR_UNSUPPORTED, "la_chunk_bwd takes LA_DTYPE_F32 or LA_DTYPE_BF16");
  if (int e = check_chunk_shape(B, H, L, dk, dv, C, mode, dtype)) return e;
  if ((size_t)B * H * ((L + (size_t)C - 1) / C) * dk * dk > (SIZE_MAX >> 4))
    return fail(LA_ERR_SHAPE, "workspace size overflows size_t");
  return LA_OK;
}

la::BwdArgs bwd_args(int B, int H, int L, int d, int mode, int dtype, void* workspace) {
  la::BwdArgs a{};
  a.B = B;
  a.H = H;
  a.L = L;
  a.d = d;
  a.mode = mode;
  a.in_bf16 = dtype != LA_DTYPE_F32;
  a.workspace = workspace;
  return a;
}

// Pointer and mode checks shared by la_chunk_bwd and la_chunk_bwd_varlen.
int check_bwd_args(const void* q, const void* k, const void* v, const float* log_alpha,
                   const float* beta, const void* grad_out, const float* grad_q,
                   const float* grad_k, const float* grad_v, const float* grad_log_alpha,
                   const float* grad_beta, int mode, int dtype) {
  if (!q || !k || !v || !grad_out || !grad_q || !grad_k || !grad_v)
    return fail(LA_ERR_NULL, "q, k, v, grad_out, grad_q, grad_k and grad_v are required");
  if (int e = check_mode_dtype(mode, dtype)) return e;
  if (int e = check_gates(mode, log_alpha, beta)) return e;
  if (la::mode_decay(mode) && !grad_log_alpha)
    return fail(LA_ERR_NULL, "grad_log_alpha is required for the gated modes");
  if (la::mode_erase(mode) && !grad_beta)
    return fail(LA_ERR_NULL, "grad_beta is required for the delta modes");
  return LA_OK;
}

// Workspace and alias checks, then the four launches.  n_x, n_g, n_s are
// the element counts of a token tensor, a gate tensor and the states; cu
// (packed batches) is an input of cu_bytes bytes.
int run_bwd(const la::BwdArgs& a, size_t n_x, size_t n_g, size_t n_s, int dtype,
            size_t workspace_bytes, size_t cu_bytes, void* stream) {
  const size_t need = la::bwd_workspace_bytes(a);
  if (!a.workspace)
    return fail(LA_ERR_WORKSPACE, "this call needs a workspace of " + std::to_string(need) +
                                      " bytes (la_chunk_bwd_workspace_bytes)");
  if (workspace_bytes < need)
    return fail(LA_ERR_WORKSPACE, "workspace has " + std::to_string(workspace_bytes) +
                                      " bytes, this call needs " + std::to_string(need));
  if (reinterpret_cast<uintptr_t>(a.workspace) % 16 != 0)
    return fail(LA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  const bool gated = la::mode_decay(a.mode), erase = la::mode_erase(a.mode);
  const size_t esz = dtype == LA_DTYPE_F32 ? 4 : 2;
  const Range rq(a.q, n_x * esz), rk(a.k, n_x * esz), rv(a.v, n_x * esz);
  const Range rdo(a.dout, n_x * esz);
  const Range rla(gated ? a.log_alpha : nullptr, n_g * 4), rb(erase ? a.beta : nullptr, n_g * 4);
  const Range rs0(a.S0, n_s * 4), rdsf(a.dS_final, n_s * 4), rcu(a.cu, cu_bytes);
  const Range oq(a.dq, n_x * 4), ok(a.dk, n_x * 4), ov(a.dv, n_x * 4);
  const Range ola(gated ? a.dlog_alpha : nullptr, n_g * 4);
  const Range ob(erase ? a.dbeta : nullptr, n_g * 4), os0(a.dS0, n_s * 4);
  const Range rws(a.workspace, need);
  const Range* ins[] = {&rq, &rk, &rv, &rdo, &rla, &rb, &rs0, &rdsf, &rcu};
  const Range* outs[] = {&oq, &ok, &ov, &ola, &ob, &os0, &rws};
  for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
    for (const Range* in : ins)
      if (outs[i]->overlaps(*in))
        return fail(LA_ERR_ALIAS, "a gradient output or the workspace overlaps an input");
    for (size_t j = 0; j < i; ++j)
      if (outs[i]->overlaps(*outs[j]))
        return fail(LA_ERR_ALIAS, "two gradient outputs (or one and the workspace) overlap");
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  struct Step {
    const char* name;
    hipError_t (*launch)(const la::BwdArgs&, hipStream_t);
  };
  const Step steps[] = {{"la_bwd_prep", la::launch_bwd_prep},
                        {"la_bwd_states", la::launch_bwd_states},
                        {"la_bwd_rev", la::launch_bwd_rev},
                        {"la_bwd_grads", la::launch_bwd_grads}};
  hipEvent_t e0 = prof_mark(st);
  for (const Step& s : steps) {
    const hipError_t e = s.launch(a, st);
    hipEvent_t e1 = prof_mark(st);
    prof_add(s.name, e0, e1);
    if (e != hipSuccess) return fail_hip(s.name, e);
    e0 = e1;
  }
  return LA_OK;
}

// Workspace of la_chunk_bwd_fused: the prologue's arrays (the inverse norms
// of q and k, the activated gates), each 256-byte aligned, then the
// backward's own workspace.
struct ProWs {
  size_t rq, rk, la, be, core;           // byte offsets
  size_t bytes;                          // in all
};

ProWs pro_ws(const la::BwdArgs& a, int flags) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t rows = (size_t)a.B * a.H * a.L;
  const bool norm = flags & LA_PRO_QK_L2NORM, gates = flags & LA_PRO_GATES;
  ProWs w{};
  size_t off = 0;
  auto take = [&](size_t n) { const size_t o = off; off += al(n); return o; };
  w.rq = take(norm ? rows * 4 : 0);
  w.rk = take(norm ? rows * 4 : 0);
  w.la = take(gates && la::mode_decay(a.mode) ? rows * 4 : 0);
  w.be = take(gates && la::mode_erase(a.mode) ? rows * 4 : 0);
  w.core = off;
  w.bytes = off + la::bwd_workspace_bytes(a);
  return w;
}

// Fused flags the backward takes: the prologue's (the epilogue's backward is
// not built).
int check_bwd_fused(const la_fused_opts_t* opts, int mode, Fused* f) {
  if (int e = check_fused(opts, mode, f)) return e;
  if (f->flags & (LA_EPI_DSKIP | LA_EPI_OUT_NORM))
    return fail(LA_ERR_UNSUPPORTED, "la_chunk_bwd_fused takes LA_PRO_GATES and "
                                    "LA_PRO_QK_L2NORM only (no backward of the epilogue)");
  return LA_OK;
}

// Device address of `scratch` on the current device, looked up on the first
// call there and kept per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip("hipGetDevice", e);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(LA_ERR_HIP, "device index " + std::to_string(dev) + " out of range");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail_hip("hipGetSymbolAddress(scratch)", e);
    if (!p) return fail(LA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LA_OK;
}

}  // namespace

extern "C" {

const char* la_last_error(void) { return g_last_error.c_str(); }

const char* la_version(void) { return "lachunk 0.4.0 gfx950"; }

int la_chunk_workspace_bytes(int B, int H, int L, int dk, int dv, int C, int mode, int dtype,
                             size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(LA_ERR_NULL, "bytes is required");
  if (int e = check_chunk_shape(B, H, L, dk, dv, C, mode, dtype)) return e;
  la::ChunkArgs a = chunk_args(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                               nullptr, B, H, L, dk, C, mode, dtype, nullptr);
  a.P = la::plan_segments(a);
  *bytes = la::chunk_workspace_bytes(a);
  return LA_OK;
}

int la_chunk_fused_workspace_bytes(int B, int H, int L, int dk, int dv, int C, int mode,
                                   int dtype, const la_fused_opts_t* opts, size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(LA_ERR_NULL, "bytes is required");
  if (int e = check_chunk_shape(B, H, L, dk, dv, C, mode, dtype)) return e;
  Fused f;
  if (int e = check_fused(opts, mode, &f)) return e;
  if (f.flags && dtype == LA_DTYPE_F32)
    return fail(LA_ERR_UNSUPPORTED, "the fused forward takes bf16 inputs");
  la::ChunkArgs a = chunk_args(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                               nullptr, B, H, L, dk, C, mode, dtype, nullptr);
  apply_fused(f, &a);
  a.P = la::plan_segments(a);
  *bytes = la::chunk_workspace_bytes(a);
  return LA_OK;
}

int la_chunk_bwd_workspace_bytes(int B, int H, int L, int dk, int dv, int C, int mode, int dtype,
                                 size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(LA_ERR_NULL, "bytes is required");
  if (int e = check_bwd_shape(B, H, L, dk, dv, C, mode, dtype)) return e;
  *bytes = la::bwd_workspace_bytes(bwd_args(B, H, L, dk, mode, dtype, nullptr));
  return LA_OK;
}

int la_chunk_bwd(const void* q, const void* k, const void* v, const float* log_alpha,
                 const float* beta, const float* S0, const void* grad_out,
                 const float* grad_S_final, float* grad_q, float* grad_k, float* grad_v,
                 float* grad_log_alpha, float* grad_beta, float* grad_S0, int B, int H, int L,
                 int dk, int dv, int C, int mode, int dtype, void* workspace,
                 size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (int e = check_bwd_args(q, k, v, log_alpha, beta, grad_out, grad_q, grad_k, grad_v,
                             grad_log_alpha, grad_beta, mode, dtype))
    return e;
  if (int e = check_bwd_shape(B, H, L, dk, dv, C, mode, dtype)) return e;
  size_t n_x, n_g, n_s;
  if (!count({B, H, L, dk}, &n_x) || !count({B, H, L}, &n_g) || !count({B, H, dk, dv}, &n_s))
    return fail(LA_ERR_SHAPE, "tensor sizes overflow size_t");
  la::BwdArgs a = bwd_args(B, H, L, dk, mode, dtype, workspace);
  a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta; a.S0 = S0;
  a.dout = grad_out; a.dS_final = grad_S_final;
  a.dq = grad_q; a.dk = grad_k; a.dv = grad_v; a.dlog_alpha = grad_log_alpha;
  a.dbeta = grad_beta; a.dS0 = grad_S0;
  return run_bwd(a, n_x, n_g, n_s, dtype, workspace_bytes, 0, stream);
}

int la_chunk_bwd_varlen_workspace_bytes(int N, int H, int T, int dk, int dv, int C, int mode,
                                        int dtype, size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(LA_ERR_NULL, "bytes is required");
  if (dtype == LA_DTYPE_BF16_F32OUT)
    return fail(LA_ERR_UNSUPPORTED, "la_chunk_bwd_varlen takes LA_DTYPE_F32 or LA_DTYPE_BF16");
  if (int e = check_varlen_shape(N, H, T, dk, dv, C, mode, dtype)) return e;
  la::BwdArgs a = bwd_args(N, H, T, dk, mode, dtype, nullptr);
  a.packed = true;
  *bytes = la::bwd_workspace_bytes(a);
  return LA_OK;
}

int la_chunk_bwd_varlen(const void* q, const void* k, const void* v, const float* log_alpha,
                        const float* beta, const float* S0, const void* grad_out,
                        const float* grad_S_final, const int* cu_seqlens, float* grad_q,
                        float* grad_k, float* grad_v, float* grad_log_alpha, float* grad_beta,
                        float* grad_S0, int N, int H, int T, int dk, int dv, int C, int mode,
                        int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!cu_seqlens) return fail(LA_ERR_NULL, "cu_seqlens is required");
  if (int e = check_bwd_args(q, k, v, log_alpha, beta, grad_out, grad_q, grad_k, grad_v,
                             grad_log_alpha, grad_beta, mode, dtype))
    return e;
  if (dtype == LA_DTYPE_BF16_F32OUT)
    return fail(LA_ERR_UNSUPPORTED, "la_chunk_bwd_varlen takes LA_DTYPE_F32 or LA_DTYPE_BF16");
  if (int e = check_varlen_shape(N, H, T, dk, dv, C, mode, dtype)) return e;
  size_t n_x, n_g, n_s;
  if (!count({H, T, dk}, &n_x) || !count({H, T}, &n_g) || !count({N, H, dk, dv}, &n_s))
    return fail(LA_ERR_SHAPE, "tensor sizes overflow size_t");
  la::BwdArgs a = bwd_args(N, H, T, dk, mode, dtype, workspace);
  a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta; a.S0 = S0;
  a.dout = grad_out; a.dS_final = grad_S_final;
  a.dq = grad_q; a.dk = grad_k; a.dv = grad_v; a.dlog_alpha = grad_log_alpha;
  a.dbeta = grad_beta; a.dS0 = grad_S0;
  a.cu = cu_seqlens;
  return run_bwd(a, n_x, n_g, n_s, dtype, workspace_bytes, (size_t)(N + 1) * sizeof(int),
                 stream);
}

int la_chunk_bwd_fused_workspace_bytes(int B, int H, int L, int dk, int dv, int C, int mode,
                                       int dtype, const la_fused_opts_t* opts, size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(LA_ERR_NULL, "bytes is required");
  if (int e = check_bwd_shape(B, H, L, dk, dv, C, mode, dtype)) return e;
  Fused f;
  if (int e = check_bwd_fused(opts, mode, &f)) return e;
  *bytes = pro_ws(bwd_args(B, H, L, dk, mode, dtype, nullptr), f.flags).bytes;
  return LA_OK;
}

int la_chunk_bwd_fused(const void* q, const void* k, const void* v, const float* a_raw,
                       const float* b_raw, const float* S0, const void* grad_out,
                       const float* grad_S_final, float* grad_q, float* grad_k, float* grad_v,
                       float* grad_a, float* grad_b, float* grad_S0, int B, int H, int L,
                       int dk, int dv, int C, int mode, int dtype, const la_fused_opts_t* opts,
                       void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (int e = check_bwd_args(q, k, v, a_raw, b_raw, grad_out, grad_q, grad_k, grad_v, grad_a,
                             grad_b, mode, dtype))
    return e;
  if (int e = check_bwd_shape(B, H, L, dk, dv, C, mode, dtype)) return e;
  Fused f;
  if (int e = check_bwd_fused(opts, mode, &f)) return e;
  size_t n_x, n_g, n_s;
  if (!count({B, H, L, dk}, &n_x) || !count({B, H, L}, &n_g) || !count({B, H, dk, dv}, &n_s))
    return fail(LA_ERR_SHAPE, "tensor sizes overflow size_t");
  la::BwdArgs a = bwd_args(B, H, L, dk, mode, dtype, nullptr);
  const ProWs w = pro_ws(a, f.flags);
  if (!workspace)
    return fail(LA_ERR_WORKSPACE, "this call needs a workspace of " + std::to_string(w.bytes) +
                                      " bytes (la_chunk_bwd_fused_workspace_bytes)");
  if (workspace_bytes < w.bytes)
    return fail(LA_ERR_WORKSPACE, "workspace has " + std::to_string(workspace_bytes) +
                                      " bytes, this call needs " + std::to_string(w.bytes));
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return fail(LA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  // every input against the outputs and the whole workspace: the prologue
  // writes its arrays before the backward proper reads v, grad_out, S0 and
  // grad_S_final, so an input inside the prologue's region would be
  // overwritten first (the backward proper checks its own part again)
  const bool gated = la::mode_decay(mode), erase = la::mode_erase(mode);
  const size_t esz = dtype == LA_DTYPE_F32 ? 4 : 2;
  const Range rq(q, n_x * esz), rk(k, n_x * esz), rv(v, n_x * esz), rdo(grad_out, n_x * esz);
  const Range ra(gated ? a_raw : nullptr, n_g * 4), rb(erase ? b_raw : nullptr, n_g * 4);
  const Range rs0(S0, n_s * 4), rdsf(grad_S_final, n_s * 4), rws(workspace, w.bytes);
  const Range oq(grad_q, n_x * 4), ok(grad_k, n_x * 4), ov(grad_v, n_x * 4);
  const Range oa(gated ? grad_a : nullptr, n_g * 4), ob(erase ? grad_b : nullptr, n_g * 4);
  const Range os0(grad_S0, n_s * 4);
  for (const Range* in : {&rq, &rk, &rv, &rdo, &ra, &rb, &rs0, &rdsf})
    for (const Range* out : {&oq, &ok, &ov, &oa, &ob, &os0, &rws})
      if (in->overlaps(*out))
        return fail(LA_ERR_ALIAS, "a gradient output or the workspace overlaps an input");
  char* base = static_cast<char*>(workspace);
  const bool norm = f.flags & LA_PRO_QK_L2NORM;
  const bool ga = (f.flags & LA_PRO_GATES) && gated, gb = (f.flags & LA_PRO_GATES) && erase;
  la::BwdProArgs p{};
  p.q = q; p.k = k; p.a_raw = a_raw; p.b_raw = b_raw;
  p.rq = reinterpret_cast<float*>(base + w.rq); p.rk = reinterpret_cast<float*>(base + w.rk);
  p.la = reinterpret_cast<float*>(base + w.la); p.be = reinterpret_cast<float*>(base + w.be);
  p.dq = grad_q; p.dk = grad_k; p.da = grad_a; p.db = grad_b;
  p.rows = n_g; p.d = dk; p.in_bf16 = dtype != LA_DTYPE_F32;
  p.norm = norm; p.gates_a = ga; p.gates_b = gb; p.scale = f.gate_scale;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool any = norm || ga || gb;
  if (any) {
    hipEvent_t e0 = prof_mark(st);
    const hipError_t e = la::launch_bwd_pro(p, false, st);
    prof_add("la_bwd_pro", e0, prof_mark(st));
    if (e != hipSuccess) return fail_hip("launching the backward prologue", e);
  }
  a.workspace = base + w.core;
  // the raw q and k, their inverse norms applied per row inside the products
  a.q = q; a.k = k; a.v = v;
  a.rq = norm ? p.rq : nullptr; a.rk = norm ? p.rk : nullptr;
  a.log_alpha = ga ? p.la : a_raw; a.beta = gb ? p.be : b_raw; a.S0 = S0;
  a.dout = grad_out; a.dS_final = grad_S_final;
  a.dq = grad_q; a.dk = grad_k; a.dv = grad_v; a.dlog_alpha = grad_a; a.dbeta = grad_b;
  a.dS0 = grad_S0;
  if (int e = run_bwd(a, n_x, n_g, n_s, dtype, w.bytes - w.core, 0, stream)) return e;
  if (any) {
    hipEvent_t e0 = prof_mark(st);
    const hipError_t e = la::launch_bwd_pro(p, true, st);
    prof_add("la_bwd_pro_grad", e0, prof_mark(st));
    if (e != hipSuccess) return fail_hip("launching the backward prologue's gradients", e);
  }
  return LA_OK;
}

int la_noncausal_workspace_bytes(int B, int H, int L, int dk, int dv, int dtype,
                                 size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(LA_ERR_NULL, "bytes is required");
  if (int e = check_noncausal(B, H, L, dk, dv, dtype)) return e;
  la::ChunkArgs a = chunk_args(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                               nullptr, B, H, L, dk, 64, LA_MODE_LINEAR, dtype, nullptr);
  a.P = la::plan_sum_segments(a);
  *bytes = la::noncausal_workspace_bytes(a);
  return LA_OK;
}

int la_noncausal_fwd(const void* q, const void* k, const void* v, const float* S0, void* out,
                     float* S_final, int B, int H, int L, int dk, int dv, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!q || !k || !v || !out) return fail(LA_ERR_NULL, "q, k, v and out are required");
  if (int e = check_noncausal(B, H, L, dk, dv, dtype)) return e;
  size_t n_qk, n_s;
  if (!count({B, H, L, dk}, &n_qk) || !count({B, H, dk, dv}, &n_s))
    return fail(LA_ERR_SHAPE, "tensor sizes overflow size_t");
  la::ChunkArgs a = chunk_args(q, k, v, nullptr, nullptr, S0, out, S_final, B, H, L, dk, 64,
                               LA_MODE_LINEAR, dtype, workspace);
  a.P = la::plan_sum_segments(a);
  const size_t need = la::noncausal_workspace_bytes(a);
  if (!workspace)
    return fail(LA_ERR_WORKSPACE, "this call needs a workspace of " + std::to_string(need) +
                                      " bytes (la_noncausal_workspace_bytes)");
  if (workspace_bytes < need)
    return fail(LA_ERR_WORKSPACE, "workspace has " + std::to_string(workspace_bytes) +
                                      " bytes, this call needs " + std::to_string(need));
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return fail(LA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  const size_t osz = dtype == LA_DTYPE_BF16 ? 2 : 4;
  const Range rq(q, n_qk * 2), rk(k, n_qk * 2), rv(v, n_qk * 2), rs0(S0, n_s * 4);
  const Range ro(out, n_qk * osz), rsf(S_final, n_s * 4), rws(workspace, need);
  for (const Range* in : {&rq, &rk, &rv, &rs0})
    if (ro.overlaps(*in)) return fail(LA_ERR_ALIAS, "out overlaps an input");
  for (const Range* in : {&rq, &rk, &rv, &ro})
    if (rsf.overlaps(*in)) return fail(LA_ERR_ALIAS, "S_final overlaps an input or out");
  if (rsf.overlaps(rs0) && S0 != S_final)
    return fail(LA_ERR_ALIAS, "S_final partially overlaps S0 (only S_final == S0 is allowed)");
  for (const Range* in : {&rq, &rk, &rv, &rs0, &ro, &rsf})
    if (rws.overlaps(*in)) return fail(LA_ERR_ALIAS, "workspace overlaps an input or output");
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = prof_mark(st);
  const hipError_t e = la::launch_noncausal(a, st);
  prof_add("la_noncausal", e0, prof_mark(st));
  if (e != hipSuccess) return fail_hip("launching the non-causal kernels", e);
  return LA_OK;
}

int la_chunk_segments(int B, int H, int L, int dk, int dv, int C, int mode, int dtype,
                      int* segments) {
  g_last_error.clear();
  if (!segments) return fail(LA_ERR_NULL, "segments is required");
  if (int e = check_chunk_shape(B, H, L, dk, dv, C, mode, dtype)) return e;
  *segments = la::plan_segments(chunk_args(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                           nullptr, nullptr, B, H, L, dk, C, mode, dtype,
                                           nullptr));
  return LA_OK;
}

int la_chunk_segmented_workspace_bytes(int B, int H, int L, int dk, int dv, int C, int mode,
                                       int dtype, int segments, size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(LA_ERR_NULL, "bytes is required");
  if (int e = check_chunk_shape(B, H, L, dk, dv, C, mode, dtype)) return e;
  if (int e = check_segments(L, C, dtype, segments)) return e;
  la::ChunkArgs a = chunk_args(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                               nullptr, B, H, L, dk, C, mode, dtype, nullptr);
  a.P = segments;
  *bytes = la::chunk_workspace_bytes(a);
  return LA_OK;
}

int la_chunk_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                 const float* beta, const float* S0, void* out, float* S_final, int B,
                 int H, int L, int dk, int dv, int C, int mode, int dtype, void* workspace,
                 size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!q || !k || !v || !out) return fail(LA_ERR_NULL, "q, k, v and out are required");
  if (int e = check_mode_dtype(mode, dtype)) return e;
  if (int e = check_gates(mode, log_alpha, beta)) return e;
  if (int e = check_chunk_shape(B, H, L, dk, dv, C, mode, dtype)) return e;
  size_t n_qk, n_v, n_g, n_s;
  if (!count({B, H, L, dk}, &n_qk) || !count({B, H, L, dv}, &n_v) ||
      !count({B, H, L}, &n_g) || !count({B, H, dk, dv}, &n_s))
    return fail(LA_ERR_SHAPE, "tensor sizes overflow size_t");
  la::ChunkArgs a = chunk_args(q, k, v, log_alpha, beta, S0, out, S_final, B, H, L, dk, C, mode,
                               dtype, workspace);
  a.P = la::plan_segments(a);
  return run_chunk(a, n_qk, n_v, n_g, n_s, dtype, workspace_bytes, 0, stream);
}

int la_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* log_alpha,
                         const float* beta, const float* S0, void* out, float* S_final, int B,
                         int H, int L, int dk, int dv, int C, int mode, int dtype,
                         void* stream) {
  g_last_error.clear();
  if (!q || !k || !v || !out) return fail(LA_ERR_NULL, "q, k, v and out are required");
  if (int e = check_mode_dtype(mode, dtype)) return e;
  if (int e = check_gates(mode, log_alpha, beta)) return e;
  if (int e = check_chunk_shape(B, H, L, dk, dv, C, mode, dtype)) return e;
  size_t n_qk, n_v, n_g, n_s;
  if (!count({B, H, L, dk}, &n_qk) || !count({B, H, L, dv}, &n_v) ||
      !count({B, H, L}, &n_g) || !count({B, H, dk, dv}, &n_s))
    return fail(LA_ERR_SHAPE, "tensor sizes overflow size_t");
  la::ChunkArgs a = chunk_args(q, k, v, log_alpha, beta, S0, out, S_final, B, H, L, dk, C, mode,
                               dtype, nullptr);
  a.P = la::plan_segments(a);
  const size_t need = la::chunk_workspace_bytes(a);
  if (need > LA_NOALLOC_SCRATCH_BYTES)
    return fail(LA_ERR_WORKSPACE, "this call needs " + std::to_string(need) +
                                      " bytes of scratch; la_chunk_fwd_noalloc holds " +
                                      std::to_string(LA_NOALLOC_SCRATCH_BYTES) +
                                      " (use la_chunk_fwd with a workspace)");
  // tensor checks first: no HIP call before every argument error is reported
  if (int e = run_chunk(a, n_qk, n_v, n_g, n_s, dtype, 0, 0, stream, true)) return e;
  if (need > 0) {
    if (int e = scratch_address(&a.workspace)) return e;
  }
  return run_chunk(a, n_qk, n_v, n_g, n_s, dtype, need, 0, stream);
}

int la_chunk_fwd_fused(const void* q, const void* k, const void* v, const float* a_raw,
                       const float* b_raw, const float* S0, void* out, float* S_final, int B,
                       int H, int L, int dk, int dv, int C, int mode, int dtype,
                       const la_fused_opts_t* opts, void* workspace, size_t workspace_bytes,
                       void* stream) {
  g_last_error.clear();
  if (!q || !k || !v || !out) return fail(LA_ERR_NULL, "q, k, v and out are required");
  if (int e = check_mode_dtype(mode, dtype)) return e;
  if (int e = check_gates(mode, a_raw, b_raw)) return e;
  if (int e = check_chunk_shape(B, H, L, dk, dv, C, mode, dtype)) return e;
  Fused f;
  if (int e = check_fused(opts, mode, &f)) return e;
  if (f.flags && dtype == LA_DTYPE_F32)
    return fail(LA_ERR_UNSUPPORTED, "the fused forward takes bf16 inputs");
  size_t n_qk, n_v, n_g, n_s;
  if (!count({B, H, L, dk}, &n_qk) || !count({B, H, L, dv}, &n_v) ||
      !count({B, H, L}, &n_g) || !count({B, H, dk, dv}, &n_s))
    return fail(LA_ERR_SHAPE, "tensor sizes overflow size_t");
  la::ChunkArgs a = chunk_args(q, k, v, a_raw, b_raw, S0, out, S_final, B, H, L, dk, C, mode,
                               dtype, workspace);
  apply_fused(f, &a);
  a.P = la::plan_segments(a);
  return run_chunk(a, n_qk, n_v, n_g, n_s, dtype, workspace_bytes, 0, stream);
}

int la_chunk_fwd_segmented(const void* q, const void* k, const void* v, const float* log_alpha,
                           const float* beta, const float* S0, void* out, float* S_final, int B,
                           int H, int L, int dk, int dv, int C, int mode, int dtype, int segments,
                           void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!q || !k || !v || !out) return fail(LA_ERR_NULL, "q, k, v and out are required");
  if (int e = check_mode_dtype(mode, dtype)) return e;
  if (int e = check_gates(mode, log_alpha, beta)) return e;
  if (int e = check_chunk_shape(B, H, L, dk, dv, C, mode, dtype)) return e;
  if (int e = check_segments(L, C, dtype, segments)) return e;
  size_t n_qk, n_v, n_g, n_s;
  if (!count({B, H, L, dk}, &n_qk) || !count({B, H, L, dv}, &n_v) ||
      !count({B, H, L}, &n_g) || !count({B, H, dk, dv}, &n_s))
    return fail(LA_ERR_SHAPE, "tensor sizes overflow size_t");
  if ((size_t)B * H * (2 * (size_t)segments) * (dv / 16) > 0x7fffffffu)
    return fail(LA_ERR_SHAPE, "B * H * segments exceeds the launch grid");
  la::ChunkArgs a = chunk_args(q, k, v, log_alpha, beta, S0, out, S_final, B, H, L, dk, C, mode,
                               dtype, workspace);
  a.P = segments;
  return run_chunk(a, n_qk, n_v, n_g, n_s, dtype, workspace_bytes, 0, stream);
}

int la_chunk_varlen_workspace_bytes(int N, int H, int T, int dk, int dv, int C, int mode,
                                    int dtype, size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(LA_ERR_NULL, "bytes is required");
  if (int e = check_varlen_shape(N, H, T, dk, dv, C, mode, dtype)) return e;
  // the size depends on N, H, T only, not on the offsets themselves
  static const int kAny = 0;
  *bytes = la::chunk_workspace_bytes(
      chunk_args(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, N, H, T,
                 dk, C, mode, dtype, nullptr, &kAny));
  return LA_OK;
}

int la_chunk_fwd_varlen(const void* q, const void* k, const void* v, const float* log_alpha,
                        const float* beta, const float* S0, void* out, float* S_final,
                        const int* cu_seqlens, int N, int H, int T, int dk, int dv, int C,
                        int mode, int dtype, void* workspace, size_t workspace_bytes,
                        void* stream) {
  g_last_error.clear();
  if (!q || !k || !v || !out || !cu_seqlens)
    return fail(LA_ERR_NULL, "q, k, v, out and cu_seqlens are required");
  if (int e = check_mode_dtype(mode, dtype)) return e;
  if (int e = check_gates(mode, log_alpha, beta)) return e;
  if (int e = check_varlen_shape(N, H, T, dk, dv, C, mode, dtype)) return e;
  size_t n_qk, n_v, n_g, n_s;
  if (!count({H, T, dk}, &n_qk) || !count({H, T, dv}, &n_v) || !count({H, T}, &n_g) ||
      !count({N, H, dk, dv}, &n_s))
    return fail(LA_ERR_SHAPE, "tensor sizes overflow size_t");
  const la::ChunkArgs a = chunk_args(q, k, v, log_alpha, beta, S0, out, S_final, N, H, T, dk,
                                     C, mode, dtype, workspace, cu_seqlens);
  return run_chunk(a, n_qk, n_v, n_g, n_s, dtype, workspace_bytes, (size_t)(N + 1) * 4,
                   stream);
}

int la_decode_step(const void* q, const void* k, const void* v, const float* log_alpha,
                   const float* beta, float* S, void* out, int B, int H, int dk, int dv,
                   int mode, int dtype, void* stream) {
  g_last_error.clear();
  return decode_step(q, k, v, log_alpha, beta, S, out, B, H, dk, dv, mode, dtype, nullptr,
                     stream);
}

int la_decode_step_fused(const void* q, const void* k, const void* v, const float* a_raw,
                         const float* b_raw, float* S, void* out, int B, int H, int dk, int dv,
                         int mode, int dtype, const la_fused_opts_t* opts, void* stream) {
  g_last_error.clear();
  return decode_step(q, k, v, a_raw, b_raw, S, out, B, H, dk, dv, mode, dtype, opts, stream);
}

int la_profile_begin(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = true;
  return LA_OK;
}

int la_profile_end(la_kernel_time_t* out, int capacity, int* count) {
  g_last_error.clear();
  if (!count) return fail(LA_ERR_NULL, "count is required");
  std::vector<TimedLaunch> recs;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_on = false;
    recs.swap(g_prof);
  }
  // Events shared by two records (one kernel's stop is the next one's
  // start) are destroyed once.
  std::map<std::string, std::pair<int, double>> agg;
  std::vector<std::string> order;
  hipError_t err = hipSuccess;
  for (const TimedLaunch& r : recs) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess && err == hipSuccess) err = e;
    auto it = agg.find(r.name);
    if (it == agg.end()) {
      order.push_back(r.name);
      it = agg.emplace(r.name, std::make_pair(0, 0.0)).first;
    }
    it->second.first += 1;
    it->second.second += ms;
  }
  std::vector<hipEvent_t> evs;
  for (const TimedLaunch& r : recs) {
    evs.push_back(r.start);
    evs.push_back(r.stop);
  }
  std::sort(evs.begin(), evs.end());
  evs.erase(std::unique(evs.begin(), evs.end()), evs.end());
  for (hipEvent_t ev : evs) (void)hipEventDestroy(ev);
  int n = 0;
  for (const std::string& name : order) {
    if (out && n < capacity) {
      std::memset(out[n].name, 0, sizeof(out[n].name));
      std::strncpy(out[n].name, name.c_str(), sizeof(out[n].name) - 1);
      out[n].launches = agg[name].first;
      out[n].total_ms = agg[name].second;
    }
    ++n;
  }
  *count = n;
  if (err != hipSuccess) return fail_hip("reading kernel timing events", err);
  return LA_OK;
}

}  // extern "C"
