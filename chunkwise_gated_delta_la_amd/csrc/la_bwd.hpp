// Internal interface of the backward (la_bwd.hip) for the C-ABI host layer.
// Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace la {

// Backward of the chunkwise forward.
//
// Gradients of sum(dO * O) + sum(dS_final * S_final) with respect to q, k,
// v, log alpha, beta and S0, fixed-length layout [B, H, L, d], any L.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* log_alpha;
  const float* beta;
  const float* S0;        // NULL: zero
  const void* dout;       // [B, H, L, dv], the input type
  const float* dS_final;  // NULL: zero
  float* dq;
  float* dk;
  float* dv;
  float* dlog_alpha;      // gated modes
  float* dbeta;           // erase modes
  float* dS0;             // NULL: not written
  int B, H, L, d, mode;   // packed batch: B sequences, L tokens in all
  bool in_bf16;
  void* workspace;        // bwd_workspace_bytes(*this) bytes, 16-byte aligned
  // Packed variable-length batch: cu_seqlens [B + 1] on the device, tokens
  // [H, L, d], gates [H, L], states [B, H, d, d]; NULL: fixed length
  // [B, H, L, d].
  const int* cu = nullptr;
  bool packed = false;    // size the workspace for a packed batch (cu may be NULL then)
  // Inverse norms of the q and k rows [rows, as the gates] (the fused
  // prologue's normalisation): q and k are then the raw rows, and every
  // product that reads them scales by these per row; NULL: q and k as given.
  const float* rq = nullptr;
  const float* rk = nullptr;
};

size_t bwd_workspace_bytes(const BwdArgs& a);
// The four launches in order: per-chunk prep (decays, T, and the
// dS-independent products P^T dO and Q^T diag(gam) dO), the forward walk
// (chunk entry states, U), the reverse walk (state gradients, dR, dv), the
// per-chunk gradients (dq, dk, dbeta, dlog alpha).
hipError_t launch_bwd_prep(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_states(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_rev(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_grads(const BwdArgs& a, hipStream_t st);


// The fused prologue around the backward (la_chunk_bwd_fused): per token
// row, the inverse norms of q and k and the activated gates (grad = false;
// the backward then reads the raw q and k with those norms, BwdArgs::rq,
// rk); after the backward, the chain rule back to the raw inputs, in place
// on the gradients (grad = true).
struct BwdProArgs {
  const void* q;          // raw q, k [rows, d], the input type
  const void* k;
  const float* a_raw;     // raw gate scores [rows]
  const float* b_raw;
  float* rq;              // inverse norms [rows] (written)
  float* rk;
  float* la;              // -scale softplus(a), sigmoid(b) [rows] (written)
  float* be;
  float* dq;              // gradients, transformed in place
  float* dk;
  float* da;
  float* db;
  size_t rows;
  int d;
  bool in_bf16;
  int norm, gates_a, gates_b;
  float scale;
};
hipError_t launch_bwd_pro(const BwdProArgs& p, bool grad, hipStream_t st);

}  // namespace la
