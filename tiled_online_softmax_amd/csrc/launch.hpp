// Internal interface between the C ABI (api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "common.hpp"

namespace fa {

// Element strides of one [B, H, N, D] tensor (D contiguous): row i of head h of
// batch entry b starts at element b*b_ + h*h_ + i*r_. With packed sequences
// (cu_q / cu_k set) b_ is unused and row i of entry b is packed row cu[b] + i.
struct Strides {
  long long b, h, r;
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const float* q_descale;  // fp8 only; nullptr means 1
  const float* k_descale;
  const float* v_descale;
  Strides sq, sk, sv, so;
  long long lse_b, lse_h;  // lse element strides (rows contiguous)
  const int* cu_q;     // packed sequences: device [B+1] row offsets of entry b, or nullptr
  const int* cu_k;
  int total_q, total_k;  // packed rows (bounds for cu_q / cu_k)
  int N;               // query rows per head (packed: the longest sequence)
  int Nk;              // key rows per head (packed: the longest sequence)
  int causal;          // keep key j for query i only if j <= i + Nk - N (bottom-right diagonal)
  int window;          // >= 0: also only if j >= i + Nk - N - window; < 0: no window
  int hq;              // query heads per batch entry
  int group;           // query heads per K/V head (1: one K/V head per query head)
  int n_qtiles;        // set by the launcher
  float scale_log2;    // scale * log2(e)
  float rescale_log2;  // conditional-rescale threshold (base-2 units)
};

// Where one query head of a forward launch and its K/V head live: row 0 of
// each tensor, row strides in bytes, and the entry's lengths.
struct HeadRows {
  const char* q;
  const char* k;
  const char* v;
  char* o;
  float* lse;
  uint32_t qrs, krs, vrs;
  int nq, nk;
};

// bh = b * hq + h over the launch's query heads; K/V head h / group.
template <int ESZ>
__device__ __forceinline__ HeadRows head_rows(const FwdParams& P, int bh) {
  constexpr int OSZ = ESZ == 4 ? 4 : 2;  // O is float for float inputs, else bf16
  const int b = bh / P.hq, h = bh % P.hq, hk = h / P.group;
  const Seq s = seq_of(P.cu_q, P.cu_k, b, P.N, P.Nk, P.total_q, P.total_k);
  const long long bb = P.cu_q ? 0 : b;  // packed sequences start at rows tq / tk instead
  HeadRows r;
  r.q = static_cast<const char*>(P.q) + (bb * P.sq.b + h * P.sq.h + s.tq * P.sq.r) * ESZ;
  r.k = static_cast<const char*>(P.k) + (bb * P.sk.b + hk * P.sk.h + s.tk * P.sk.r) * ESZ;
  r.v = static_cast<const char*>(P.v) + (bb * P.sv.b + hk * P.sv.h + s.tk * P.sv.r) * ESZ;
  r.o = static_cast<char*>(P.o) + (bb * P.so.b + h * P.so.h + s.tq * P.so.r) * OSZ;
  r.lse = P.lse + bb * P.lse_b + h * P.lse_h + s.tq;
  r.qrs = (uint32_t)(P.sq.r * ESZ);
  r.krs = (uint32_t)(P.sk.r * ESZ);
  r.vrs = (uint32_t)(P.sv.r * ESZ);
  r.nq = s.nq;
  r.nk = s.nk;
  return r;
}

bool fwd_supported(Elt e, int D);
// H: query heads; K and V have H / p.group heads.
hipError_t fwd_dispatch(Elt e, int D, const FwdParams& p, int B, int H, hipStream_t st);

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dO;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  Strides sq, sk, sv, so, sdo, sdq, sdk, sdv;
  long long lse_b, lse_h;
  const int* cu_q;   // as in FwdParams
  const int* cu_k;
  int total_q, total_k;
  // Workspace rows: query row i of head h of entry b is row b*ld_b + h*ld_h + i
  // (+ cu_q[b] for packed sequences) of ld (lse * log2(e)), of ld + rows
  // (-rowsum(dO * O)) and of dq_accum (D floats per row).
  float* ld;
  long long rows;
  long long ld_b, ld_h;
  float* dq_accum;  // float workspace (atomic variant), else nullptr
  int n_batch;       // B
  int N;             // query rows per head (packed: the longest sequence)
  int Nk;            // key rows per head (packed: the longest sequence)
  int causal;        // as in FwdParams
  int window;        // as in FwdParams
  int hq;            // query heads per batch entry (H above)
  int group;         // query heads per K/V head
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
};

bool bwd_supported(int D);
// variant: 0 atomic, 1 deterministic, 2 dK/dV only (no dQ). H: query heads.
hipError_t bwd_dispatch(int D, int variant, const BwdParams& p, int B, int H, hipStream_t st);

hipError_t quantize_fp8_launch(const float* x, size_t n, void* codes, float* descale, hipStream_t st);

}  // namespace fa
