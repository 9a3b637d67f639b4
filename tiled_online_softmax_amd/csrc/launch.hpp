// Internal interface between the C ABI (api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "common.hpp"

namespace fa {

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const float* q_descale;  // fp8 only; nullptr means 1
  const float* k_descale;
  const float* v_descale;
  int N;               // query rows per head
  int Nk;              // key rows per head
  int causal;          // keep key j for query i only if j <= i + Nk - N (bottom-right diagonal)
  int window;          // >= 0: also only if j >= i + Nk - N - window; < 0: no window
  int hq;              // query heads per batch entry
  int group;           // query heads per K/V head (1: one K/V head per query head)
  int n_qtiles;        // set by the launcher
  float scale_log2;    // scale * log2(e)
  float rescale_log2;  // conditional-rescale threshold (base-2 units)
};

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
  float* ld;        // workspace: [B*H*N] lse * log2(e), then [B*H*N] -rowsum(dO * O) (H query heads)
  long long rows;   // B * H * N
  float* dq_accum;  // [B,H,N,D] float workspace (atomic variant), else nullptr
  int N;             // query rows per head
  int Nk;            // key rows per head
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
