// The C ABI of libfa (declared in include/fa.h): argument validation, status
// codes, the per-thread error string, and dispatch to the kernel launchers.
// Validation never touches the HIP runtime, so it can be exercised on a host
// without a GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "../../include/fa.h"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return FA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int dtype_bytes(int dtype) {
  switch (dtype) {
    case FA_F32: return 4;
    case FA_BF16: return 2;
    case FA_FP8_E4M3: return 1;
    default: return 0;
  }
}

// Checks shared by every attention entry point.
int check_common(int B, int H, int N, int D, int causal, float scale, int esz) {
  if (B < 1 || H < 1 || N < 1 || D < 1) return fail(FA_ERR_INVALID_ARG, "B, H, N, D must be >= 1 (got %d, %d, %d, %d)", B, H, N, D);
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(FA_ERR_INVALID_ARG, "scale must be finite and > 0 (got %g)", (double)scale);
  if ((long long)N * D * esz >= (1LL << 31)) return fail(FA_ERR_INVALID_ARG, "one head (N*D*elem = %lld bytes) must be < 2^31 bytes", (long long)N * D * esz);
  if ((long long)B * H * N >= (1LL << 40)) return fail(FA_ERR_INVALID_ARG, "B*H*N too large");
  return FA_OK;
}

int check_ptrs(std::initializer_list<const void*> ps) {
  int i = 0;
  for (const void* p : ps) {
    if (!p) return fail(FA_ERR_INVALID_ARG, "pointer argument %d is NULL", i);
    if (!aligned16(p)) return fail(FA_ERR_INVALID_ARG, "pointer argument %d is not 16-byte aligned", i);
    ++i;
  }
  return FA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(FA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Query heads H, K/V heads Hkv: H must be a multiple of Hkv.
int check_heads(int H, int Hkv) {
  if (Hkv < 1 || Hkv > H || H % Hkv != 0)
    return fail(FA_ERR_INVALID_ARG, "K/V heads must divide the query heads (H=%d, Hkv=%d)", H, Hkv);
  return FA_OK;
}

// Key length Nk (queries N) and the left window: checks shared by the forward and backward.
int check_keys(int N, int Nk, int D, int causal, int window, int esz) {
  if (Nk < 1) return fail(FA_ERR_INVALID_ARG, "Nk must be >= 1 (got %d)", Nk);
  if ((long long)Nk * D * esz >= (1LL << 31)) return fail(FA_ERR_INVALID_ARG, "one K/V head (Nk*D*elem = %lld bytes) must be < 2^31 bytes", (long long)Nk * D * esz);
  if (causal && Nk < N) return fail(FA_ERR_INVALID_ARG, "causal attention needs Nk >= Nq (got Nq=%d, Nk=%d): the first rows would keep no key", N, Nk);
  if (window < -1) return fail(FA_ERR_INVALID_ARG, "window must be -1 (none) or >= 0 (got %d)", window);
  return FA_OK;
}

int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N, int Nk,
             int D, int causal, int window, float scale, int dtype, float rescale_log2, const float* dq,
             const float* dk, const float* dv, void* stream) {
  const int esz = dtype_bytes(dtype);
  if (!esz) return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (int s = check_common(B, H, N, D, causal, scale, esz)) return s;
  if (int s = check_heads(H, Hkv)) return s;
  if (int s = check_keys(N, Nk, D, causal, window, esz)) return s;
  if (!std::isfinite(rescale_log2) || rescale_log2 < 0.f)
    return fail(FA_ERR_INVALID_ARG, "rescale threshold must be finite and >= 0 (got %g)", (double)rescale_log2);
  if (int s = check_ptrs({q, k, v, o, lse})) return s;
  const fa::Elt e = dtype == FA_F32 ? fa::Elt::F32 : dtype == FA_BF16 ? fa::Elt::BF16 : fa::Elt::FP8;
  if (!fa::fwd_supported(e, D)) return fail(FA_ERR_UNSUPPORTED, "forward: D=%d is not in the parameter table for dtype %d", D, dtype);
  fa::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.q_descale = dq; p.k_descale = dk; p.v_descale = dv;
  p.N = N; p.Nk = Nk; p.causal = causal; p.window = window;
  p.hq = H; p.group = H / Hkv;
  p.scale_log2 = scale * fa::kLog2e;
  p.rescale_log2 = rescale_log2;
  return hip_status(fa::fwd_dispatch(e, D, p, B, H, reinterpret_cast<hipStream_t>(stream)), "fa_fwd launch");
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int D, int causal,
           float scale, int dtype, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, H, N, N, D, causal, -1, scale, dtype, 8.0f, nullptr, nullptr, nullptr,
                  stream);
}

int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N, int D,
               int causal, float scale, int dtype, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, Hkv, N, N, D, causal, -1, scale, dtype, 8.0f, nullptr, nullptr, nullptr,
                  stream);
}

int fa_fwd_general(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int Nq,
                   int Nk, int D, int causal, int window, float scale, int dtype, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, Hkv, Nq, Nk, D, causal, window, scale, dtype, 8.0f, nullptr, nullptr,
                  nullptr, stream);
}

int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int D,
              int causal, float scale, int dtype, float rescale_log2, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, H, N, N, D, causal, -1, scale, dtype, rescale_log2, nullptr, nullptr,
                  nullptr, stream);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int D,
               int causal, float scale, const float* q_descale, const float* k_descale, const float* v_descale,
               void* stream) {
  for (const float* d : {q_descale, k_descale, v_descale})
    if (d && (reinterpret_cast<uintptr_t>(d) & 3u)) return fail(FA_ERR_INVALID_ARG, "descale pointer not 4-byte aligned");
  return fwd_impl(q, k, v, o, lse, B, H, H, N, N, D, causal, -1, scale, FA_FP8_E4M3, 0.0f, q_descale, k_descale,
                  v_descale, stream);
}

int fa_quantize_fp8(const float* x, size_t n, void* codes, float* descale, void* stream) {
  if (n < 1 || n >= (1ULL << 40)) return fail(FA_ERR_INVALID_ARG, "n must be in [1, 2^40) (got %zu)", n);
  if (int s = check_ptrs({x, codes})) return s;
  if (!descale || (reinterpret_cast<uintptr_t>(descale) & 3u)) return fail(FA_ERR_INVALID_ARG, "descale must be a non-NULL 4-byte aligned pointer");
  return hip_status(fa::quantize_fp8_launch(x, n, codes, descale, reinterpret_cast<hipStream_t>(stream)),
                    "fa_quantize_fp8 launch");
}

size_t fa_bwd_workspace_size(int B, int H, int N, int D, int dtype, int variant) {
  if (B < 1 || H < 1 || N < 1 || D < 1 || dtype != FA_BF16) return 0;
  if (variant != FA_BWD_ATOMIC && variant != FA_BWD_DETERMINISTIC) return 0;
  const size_t rows = (size_t)B * H * N;
  size_t bytes = (rows * 2 * sizeof(float) + 255) & ~(size_t)255;
  if (variant == FA_BWD_ATOMIC) bytes += rows * (size_t)D * sizeof(float);
  return bytes;
}

}  // extern "C"

namespace {

// Shared by fa_bwd and fa_bwd_dkdv; variant 2 is the dK/dV-only pass.
int bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse, void* dq,
             void* dk, void* dv, int B, int H, int Hkv, int N, int Nk, int D, int causal, int window, float scale,
             int dtype, int variant, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != FA_BF16) {
    if (!dtype_bytes(dtype)) return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    return fail(FA_ERR_UNSUPPORTED, "backward is built for FA_BF16 only (got dtype %d)", dtype);
  }
  if (int s = check_common(B, H, N, D, causal, scale, 2)) return s;
  if (int s = check_heads(H, Hkv)) return s;
  if (int s = check_keys(N, Nk, D, causal, window, 2)) return s;
  if ((long long)(H / Hkv) * N * D * 2 >= (1LL << 32))
    return fail(FA_ERR_UNSUPPORTED, "backward: the %d query heads sharing a K/V head must span < 2^32 bytes", H / Hkv);
  if (variant != FA_BWD_ATOMIC && variant != FA_BWD_DETERMINISTIC && variant != 2)
    return fail(FA_ERR_INVALID_ARG, "variant must be FA_BWD_ATOMIC or FA_BWD_DETERMINISTIC (got %d)", variant);
  if (variant == 2) {
    if (int s = check_ptrs({q, k, v, o, dO, lse, dk, dv, workspace})) return s;
  } else {
    if (int s = check_ptrs({q, k, v, o, dO, lse, dq, dk, dv, workspace})) return s;
  }
  if (!fa::bwd_supported(D)) return fail(FA_ERR_UNSUPPORTED, "backward: D=%d is not in the parameter table", D);
  if ((unsigned long long)B * H * N * 8ULL >= (1ULL << 32))
    return fail(FA_ERR_UNSUPPORTED, "backward: B*H*N = %lld rows exceeds the 2^29 rows one call supports", (long long)B * H * N);
  const size_t need = fa_bwd_workspace_size(B, H, N, D, dtype, variant == 2 ? FA_BWD_DETERMINISTIC : variant);
  if (workspace_bytes < need) return fail(FA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  fa::BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.dO = dO; p.lse = lse;
  p.dq = dq; p.dk = dk; p.dv = dv;
  p.ld = reinterpret_cast<float*>(workspace);
  const size_t rows = (size_t)B * H * N;
  p.dq_accum = variant == FA_BWD_ATOMIC
                   ? reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + ((rows * 2 * sizeof(float) + 255) & ~(size_t)255))
                   : nullptr;
  p.N = N; p.Nk = Nk; p.causal = causal; p.window = window;
  p.scale = scale; p.scale_log2 = scale * fa::kLog2e;
  p.hq = H; p.group = H / Hkv;
  p.rows = (long long)rows;
  return hip_status(fa::bwd_dispatch(D, variant, p, B, H, reinterpret_cast<hipStream_t>(stream)), "fa_bwd launch");
}

}  // namespace

extern "C" {

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse, void* dq,
           void* dk, void* dv, int B, int H, int N, int D, int causal, float scale, int dtype, int variant,
           void* workspace, size_t workspace_bytes, void* stream) {
  if (variant != FA_BWD_ATOMIC && variant != FA_BWD_DETERMINISTIC)
    return fail(FA_ERR_INVALID_ARG, "variant must be FA_BWD_ATOMIC or FA_BWD_DETERMINISTIC (got %d)", variant);
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, B, H, H, N, N, D, causal, -1, scale, dtype, variant, workspace,
                  workspace_bytes, stream);
}

int fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse, void* dq,
               void* dk, void* dv, int B, int H, int Hkv, int N, int D, int causal, float scale, int dtype,
               int variant, void* workspace, size_t workspace_bytes, void* stream) {
  if (variant != FA_BWD_ATOMIC && variant != FA_BWD_DETERMINISTIC)
    return fail(FA_ERR_INVALID_ARG, "variant must be FA_BWD_ATOMIC or FA_BWD_DETERMINISTIC (got %d)", variant);
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, B, H, Hkv, N, N, D, causal, -1, scale, dtype, variant, workspace,
                  workspace_bytes, stream);
}

int fa_bwd_general(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                   void* dq, void* dk, void* dv, int B, int H, int Hkv, int Nq, int Nk, int D, int causal, int window,
                   float scale, int dtype, int variant, void* workspace, size_t workspace_bytes, void* stream) {
  if (variant != FA_BWD_ATOMIC && variant != FA_BWD_DETERMINISTIC)
    return fail(FA_ERR_INVALID_ARG, "variant must be FA_BWD_ATOMIC or FA_BWD_DETERMINISTIC (got %d)", variant);
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, B, H, Hkv, Nq, Nk, D, causal, window, scale, dtype, variant,
                  workspace, workspace_bytes, stream);
}

int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                void* dk, void* dv, int B, int H, int N, int D, int causal, float scale, int dtype, void* workspace,
                size_t workspace_bytes, void* stream) {
  return bwd_impl(q, k, v, o, dO, lse, nullptr, dk, dv, B, H, H, N, N, D, causal, -1, scale, dtype, 2, workspace,
                  workspace_bytes, stream);
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    default: return "FA_UNKNOWN_STATUS";
  }
}

const char* fa_last_error(void) { return g_err; }

}  // extern "C"
