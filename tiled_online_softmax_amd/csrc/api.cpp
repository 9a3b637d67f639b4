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
int check_keys(int Nk, int window) {
  if (Nk < 1) return fail(FA_ERR_INVALID_ARG, "Nk must be >= 1 (got %d)", Nk);
  if (window < -1) return fail(FA_ERR_INVALID_ARG, "window must be -1 (none) or >= 0 (got %d)", window);
  return FA_OK;
}

// Where every tensor of a call lives: element strides (batch, head, row; D
// contiguous) and, for packed sequences, the device offset arrays.
struct Layout {
  fa::Strides q, k, v, o, dO, dq, dk, dv;
  long long lse_b, lse_h;
  const int* cu_q = nullptr;
  const int* cu_k = nullptr;
  int total_q = 0, total_k = 0;
  // block lists of a block-sparse call (see fa_block_lists), else null
  const int* kv_count = nullptr;
  const int* kv_index = nullptr;
  const int* q_count = nullptr;
  const int* q_index = nullptr;
};

int blocks(int n) { return (n + fa::kBlock - 1) / fa::kBlock; }

int check_lists(std::initializer_list<const int*> ps) {
  for (const int* p : ps) {
    if (!p) return fail(FA_ERR_INVALID_ARG, "a block-list pointer is NULL");
    if (reinterpret_cast<uintptr_t>(p) & 3u) return fail(FA_ERR_INVALID_ARG, "block-list pointers must be 4-byte aligned");
  }
  return FA_OK;
}

// Contiguous [B, H, Nq, D] queries (and O, dO, dQ), [B, Hkv, Nk, D] keys and values, [B, H, Nq] lse.
Layout contiguous(int H, int Hkv, int Nq, int Nk, int D) {
  Layout L;
  const fa::Strides sq{(long long)H * Nq * D, (long long)Nq * D, D}, sk{(long long)Hkv * Nk * D, (long long)Nk * D, D};
  L.q = L.o = L.dO = L.dq = sq;
  L.k = L.v = L.dk = L.dv = sk;
  L.lse_b = (long long)H * Nq;
  L.lse_h = Nq;
  return L;
}

// Packed sequences: [total_q, H, D] queries, [total_k, Hkv, D] keys and values, lse [H, total_q].
Layout packed(int H, int Hkv, int D, const int* cu_q, const int* cu_k, int total_q, int total_k) {
  Layout L;
  const fa::Strides sq{0, D, (long long)H * D}, sk{0, D, (long long)Hkv * D};
  L.q = L.o = L.dO = L.dq = sq;
  L.k = L.v = L.dk = L.dv = sk;
  L.lse_b = 0;
  L.lse_h = total_q;
  L.cu_q = cu_q;
  L.cu_k = cu_k;
  L.total_q = total_q;
  L.total_k = total_k;
  return L;
}

// Strides: non-negative, rows at least D elements apart, every stride a
// multiple of 16 bytes (loads and stores move 8- and 16-byte pieces of rows).
// Kernels address one head's rows (and, in the backward key pass, a group of
// heads) with 32-bit byte offsets, so each head's extent plus a tile of
// padding rows must stay below 2^31 bytes.
int check_strides(const char* name, const fa::Strides& s, int esz, int D, int n, int heads_spanned) {
  if (s.b < 0 || s.h < 0 || s.r < D)
    return fail(FA_ERR_INVALID_ARG, "%s strides (%lld, %lld, %lld) must be >= 0 with a row stride >= D = %d", name, s.b,
                s.h, s.r, D);
  if ((s.b * esz) % 16 || (s.h * esz) % 16 || (s.r * esz) % 16)
    return fail(FA_ERR_INVALID_ARG, "%s strides (%lld, %lld, %lld) must be multiples of 16 bytes", name, s.b, s.h, s.r);
  const long long extent = ((long long)n + 256) * s.r * esz + (long long)(heads_spanned - 1) * s.h * esz;
  if (extent >= (1LL << 31))
    return fail(FA_ERR_UNSUPPORTED, "%s: one head's rows span %lld bytes; the kernels address < 2^31", name, extent);
  return FA_OK;
}

int check_packed(const Layout& L, int B) {
  if (!L.cu_q) return FA_OK;
  if (!L.cu_k) return fail(FA_ERR_INVALID_ARG, "cu_seqlens_k is NULL");
  if ((reinterpret_cast<uintptr_t>(L.cu_q) | reinterpret_cast<uintptr_t>(L.cu_k)) & 3u)
    return fail(FA_ERR_INVALID_ARG, "cu_seqlens pointers must be 4-byte aligned");
  if (L.total_q < 1 || L.total_k < 1)
    return fail(FA_ERR_INVALID_ARG, "total_q and total_k must be >= 1 (got %d, %d)", L.total_q, L.total_k);
  if (B < 1) return fail(FA_ERR_INVALID_ARG, "B must be >= 1");
  return FA_OK;
}

int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N, int Nk,
             int D, int causal, int window, float scale, int dtype, float rescale_log2, const float* dq,
             const float* dk, const float* dv, const Layout& L, void* stream) {
  const int esz = dtype_bytes(dtype);
  if (!esz) return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (int s = check_common(B, H, N, D, causal, scale, esz)) return s;
  if (int s = check_heads(H, Hkv)) return s;
  if (int s = check_keys(Nk, window)) return s;
  if (!std::isfinite(rescale_log2) || rescale_log2 < 0.f)
    return fail(FA_ERR_INVALID_ARG, "rescale threshold must be finite and >= 0 (got %g)", (double)rescale_log2);
  if (int s = check_ptrs({q, k, v, o, lse})) return s;
  if (int s = check_packed(L, B)) return s;
  const int osz = dtype == FA_F32 ? 4 : 2;
  if (int s = check_strides("q", L.q, esz, D, N, 1)) return s;
  if (int s = check_strides("k", L.k, esz, D, Nk, 1)) return s;
  if (int s = check_strides("v", L.v, esz, D, Nk, 1)) return s;
  if (int s = check_strides("o", L.o, osz, D, N, 1)) return s;
  if (L.lse_b < 0 || L.lse_h < 0) return fail(FA_ERR_INVALID_ARG, "lse strides must be >= 0");
  const fa::Elt e = dtype == FA_F32 ? fa::Elt::F32 : dtype == FA_BF16 ? fa::Elt::BF16 : fa::Elt::FP8;
  if (!fa::fwd_supported(e, D)) return fail(FA_ERR_UNSUPPORTED, "forward: D=%d is not in the parameter table for dtype %d", D, dtype);
  fa::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.q_descale = dq; p.k_descale = dk; p.v_descale = dv;
  p.sq = L.q; p.sk = L.k; p.sv = L.v; p.so = L.o;
  p.lse_b = L.lse_b; p.lse_h = L.lse_h;
  p.cu_q = L.cu_q; p.cu_k = L.cu_k; p.total_q = L.total_q; p.total_k = L.total_k;
  p.kv_count = L.kv_count; p.kv_index = L.kv_index; p.nqb = blocks(N); p.nkb = blocks(Nk);
  p.N = N; p.Nk = Nk; p.causal = causal; p.window = window;
  p.hq = H; p.group = H / Hkv;
  p.scale_log2 = scale * fa::kLog2e;
  p.rescale_log2 = rescale_log2;
  return hip_status(fa::fwd_dispatch(e, D, p, B, H, reinterpret_cast<hipStream_t>(stream)), "fa_fwd launch");
}

// Descale pointers are optional (NULL reads as 1.0) and read by the kernel as floats.
int check_descales(const float* q_descale, const float* k_descale, const float* v_descale) {
  for (const float* d : {q_descale, k_descale, v_descale})
    if (d && (reinterpret_cast<uintptr_t>(d) & 3u)) return fail(FA_ERR_INVALID_ARG, "descale pointer not 4-byte aligned");
  return FA_OK;
}

Layout strides_from(const long long* st, int n_tensors) {
  Layout L{};
  fa::Strides* t[] = {&L.q, &L.k, &L.v, &L.o, &L.dO, &L.dq, &L.dk, &L.dv};
  for (int i = 0; i < n_tensors; ++i) *t[i] = fa::Strides{st[3 * i], st[3 * i + 1], st[3 * i + 2]};
  L.lse_b = st[3 * n_tensors];
  L.lse_h = st[3 * n_tensors + 1];
  return L;
}

}  // namespace

int fa::api_fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int D, int causal,
           float scale, int dtype, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, H, N, N, D, causal, -1, scale, dtype, 8.0f, nullptr, nullptr, nullptr,
                  contiguous(H, H, N, N, D), stream);
}

int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N, int D,
               int causal, float scale, int dtype, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, Hkv, N, N, D, causal, -1, scale, dtype, 8.0f, nullptr, nullptr, nullptr,
                  contiguous(H, Hkv, N, N, D), stream);
}

int fa_fwd_general(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int Nq,
                   int Nk, int D, int causal, int window, float scale, int dtype, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, Hkv, Nq, Nk, D, causal, window, scale, dtype, 8.0f, nullptr, nullptr,
                  nullptr, contiguous(H, Hkv, Nq, Nk, D), stream);
}

int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int Nq,
                   int Nk, int D, int causal, int window, float scale, int dtype, const long long* strides,
                   void* stream) {
  if (!strides) return fail(FA_ERR_INVALID_ARG, "strides is NULL");
  return fwd_impl(q, k, v, o, lse, B, H, Hkv, Nq, Nk, D, causal, window, scale, dtype, 8.0f, nullptr, nullptr,
                  nullptr, strides_from(strides, 4), stream);
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_seqlens_q,
                  const int* cu_seqlens_k, int B, int H, int Hkv, int total_q, int total_k, int max_seqlen_q,
                  int max_seqlen_k, int D, int causal, int window, float scale, int dtype, void* stream) {
  if (!cu_seqlens_q) return fail(FA_ERR_INVALID_ARG, "cu_seqlens_q is NULL");
  return fwd_impl(q, k, v, o, lse, B, H, Hkv, max_seqlen_q, max_seqlen_k, D, causal, window, scale, dtype, 8.0f,
                  nullptr, nullptr, nullptr, packed(H, Hkv, D, cu_seqlens_q, cu_seqlens_k, total_q, total_k), stream);
}

int fa_block_lists(const void* mask, const long long* mask_strides, int B, int H, int Nq, int Nk, int causal,
                   int window, int* kv_count, int* kv_index, int* q_count, int* q_index, void* stream) {
  if (!mask) return fail(FA_ERR_INVALID_ARG, "mask is NULL");
  if (!mask_strides) return fail(FA_ERR_INVALID_ARG, "mask_strides is NULL");
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return fail(FA_ERR_INVALID_ARG, "B, H, Nq, Nk must be >= 1");
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
  if (window < -1) return fail(FA_ERR_INVALID_ARG, "window must be -1 (none) or >= 0 (got %d)", window);
  for (int i = 0; i < 3; ++i)
    if (mask_strides[i] < 0) return fail(FA_ERR_INVALID_ARG, "mask strides must be >= 0");
  if (int s = check_lists({kv_count, kv_index, q_count, q_index})) return s;
  if ((long long)B * H * blocks(Nq) * blocks(Nk) >= (1LL << 31))
    return fail(FA_ERR_UNSUPPORTED, "block lists of %lld entries exceed 2^31", (long long)B * H * blocks(Nq) * blocks(Nk));
  fa::BlockListParams p{};
  p.mask = static_cast<const unsigned char*>(mask);
  p.mb = mask_strides[0]; p.mh = mask_strides[1]; p.mq = mask_strides[2];
  p.kv_count = kv_count; p.kv_index = kv_index; p.q_count = q_count; p.q_index = q_index;
  p.H = H; p.Nq = Nq; p.Nk = Nk; p.causal = causal; p.window = window;
  p.nqb = blocks(Nq); p.nkb = blocks(Nk);
  return hip_status(fa::block_lists_launch(p, B, reinterpret_cast<hipStream_t>(stream)), "fa_block_lists launch");
}

int fa_fwd_sparse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int Nq,
                  int Nk, int D, int causal, int window, float scale, int dtype, const int* kv_count,
                  const int* kv_index, void* stream) {
  if (int s = check_lists({kv_count, kv_index})) return s;
  Layout L = contiguous(H, Hkv, Nq, Nk, D);
  L.kv_count = kv_count;
  L.kv_index = kv_index;
  return fwd_impl(q, k, v, o, lse, B, H, Hkv, Nq, Nk, D, causal, window, scale, dtype, 8.0f, nullptr, nullptr,
                  nullptr, L, stream);
}

int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int D,
              int causal, float scale, int dtype, float rescale_log2, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, H, N, N, D, causal, -1, scale, dtype, rescale_log2, nullptr, nullptr,
                  nullptr, contiguous(H, H, N, N, D), stream);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int D,
               int causal, float scale, const float* q_descale, const float* k_descale, const float* v_descale,
               void* stream) {
  return fa_fwd_fp8_general(q, k, v, o, lse, B, H, H, N, N, D, causal, -1, scale, q_descale, k_descale, v_descale,
                            stream);
}

int fa_fwd_fp8_general(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv,
                       int Nq, int Nk, int D, int causal, int window, float scale, const float* q_descale,
                       const float* k_descale, const float* v_descale, void* stream) {
  if (int s = check_descales(q_descale, k_descale, v_descale)) return s;
  return fwd_impl(q, k, v, o, lse, B, H, Hkv, Nq, Nk, D, causal, window, scale, FA_FP8_E4M3, 0.0f, q_descale,
                  k_descale, v_descale, contiguous(H, Hkv, Nq, Nk, D), stream);
}

int fa_fwd_fp8_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_seqlens_q,
                      const int* cu_seqlens_k, int B, int H, int Hkv, int total_q, int total_k, int max_seqlen_q,
                      int max_seqlen_k, int D, int causal, int window, float scale, const float* q_descale,
                      const float* k_descale, const float* v_descale, void* stream) {
  if (!cu_seqlens_q) return fail(FA_ERR_INVALID_ARG, "cu_seqlens_q is NULL");
  if (int s = check_descales(q_descale, k_descale, v_descale)) return s;
  return fwd_impl(q, k, v, o, lse, B, H, Hkv, max_seqlen_q, max_seqlen_k, D, causal, window, scale, FA_FP8_E4M3,
                  0.0f, q_descale, k_descale, v_descale,
                  packed(H, Hkv, D, cu_seqlens_q, cu_seqlens_k, total_q, total_k), stream);
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
             int dtype, int variant, void* workspace, size_t workspace_bytes, const Layout& L, void* stream) {
  if (dtype != FA_BF16) {
    if (!dtype_bytes(dtype)) return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    return fail(FA_ERR_UNSUPPORTED, "backward is built for FA_BF16 only (got dtype %d)", dtype);
  }
  if (int s = check_common(B, H, N, D, causal, scale, 2)) return s;
  if (int s = check_heads(H, Hkv)) return s;
  if (int s = check_keys(Nk, window)) return s;
  if (variant != FA_BWD_ATOMIC && variant != FA_BWD_DETERMINISTIC && variant != 2)
    return fail(FA_ERR_INVALID_ARG, "variant must be FA_BWD_ATOMIC or FA_BWD_DETERMINISTIC (got %d)", variant);
  if (variant == 2) {
    if (int s = check_ptrs({q, k, v, o, dO, lse, dk, dv, workspace})) return s;
  } else {
    if (int s = check_ptrs({q, k, v, o, dO, lse, dq, dk, dv, workspace})) return s;
  }
  if (int s = check_packed(L, B)) return s;
  const int group = H / Hkv;
  // the key pass reads the Q and dO rows of a whole group of query heads through one buffer resource
  if (int s = check_strides("q", L.q, 2, D, N, group)) return s;
  if (int s = check_strides("dO", L.dO, 2, D, N, group)) return s;
  if (int s = check_strides("k", L.k, 2, D, Nk, 1)) return s;
  if (int s = check_strides("v", L.v, 2, D, Nk, 1)) return s;
  if (int s = check_strides("o", L.o, 2, D, N, 1)) return s;
  if (int s = check_strides("dq", L.dq, 2, D, N, 1)) return s;
  if (int s = check_strides("dk", L.dk, 2, D, Nk, 1)) return s;
  if (int s = check_strides("dv", L.dv, 2, D, Nk, 1)) return s;
  if (L.lse_b < 0 || L.lse_h < 0) return fail(FA_ERR_INVALID_ARG, "lse strides must be >= 0");
  if (!fa::bwd_supported(D)) return fail(FA_ERR_UNSUPPORTED, "backward: D=%d is not in the parameter table", D);
  // workspace rows: B entries of N rows per head, or the packed rows of every head
  const int Bp = L.cu_q ? 1 : B, Np = L.cu_q ? L.total_q : N;
  if ((unsigned long long)Bp * H * Np * 8ULL >= (1ULL << 32))
    return fail(FA_ERR_UNSUPPORTED, "backward: %lld query rows exceed the 2^29 rows one call supports", (long long)Bp * H * Np);
  const size_t need = fa_bwd_workspace_size(Bp, H, Np, D, dtype, variant == 2 ? FA_BWD_DETERMINISTIC : variant);
  if (workspace_bytes < need) return fail(FA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  fa::BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.dO = dO; p.lse = lse;
  p.dq = dq; p.dk = dk; p.dv = dv;
  p.sq = L.q; p.sk = L.k; p.sv = L.v; p.so = L.o; p.sdo = L.dO; p.sdq = L.dq; p.sdk = L.dk; p.sdv = L.dv;
  p.lse_b = L.lse_b; p.lse_h = L.lse_h;
  p.cu_q = L.cu_q; p.cu_k = L.cu_k; p.total_q = L.total_q; p.total_k = L.total_k;
  p.kv_count = L.kv_count; p.kv_index = L.kv_index; p.q_count = L.q_count; p.q_index = L.q_index;
  p.nqb = blocks(N); p.nkb = blocks(Nk);
  p.ld = reinterpret_cast<float*>(workspace);
  const size_t rows = (size_t)Bp * H * Np;
  p.dq_accum = variant == FA_BWD_ATOMIC
                   ? reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + ((rows * 2 * sizeof(float) + 255) & ~(size_t)255))
                   : nullptr;
  p.rows = (long long)rows;
  p.ld_b = L.cu_q ? 0 : (long long)H * N;
  p.ld_h = Np;
  p.n_batch = B;
  p.N = N; p.Nk = Nk; p.causal = causal; p.window = window;
  p.scale = scale; p.scale_log2 = scale * fa::kLog2e;
  p.hq = H; p.group = group;
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
                  workspace_bytes, contiguous(H, H, N, N, D), stream);
}

int fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse, void* dq,
               void* dk, void* dv, int B, int H, int Hkv, int N, int D, int causal, float scale, int dtype,
               int variant, void* workspace, size_t workspace_bytes, void* stream) {
  if (variant != FA_BWD_ATOMIC && variant != FA_BWD_DETERMINISTIC)
    return fail(FA_ERR_INVALID_ARG, "variant must be FA_BWD_ATOMIC or FA_BWD_DETERMINISTIC (got %d)", variant);
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, B, H, Hkv, N, N, D, causal, -1, scale, dtype, variant, workspace,
                  workspace_bytes, contiguous(H, Hkv, N, N, D), stream);
}

int fa_bwd_general(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                   void* dq, void* dk, void* dv, int B, int H, int Hkv, int Nq, int Nk, int D, int causal, int window,
                   float scale, int dtype, int variant, void* workspace, size_t workspace_bytes, void* stream) {
  if (variant != FA_BWD_ATOMIC && variant != FA_BWD_DETERMINISTIC)
    return fail(FA_ERR_INVALID_ARG, "variant must be FA_BWD_ATOMIC or FA_BWD_DETERMINISTIC (got %d)", variant);
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, B, H, Hkv, Nq, Nk, D, causal, window, scale, dtype, variant,
                  workspace, workspace_bytes, contiguous(H, Hkv, Nq, Nk, D), stream);
}

int fa_bwd_strided(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                   void* dq, void* dk, void* dv, int B, int H, int Hkv, int Nq, int Nk, int D, int causal, int window,
                   float scale, int dtype, int variant, void* workspace, size_t workspace_bytes,
                   const long long* strides, void* stream) {
  if (variant != FA_BWD_ATOMIC && variant != FA_BWD_DETERMINISTIC)
    return fail(FA_ERR_INVALID_ARG, "variant must be FA_BWD_ATOMIC or FA_BWD_DETERMINISTIC (got %d)", variant);
  if (!strides) return fail(FA_ERR_INVALID_ARG, "strides is NULL");
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, B, H, Hkv, Nq, Nk, D, causal, window, scale, dtype, variant,
                  workspace, workspace_bytes, strides_from(strides, 8), stream);
}

int fa_bwd_sparse(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                  void* dq, void* dk, void* dv, int B, int H, int Hkv, int Nq, int Nk, int D, int causal, int window,
                  float scale, int dtype, int variant, const int* kv_count, const int* kv_index, const int* q_count,
                  const int* q_index, void* workspace, size_t workspace_bytes, void* stream) {
  if (variant != FA_BWD_ATOMIC && variant != FA_BWD_DETERMINISTIC)
    return fail(FA_ERR_INVALID_ARG, "variant must be FA_BWD_ATOMIC or FA_BWD_DETERMINISTIC (got %d)", variant);
  if (int s = check_lists({kv_count, kv_index, q_count, q_index})) return s;
  Layout L = contiguous(H, Hkv, Nq, Nk, D);
  L.kv_count = kv_count;
  L.kv_index = kv_index;
  L.q_count = q_count;
  L.q_index = q_index;
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, B, H, Hkv, Nq, Nk, D, causal, window, scale, dtype, variant,
                  workspace, workspace_bytes, L, stream);
}

int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                  void* dq, void* dk, void* dv, const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int H,
                  int Hkv, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int D, int causal,
                  int window, float scale, int dtype, int variant, void* workspace, size_t workspace_bytes,
                  void* stream) {
  if (variant != FA_BWD_ATOMIC && variant != FA_BWD_DETERMINISTIC)
    return fail(FA_ERR_INVALID_ARG, "variant must be FA_BWD_ATOMIC or FA_BWD_DETERMINISTIC (got %d)", variant);
  if (!cu_seqlens_q) return fail(FA_ERR_INVALID_ARG, "cu_seqlens_q is NULL");
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, B, H, Hkv, max_seqlen_q, max_seqlen_k, D, causal, window, scale,
                  dtype, variant, workspace, workspace_bytes,
                  packed(H, Hkv, D, cu_seqlens_q, cu_seqlens_k, total_q, total_k), stream);
}

int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                void* dk, void* dv, int B, int H, int N, int D, int causal, float scale, int dtype, void* workspace,
                size_t workspace_bytes, void* stream) {
  return bwd_impl(q, k, v, o, dO, lse, nullptr, dk, dv, B, H, H, N, N, D, causal, -1, scale, dtype, 2, workspace,
                  workspace_bytes, contiguous(H, H, N, N, D), stream);
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
