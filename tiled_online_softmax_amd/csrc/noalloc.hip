// fa_bwd_noalloc: the backward of fa_bwd with its workspace in a static
// device array instead of a caller-provided buffer, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The array lives in this library's code object; the HIP runtime places one
// copy on every device the library is loaded on, at load time, and keeps it
// until the process ends. Host code never uses the array's name as an address
// (on the host it names a stand-in, not device memory): the first call on a
// device looks the device copy up with hipGetSymbolAddress and keeps that
// pointer per device; every kernel then gets the pointer, exactly as it gets a
// caller's workspace from fa_bwd.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../../include/fa.h"
#include "launch.hpp"

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;  // FA_NOALLOC_SCRATCH_BYTES in include/fa.h
static_assert(kScratchBytes == FA_NOALLOC_SCRATCH_BYTES, "header and library agree on the scratch size");

__device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The device copy of `scratch` on the current device (looked up once per device).
hipError_t scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                              const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int D, int causal,
                              float scale, int dtype, int variant, void* stream) {
  // Validate every argument first, before any HIP call: fa_bwd with a stand-in workspace of
  // 0 bytes runs all of its checks and, when they pass, refuses the workspace size -- it never
  // dereferences the pointer or launches anything. Its other errors are the caller's.
  void* const stand_in = reinterpret_cast<void*>(static_cast<uintptr_t>(256));
  const int s = fa_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, D, causal, scale, dtype, variant, stand_in, 0,
                       stream);
  if (s != FA_ERR_WORKSPACE) return s;
  const size_t need = fa_bwd_workspace_size(B, H, N, D, dtype, variant);
  if (need > kScratchBytes)
    return fa::api_fail(FA_ERR_WORKSPACE,
                        "fa_bwd_noalloc: this problem needs %zu bytes of workspace; the static scratch holds %zu "
                        "(use fa_bwd with a caller-provided workspace)",
                        need, kScratchBytes);
  void* ws = nullptr;
  const hipError_t e = scratch_ptr(&ws);
  if (e != hipSuccess) return fa::api_fail(FA_ERR_HIP, "fa_bwd_noalloc: scratch lookup: %s", hipGetErrorString(e));
  return fa_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, D, causal, scale, dtype, variant, ws, kScratchBytes, stream);
}
