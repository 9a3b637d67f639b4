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
  // Block sparsity: the listed key blocks of each (b, h, query block), or nullptr (dense).
  const int* kv_count;  // [B, H, nqb]
  const int* kv_index;  // [B, H, nqb, nkb], ascending
  int nqb, nkb;
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

// The key tiles (BN keys each) a query tile [q0, q1) of head bh visits,
// j = 0 .. n-1. Dense: the tiles [t_lo, t_end) that hold every key one of its
// rows keeps. SPARSE: the tiles of the key blocks listed for its query block
// q0 / kBlock (ascending); a list count outside [0, nkb] is clamped so that
// list reads stay inside the list.
// Read-only data read at wave-uniform addresses: through the constant address
// space the loads are scalar (s_load) and their results wave-uniform.
typedef __attribute__((address_space(4))) const int* const_int_ptr;

template <bool SPARSE, int BN>
struct KeyTiles {
  static constexpr int TPB = kBlock / BN;  // tiles per block
  const_int_ptr idx;
  int t_lo, n;
  template <class Params>
  __device__ __forceinline__ KeyTiles(const Params& P, int bh, const KeyBounds& kb, int q0, int q1) {
    if constexpr (SPARSE) {
      const long long row = (long long)bh * P.nqb + q0 / kBlock;
      idx = (const_int_ptr)(P.kv_index + row * P.nkb);
      n = min(max(((const_int_ptr)P.kv_count)[row], 0), P.nkb) * TPB;
      t_lo = 0;
    } else {
      idx = nullptr;
      t_lo = kb.lo(q0) / BN;
      n = kb.hi(min(q1, kb.nq) - 1) / BN + 1 - t_lo;
    }
  }
  __device__ __forceinline__ int at(int j) const {
    if constexpr (SPARSE)
      return idx[j / TPB] * TPB + j % TPB;
    else
      return t_lo + j;
  }
  // at(j) for j clamped into [0, n - 1] (0 when there are no tiles): list reads
  // that run ahead of the loop stay inside the list.
  __device__ __forceinline__ int at_clamped(int j) const {
    if constexpr (SPARSE)
      return n > 0 ? at(min(j, n - 1)) : 0;
    else
      return t_lo + j;
  }
  // Tiles [0, live_count(hi)) start at or before key hi.
  __device__ __forceinline__ int live_count(int hi) const {
    if constexpr (SPARSE) {
      int c = n;
      while (c > 0 && at(c - 1) * BN > hi) --c;
      return c;
    } else {
      return min(n, hi / BN + 1 - t_lo);
    }
  }
};

bool fwd_supported(Elt e, int D);
// bf16 forward with O in AGPRs at two waves per SIMD (fwd_lean.hip), D = 256.
hipError_t fwd_lean_dispatch(int D, const FwdParams& p, int B, int H, hipStream_t st);
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
  // Block sparsity (as in FwdParams), plus the listed query blocks of each (b, h, key block).
  const int* kv_count;
  const int* kv_index;
  const int* q_count;  // [B, H, nkb]
  const int* q_index;  // [B, H, nkb, nqb], ascending
  int nqb, nkb;
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

// The query tiles (BQ rows each) the key tile of key block kbk of a K/V head
// visits, head by head of its group (g = 0 .. group-1 is query head h0 + g).
// Dense: tiles [qt0, nq) of every head. SPARSE: the tiles of the query blocks
// listed for key block kbk of each head (ascending), passing over heads whose
// list is empty; list counts are clamped into [0, nqb]. The position (g, j)
// is valid while g < group.
template <bool SPARSE, int BQ>
struct QueryTiles {
  static constexpr int TPB = kBlock / BQ;  // tiles per block
  int g, j, lo, n, group, nqb;
  const_int_ptr cnt, idx;  // head h0's count and list; head h0 + g's are g * cs, g * is further on
  long long cs, is;
  __device__ __forceinline__ QueryTiles(const BwdParams& P, long long bh0, int kbk, int qt0, int nq, int group_)
      : g(0), group(group_), nqb(P.nqb) {
    if constexpr (SPARSE) {
      cnt = (const_int_ptr)(P.q_count + bh0 * P.nkb + kbk);
      idx = (const_int_ptr)(P.q_index + (bh0 * P.nkb + kbk) * P.nqb);
      cs = P.nkb;
      is = (long long)P.nkb * P.nqb;
      lo = j = 0;
      n = head_n(0);
      while (n == 0 && ++g < group) n = head_n(g);
    } else {
      cnt = idx = nullptr;
      cs = is = 0;
      lo = j = qt0;
      n = nq;
      if (qt0 >= nq) g = group;  // nothing to visit
    }
  }
  __device__ __forceinline__ int head_n(int gg) const { return min(max(cnt[gg * cs], 0), nqb) * TPB; }
  __device__ __forceinline__ bool valid() const { return g < group; }
  // first query row of the current tile
  __device__ __forceinline__ int row() const {
    if constexpr (SPARSE)
      return idx[g * is + j / TPB] * kBlock + (j % TPB) * BQ;
    else
      return j * BQ;
  }
  __device__ __forceinline__ void advance() {
    if (++j < n) return;
    j = lo;
    if constexpr (SPARSE) {
      n = 0;
      while (n == 0 && ++g < group) n = head_n(g);
    } else {
      ++g;
    }
  }
};

bool bwd_supported(int D);
// variant: 0 atomic, 1 deterministic, 2 dK/dV only (no dQ). H: query heads.
hipError_t bwd_dispatch(int D, int variant, const BwdParams& p, int B, int H, hipStream_t st);

// Block lists of a block mask (see sparse.hip).
struct BlockListParams {
  const unsigned char* mask;  // element (b, h, qb, kb) at b*mb + h*mh + qb*mq + kb
  long long mb, mh, mq;
  int* kv_count;
  int* kv_index;
  int* q_count;
  int* q_index;
  int H, Nq, Nk, causal, window, nqb, nkb;
};
hipError_t block_lists_launch(const BlockListParams& p, int B, hipStream_t st);

hipError_t quantize_fp8_launch(const float* x, size_t n, void* codes, float* descale, hipStream_t st);

// Sets the calling thread's error message (fa_last_error) and returns `status`.
int api_fail(int status, const char* fmt, ...);

}  // namespace fa
