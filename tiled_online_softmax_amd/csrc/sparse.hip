// Block lists for block-sparse attention.
//
// A block mask keeps or drops whole 128 x 128 blocks of the score matrix (the
// block-sparsity customisation named in the "FlashAttention (Metal Port)"
// README, section "Documentation"). The tile loops do not read the mask
// itself: they walk lists of the blocks that can hold a kept score, built
// here once per mask and reusable by every call with the same mask and
// geometry (the forward and dQ passes walk the key blocks of a query block,
// the key-tile pass the query blocks of a key block).
//
// A block (qb, kb) is listed when its mask byte is non-zero and it meets the
// causal / window band: the band rows i of query block qb keep keys
// [key_lo(i), key_hi(i)], both non-decreasing in i, so the block meets the
// band iff its first key is <= key_hi(last row) and its last key is
// >= key_lo(first row). Lists are in ascending block order.
#include "common.hpp"
#include "launch.hpp"

namespace fa {

// One wave per list: lists 0 .. nqb-1 of a head are the key blocks of query
// block r, lists nqb .. nqb+nkb-1 the query blocks of key block r - nqb.
__global__ void __launch_bounds__(64) block_lists_kernel(BlockListParams P) {
  const int lane = threadIdx.x;
  const int per_head = P.nqb + P.nkb;
  const int bh = (int)blockIdx.x / per_head, r = (int)blockIdx.x - bh * per_head;
  const int b = bh / P.H, h = bh - b * P.H;
  const KeyBounds kb{P.Nq, P.Nk, P.causal, P.window};
  const unsigned char* m = P.mask + b * P.mb + h * P.mh;
  const bool rows = r < P.nqb;  // key blocks of one query block
  const int fixed = rows ? r : r - P.nqb;
  const int n = rows ? P.nkb : P.nqb;
  int* out = rows ? P.kv_index + ((long long)bh * P.nqb + fixed) * P.nkb
                  : P.q_index + ((long long)bh * P.nkb + fixed) * P.nqb;
  int count = 0;
  for (int c0 = 0; c0 < n; c0 += 64) {
    const int x = c0 + lane;
    bool live = false;
    if (x < n) {
      const int qb = rows ? fixed : x, kbk = rows ? x : fixed;
      const int i0 = qb * kBlock, i1 = min(i0 + kBlock, P.Nq) - 1;
      const int j0 = kbk * kBlock, j1 = min(j0 + kBlock, P.Nk) - 1;
      live = m[qb * P.mq + kbk] != 0 && j0 <= kb.hi(i1) && j1 >= kb.lo(i0) && kb.lo(i1) <= kb.hi(i1);
    }
    const unsigned long long bal = __ballot(live);
    const int before = __builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0));
    if (live) out[count + before] = x;
    count += __popcll(bal);
  }
  if (lane == 0) {
    if (rows)
      P.kv_count[(long long)bh * P.nqb + fixed] = count;
    else
      P.q_count[(long long)bh * P.nkb + fixed] = count;
  }
}

hipError_t block_lists_launch(const BlockListParams& p, int B, hipStream_t st) {
  const long long grid = (long long)B * p.H * (p.nqb + p.nkb);
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(block_lists_kernel, dim3((unsigned)grid), dim3(64), 0, st, p);
  return hipGetLastError();
}

}  // namespace fa
