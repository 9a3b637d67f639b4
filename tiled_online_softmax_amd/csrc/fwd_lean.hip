// bf16 forward at D = 256 with the output accumulators in AGPRs (gfx950).
//
// Each wave owns 32 query rows, as in the other forward kernels, and walks
// 32-key tiles without carrying scores across tiles, so few values are live
// besides Q (32 x 256 bf16, 64 VGPRs) and the O accumulator (32 x 256 float,
// 128 registers). O sits in the AGPR half of the register file -- the P.V
// MFMAs accumulate there -- and everything the softmax touches sits in VGPRs.
// A function that uses AGPRs gets half of its register budget as AGPRs, and at
// two waves per SIMD that is 128 of each: O fills the AGPRs and the rest fits
// the VGPRs. The software-pipelined kernel, with 64-key tiles and two score
// tiles in flight, needs about 450 registers and runs one wave per SIMD; two
// waves let one wave's softmax and LDS reads overlap the other's MFMAs.
//
// The compiler does not keep such a split by itself, so the MFMAs are inline
// asm with explicit operand classes. It then tracks neither their results nor
// the VALU writes they read, and the wait states the ISA requires are explicit:
//   * a VALU write of a VGPR needs 2 wait states before an MFMA reads it: the
//     first P.V MFMA of a 16-key chunk, which reads P just packed by VALU
//     instructions, starts with s_nop 1 (the later ones of the chunk read the
//     same P after the earlier MFMAs have issued);
//   * an MFMA result needs up to 19 wait states (16 passes + 3) before a VALU
//     instruction (or v_accvgpr_read) reads or overwrites it: settle() issues
//     20 and ties the result registers to that point -- before the softmax
//     reads the scores, before a rescale and before the epilogue read O;
//   * an MFMA accumulating onto the previous MFMA's result (the same registers
//     as srcC and vdst) needs none; a score chain starts from the inline
//     constant 0 as srcC rather than from zeroed registers; and no MFMA result
//     is read as another MFMA's srcA or srcB.
// Per row, the arithmetic and its order are those of the other kernels with
// 32-key tiles: scores, mask, running max, conditional rescale, exponentials,
// bf16 P and its row sums, P.V.
#include "common.hpp"
#include "launch.hpp"

namespace fa {

namespace {

// acc (AGPRs) += a * b, 32x32x16 bf16; AFTER_VALU: after the 2 wait states a VALU write of b needs.
template <bool AFTER_VALU>
__device__ __forceinline__ void mfma_acc_agpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  if constexpr (AFTER_VALU)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// d (VGPRs) = a * b (FIRST) or d += a * b.
template <bool FIRST>
__device__ __forceinline__ void mfma_vgpr(f32x16& d, const bf16x8& a, const bf16x8& b) {
  if constexpr (FIRST)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
// 20 wait states after the MFMAs that last wrote x, before anything reads or overwrites it.
__device__ __forceinline__ void settle_v(f32x16& x) { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(x)); }
template <int NE>
__device__ __forceinline__ void settle_a(f32x16 (&x)[NE]) {
  static_assert(NE == 4 || NE == 8, "accumulator blocks");
  if constexpr (NE == 4)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+a"(x[0]), "+a"(x[1]), "+a"(x[2]), "+a"(x[3]));
  else
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
                 : "+a"(x[0]), "+a"(x[1]), "+a"(x[2]), "+a"(x[3]), "+a"(x[4]), "+a"(x[5]), "+a"(x[6]), "+a"(x[7]));
}

}  // namespace

template <int D_, int OCC_, int BN_>
struct FwdLeanCfg {
  static constexpr int D = D_, OCC = OCC_, BN = BN_, NW = 4;
  static constexpr int BM = 32 * NW;
  static constexpr int NT = 64 * NW;
  static constexpr int RB = D * 2;               // bytes per K / V row
  static constexpr int TILE = BN * RB;           // one K (or V) tile
  static constexpr int STAGE = 2 * TILE;         // K tile, then V tile
  static constexpr int LDS = 2 * STAGE;
  static constexpr int LPW = TILE / 1024 / NW;   // 1 KB DMA loads per wave per tile
  static constexpr int NP = RB / 32;             // 16-byte Q pieces per lane
  static constexpr int NE = D / 32, NB = BN / 32, NC = BN / 16;
  static_assert(TILE % (1024 * NW) == 0, "tile must split into whole 1 KB loads per wave");
  static_assert(OCC * LDS <= 160 * 1024, "LDS budget");
};

template <class C, bool SAME>
__global__ void __launch_bounds__(C::NT)
__attribute__((amdgpu_waves_per_eu(C::OCC, C::OCC)))
fwd_lean_kernel(FwdParams P) {
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
  constexpr int BN = C::BN, NE = C::NE, RB = C::RB, NP = C::NP, NC = C::NC;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hf = lane >> 5;

  int bh, qt;
  wg_map(P.n_qtiles, rank_major(P.cu_q != nullptr, P.causal, P.window, min(P.N, P.Nk), true), P.group, bh, qt,
         long_causal_forward(P.cu_q != nullptr, P.causal, P.window));
  const HeadRows hr = head_rows<2>(P, bh);
  const int N = hr.nq;
  const int n_qt = (N + C::BM - 1) / C::BM;
  if (P.causal) qt = n_qt - 1 - qt;
  if (qt < 0 || qt >= n_qt) return;  // whole workgroup, before any barrier
  const int q0 = qt * C::BM;
  const int qw = q0 + 32 * wave;
  const int qrow = qw + li;

  const KeyBounds kb{N, hr.nk, P.causal, P.window};
  const auto rq = make_rsrc(hr.q, head_span(N, hr.qrs, RB));
  const auto rk = make_rsrc(hr.k, head_span(hr.nk, hr.krs, RB));
  const auto rv = make_rsrc(hr.v, head_span(hr.nk, hr.vrs, RB));
  const float sc = P.scale_log2;
  const float tau = P.rescale_log2;

  static_assert(tile_rows_affine_ok<RB, C::LPW, C::NW>(), "loader rows");
  TileLoader<C::LPW, RB, SAME> tl(wave, lane, hr.krs, hr.vrs);
  auto issue = [&](int first_key, char* dst) {
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      const int m = wave * C::LPW + i;
      buf_load_lds16(rk, tl.a(i, first_key), 0, (lds_void*)(dst + m * 1024));
      buf_load_lds16(rv, tl.b(i, first_key), 0, (lds_void*)(dst + C::TILE + m * 1024));
    }
  };

  // Q^T pieces (B operand of S^T = K Q^T): lane-half h holds bytes 32p + 16h.
  i32x4 qf[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) qf[p] = buf_load16(rq, (uint32_t)qrow * hr.qrs + 32 * p + 16 * hf);

  static_assert(piece_xor_ok<RB, NP>() && tr16_xor_ok<RB, true, NE>(), "offset XOR form");
  uint32_t kbase = tile_off<RB>(li, hf);
  uint32_t vbase = tr16_off<RB, true>(lane, 0, 0);

  f32x16 acc[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) acc[e] = f32x16{};
  float m_ref = -INFINITY, l_part = 0.f;

  const KeyTiles<false, BN> ts(P, bh, kb, q0, q0 + C::BM);
  const int n_tiles = ts.n;
  const int hi_w = kb.hi(qw + 31);

  if (n_tiles > 0) issue(ts.at(0) * BN, smem);
  wait_vmem();  // unconditional: no path reaches the tile loop with the Q loads pending
  __syncthreads();

  auto tile = [&](int j, const char* __restrict__ cur, char* __restrict__ nxt) __attribute__((always_inline)) {
    const int key0 = ts.at(j) * BN;
    const bool more = j + 1 < n_tiles;
    if (more) issue(key0 + BN, nxt);
    const char* ks = cur;
    const char* vs = cur + C::TILE;
    opaque(kbase);
    opaque(vbase);
    if (key0 <= hi_w) {
      // ---- S^T = K Q^T: K pieces read two ahead ----
      f32x16 s[C::NB];
      constexpr int KLA = 2;
      i32x4 ka[KLA + 1][C::NB];
#pragma unroll
      for (int p = 0; p < KLA; ++p)
#pragma unroll
        for (int b = 0; b < C::NB; ++b) ka[p][b] = *reinterpret_cast<const i32x4*>(ks + (kbase ^ piece_xor(p)) + 32 * b * RB);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        if (p + KLA < NP) {
#pragma unroll
          for (int b = 0; b < C::NB; ++b)
            ka[(p + KLA) % (KLA + 1)][b] = *reinterpret_cast<const i32x4*>(ks + (kbase ^ piece_xor(p + KLA)) + 32 * b * RB);
        }
#pragma unroll
        for (int b = 0; b < C::NB; ++b) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, ka[p % (KLA + 1)][b]), bq = __builtin_bit_cast(bf16x8, qf[p]);
          if (p == 0)
            mfma_vgpr<true>(s[b], a, bq);
          else
            mfma_vgpr<false>(s[b], a, bq);
        }
      }
#pragma unroll
      for (int b = 0; b < C::NB; ++b) settle_v(s[b]);
      // ---- mask (causal diagonal, window start, ragged tail) and tile row max ----
      if (kb.mask_tile<BN>(key0, qw)) {
        // key key0 + 8(v/4) + 4h + v%4 is kept iff key_lo(qrow) <= key <= key_hi(qrow)
        int hi = kb.hi(qrow) - key0 - 4 * hf, lo = kb.lo(qrow) - key0 - 4 * hf;
        opaque(hi);
        opaque(lo);
#pragma unroll
        for (int b = 0; b < C::NB; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int r = 32 * b + (v >> 2) * 8 + (v & 3);
            if (r > hi || r < lo) s[b][v] = -INFINITY;
          }
      }
      float m2[2] = {-INFINITY, -INFINITY};
#pragma unroll
      for (int b = 0; b < C::NB; ++b)
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          float& m = m2[(v >> 3) & 1];
          m = fmaxf(fmaxf(m, s[b][v]), s[b][v + 1]);
        }
      const float mx = pair_max32(fmaxf(m2[0], m2[1])) * sc;
      // ---- conditional rescale ----
      const bool grow = mx > m_ref + tau;
      if (wave_any(grow)) {
        settle_a(acc);
        const float m_new = grow ? mx : m_ref;
        // rows that do not grow keep their scale (also when m_ref is still -inf: -inf - -inf is NaN)
        const float alpha = grow ? fast_exp2(m_ref - m_new) : 1.f;
        m_ref = m_new;
        l_part *= alpha;
        // One 16-register block at a time: the empty asm needs each scaled block back in its
        // AGPRs before the next one is copied out, so no more than 16 VGPRs hold O at once.
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          acc[e] *= alpha;
          asm volatile("" : "+a"(acc[e]));
        }
      }
      // a row that has kept no key yet (m_ref = -inf, only under a window) gets p = 2^-inf = 0
      const float neg_m = m_ref == -INFINITY ? 0.f : -m_ref;
      // ---- P = 2^(s sc - m) in bf16, row sums, O^T += V^T P^T per 16-key chunk ----
      float l4[4] = {0.f, 0.f, 0.f, 0.f};
      s16x4 va[2][2];
#pragma unroll
      for (int u = 0; u < 2; ++u) va[0][u] = lds_read_tr16(vs + (vbase ^ tr16_xor<RB, true>(0, u)));
#pragma unroll
      for (int kc = 0; kc < NC; ++kc) {
        const int o8 = (kc & 1) * 8;
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[i] = (__bf16)fast_exp2(__builtin_fmaf(s[kc >> 1][o8 + i], sc, neg_m));
        const i32x4 pw = __builtin_bit_cast(i32x4, pb);
#pragma unroll
        for (int i = 0; i < 4; ++i) l4[i] = dot2_bf16_sum(pw[i], l4[i]);
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          // V^T operand (e + 1, this chunk) or (0, next chunk) one step ahead
          const int st = kc * NE + e + 1;
          if (st < NC * NE) {
            const int kn = st / NE, en = st % NE;
#pragma unroll
            for (int u = 0; u < 2; ++u)
              va[st & 1][u] = lds_read_tr16(vs + (vbase ^ tr16_xor<RB, true>(en, u)) + kn * 16 * RB);
          }
          const bf16x8 a = __builtin_bit_cast(bf16x8, va[(st - 1) & 1]);
          if (e == 0)
            mfma_acc_agpr<true>(acc[e], a, pb);
          else
            mfma_acc_agpr<false>(acc[e], a, pb);
        }
      }
      l_part += (l4[0] + l4[1]) + (l4[2] + l4[3]);
    }
    if (more) wait_vmem();
    __syncthreads();
  };
  for (int j = 0; j < n_tiles; j += 2) {
    tile(j, smem, smem + C::STAGE);
    if (j + 1 < n_tiles) tile(j + 1, smem + C::STAGE, smem);
  }

  // ---- epilogue: O = acc / l, lse = ln(sum exp(s)); O = 0, lse = -inf for a row that kept no key ----
  settle_a(acc);
  const float l_tot = pair_sum32(l_part);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < N) {
    __bf16* orow = reinterpret_cast<__bf16*>(hr.o) + (size_t)qrow * P.so.r;
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 o4 = {(__bf16)(acc[e][4 * g] * inv), (__bf16)(acc[e][4 * g + 1] * inv),
                     (__bf16)(acc[e][4 * g + 2] * inv), (__bf16)(acc[e][4 * g + 3] * inv)};
        *reinterpret_cast<bf16x4*>(orow + 32 * e + 8 * g + 4 * hf) = o4;
      }
    if (hf == 0) hr.lse[qrow] = (m_ref + __builtin_log2f(l_tot)) * kLn2;
  }
}

template <class C>
static hipError_t launch_fwd_lean(const FwdParams& p0, int B, int H, hipStream_t st) {
  FwdParams p = p0;
  p.n_qtiles = (p.N + C::BM - 1) / C::BM;
  const long long grid = (long long)p.n_qtiles * B * H;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (p.sk.r == p.sv.r)
    hipLaunchKernelGGL((fwd_lean_kernel<C, true>), dim3((unsigned)grid), dim3(C::NT), 0, st, p);
  else
    hipLaunchKernelGGL((fwd_lean_kernel<C, false>), dim3((unsigned)grid), dim3(C::NT), 0, st, p);
  return hipGetLastError();
}

hipError_t fwd_lean_dispatch(int D, const FwdParams& p, int B, int H, hipStream_t st) {
  if (D == 256) return launch_fwd_lean<FwdLeanCfg<256, 2, 32>>(p, B, H, st);
  return hipErrorInvalidValue;
}

}  // namespace fa
