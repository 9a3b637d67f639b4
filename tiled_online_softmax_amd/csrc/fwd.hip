// Forward attention kernels for gfx950: float32, bf16 and e4m3 inputs.
//
// Algorithm (page "r/mlscaling", version list): each workgroup owns one tile
// of query rows (FA2's query-tile ownership) and walks the key/value tiles of
// its head with a running row max and row sum (FA1's tiled online softmax),
// normalising the output once at the end (FA2's deferred normalisation). K/V
// tiles are staged through two LDS buffers so the next tile's global loads
// are in flight while the current one is multiplied (FA3's ping-pong tile
// buffers). A row's reference max is only moved -- and its accumulator only
// rescaled -- when a tile's max exceeds it by more than a threshold (FA4's
// conditional rescaling; also the FlashAttention-4 entry on the page
// "FlashAttention" entity trail, section "Corpus findings").
//
// CDNA4 mapping. Each wave owns 32 query rows and computes the transposed
// score block S^T = K Q^T with 32x32 MFMAs, so one lane holds one query's
// scores for 16 keys of every 32-key block. Row max, row sum, the rescale
// factor and lse are then per-lane scalars (plus one exchange with the lane 32
// away), and the output is accumulated transposed, O^T = V^T P^T, directly
// from the score registers. K and V tiles are copied row-major into LDS by
// LDS-DMA loads; V^T operands are read with transposing LDS reads. Q stays in
// registers for the whole loop.
#include "common.hpp"
#include "launch.hpp"

namespace fa {

// A compile-time flag passed as a value (to instantiate a lambda per case).
template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

// ---------------------------------------------------------------------------
// Forward with direct global->LDS tile loads (float32 and e4m3 inputs; bf16
// inputs take the kernels further down).
//
// K and V tiles are copied row-major into swizzled LDS tiles by LDS-DMA
// buffer loads (no register staging, no LDS store instructions). S^T = K Q^T
// reads K rows as MFMA A operands.
//   * float32: the 32x32x2 MFMA contracts two keys held by the two lane
//     halves, so P.V reads V rows directly.
//   * e4m3: both products run on the 32x32x64 fp8 MFMA. The descales fold
//     into the score scale and the output; V^T operands are read with
//     transposing 8-bit LDS reads (ds_read_b64_tr_b8); P is encoded as
//     e4m3(p * 112), the exponent offset by log2 112, so a row's reference
//     max may trail its true max by up to 2 (base 2) before the accumulator
//     must be rescaled (p <= 4 still fits e4m3's 448). The exponential and
//     the encoding are one step, an emulated exponential with an e4m3 result
//     (kCodeShift below): a fused multiply-add and a byte conversion per
//     score, where the hardware exponential, a multiply-add and half a
//     two-value conversion cost about three times as much issue time. e4m3
//     keeps 3 significand bits, so an encoded probability is off by several
//     percent of itself, and a row whose keys all sit in one or two tiles
//     would carry that into O almost undiluted. On tiles that need masking
//     (the causal diagonal, the ragged tail, a window start: all the keys of
//     such short rows), and for rows that keep few keys, P is therefore
//     encoded as two e4m3 terms: the code, and the rest of p * 112 (from the
//     hardware exponential) rounded to nearest, which multiply the same V^T
//     operand: well under 1% relative error.
// The tile loop is unrolled by two so the stage base of every LDS read is an
// immediate.
// ---------------------------------------------------------------------------
// e4m3's largest finite value is 448 = 4 * 112; P is encoded as e4m3(p * 112)
// for p <= 2^kTauP8 = 4, which fixes the rescale threshold at kTauP8.
constexpr float kTauP8 = 2.f;
constexpr float kLog2P8 = 6.80735492205760410744f;  // log2(112)
// Emulated exponential for unmasked e4m3 tiles. For t = log2(p * 112), the
// e4m3 code of 2^t (normal range) is 8 (floor(t) + 7) + 8 (2^f - 1) rounded,
// f = t - floor(t): bias 7, three significand bits. Replacing 2^f - 1 by its
// chord f gives the code straight from t, round(8 t + 56 - shift); the chord
// lies above the curve by up to 0.69 code units, and the shift 0.4566 makes
// the decoded value's ratio to 2^t average 1 over a uniform f (its rms
// deviation is 3.1%, against 2.6% for round-to-nearest). t <= log2 448 keeps
// the code at most 126 (448); t below -7 gives a negative value, which the
// byte conversion clamps to code 0.
constexpr float kCodeShift = 0.4566f;
// Rows keeping at most this many keys take the residual term on every tile.
constexpr int kFewKeysP8 = 256;

template <Elt E, int D_, int BN_, int NW_, int OCC_>
struct FwdDCfg {
  static constexpr Elt elt = E;
  static constexpr int D = D_, BN = BN_, NW = NW_, OCC = OCC_;
  static constexpr int ESZ = EltInfo<E>::bytes;
  static constexpr int BM = 32 * NW;
  static constexpr int NT = 64 * NW;
  static constexpr int RB = D * ESZ;             // bytes per K / V row
  static constexpr int TILE = BN * RB;           // one K (or V) tile
  static constexpr int STAGE = 2 * TILE;         // K tile, then V tile
  static constexpr int LDS = 2 * STAGE;
  static constexpr int LPW = TILE / 1024 / NW;   // 1 KB DMA loads per wave per tile
  static constexpr int NP = RB / 32;             // 16-byte Q pieces per lane
  static constexpr int NB = BN / 32, NE = D / 32;
  static_assert(E != Elt::FP8 || BN % 64 == 0, "fp8 contracts 64 keys per MFMA");
  static_assert(TILE % (1024 * NW) == 0, "tile must split into whole 1 KB loads per wave");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// SAME: K and V rows are equally spaced (one loader offset serves both).
// SPARSE: walk only the key tiles of the blocks listed for this query block.
template <class C, bool SAME, bool SPARSE>
__global__ void __launch_bounds__(C::NT)
__attribute__((amdgpu_waves_per_eu(C::OCC, C::OCC)))
fwd_kernel(FwdParams P) {
  static_assert(C::elt != Elt::BF16, "bf16 inputs take fwd_pipe_kernel / fwd_pp_kernel");
  constexpr bool FP8 = C::elt == Elt::FP8;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
  constexpr int D = C::D, BN = C::BN, NB = C::NB, NE = C::NE, RB = C::RB, NP = C::NP;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps per-wave branches scalar
  const int li = lane & 31, hf = lane >> 5;

  // Workgroup -> (head, query tile); under causal masking the last query
  // tiles carry the most key tiles, so rank 0 is the last one.
  int bh, qt;
  wg_map(P.n_qtiles, rank_major(P.cu_q != nullptr || P.kv_index != nullptr, P.causal, P.window, min(P.N, P.Nk), true), P.group, bh, qt,
         long_causal_forward(P.cu_q != nullptr || P.kv_index != nullptr, P.causal, P.window));
  const HeadRows hr = head_rows<C::ESZ>(P, bh);
  const int N = hr.nq;
  const int n_qt = (N + C::BM - 1) / C::BM;  // this entry's query tiles (fewer for a short packed sequence)
  if (P.causal) qt = n_qt - 1 - qt;
  if (qt < 0 || qt >= n_qt) return;  // whole workgroup: nothing of this entry is left
  const int q0 = qt * C::BM;
  const int qw = q0 + 32 * wave;
  const int qrow = qw + li;

  const KeyBounds kb{N, hr.nk, P.causal, P.window};
  const auto rq = make_rsrc(hr.q, head_span(N, hr.qrs, RB));
  const auto rk = make_rsrc(hr.k, head_span(hr.nk, hr.krs, RB));
  const auto rv = make_rsrc(hr.v, head_span(hr.nk, hr.vrs, RB));
  float sc = P.scale_log2;
  float tau = P.rescale_log2;
  float out_mul = 1.f;
  if constexpr (FP8) {
    // descales fold into the score scale and the output; P is encoded as
    // e4m3(p * 112), which needs p <= 4, hence the threshold kTauP8 = 2.
    // The exponent is offset by log2 112, so the codes (and, on masked
    // tiles, the exponentials) stand for p * 112 directly; the row sums then
    // also carry the factor, which cancels in O and is taken out of lse.
    const float dq = P.q_descale ? *P.q_descale : 1.f;
    const float dk = P.k_descale ? *P.k_descale : 1.f;
    const float dv = P.v_descale ? *P.v_descale : 1.f;
    sc *= dq * dk;
    out_mul = dv;
    tau = kTauP8;
  }

  // Loader: 16-byte slot `lane` of 1 KB block m of a tile comes from tile_pos(slot).
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

  // Per-lane LDS read offsets (tile-relative); blocks and key chunks add whole rows.
  uint32_t koff[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) koff[p] = tile_off<RB>(li, 2 * p + hf);
  uint32_t voff[NE];
  if constexpr (FP8) {
#pragma unroll
    for (int e = 0; e < NE; ++e) voff[e] = tr8_off<RB>(lane, e);
  }

  f32x16 acc[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) acc[e] = f32x16{};
  float m_ref = -INFINITY, l_part = 0.f;
  float neg_m = FP8 ? kLog2P8 : 0.f;  // exponent offset of p: -m_ref (0 while m_ref = -inf), + log2 112 for e4m3
  // e4m3: the row sums run on the matrix core. A 16x16x128 MFMA contracts the
  // P operand of the 32x32x64 product (lane L: query row L % 32, 32 of the 64
  // keys) against a 0 / 1 pattern that adds, for output lane l, the four
  // operand lanes of row l % 32 (lane groups of 16 with the parity of l / 16):
  // every lane receives its row's sum of the encoded probabilities, exactly the
  // weights P.V used, in all four accumulator entries.
  f32x4 l_acc = {0.f, 0.f, 0.f, 0.f};
  i32x8 ones_sel;
  // e4m3 P operand. Each word is written byte by byte (or, for the residual
  // term, by two half-word packs), each conversion keeping the rest of its
  // `old` operand: passing the previous tile's word there (overwritten
  // anyway) keeps the words in place without zeroing moves.
  i32x8 pb = {};
  if constexpr (FP8) {
    const int v = ((lane >> 2) & 1) == ((lane >> 4) & 1) ? 0x38383838 : 0;  // e4m3 1.0 = 0x38
#pragma unroll
    for (int i = 0; i < 8; ++i) ones_sel[i] = v;
  }

  // The workgroup's key tiles, j = 0 .. n_tiles-1: dense, the tiles
  // [t_lo, t_end) that hold every key a row of it keeps; sparse, the tiles of
  // the listed key blocks (ascending). This wave's rows keep no key past hi_w.
  static_assert(!SPARSE || (C::BM == kBlock && kBlock % BN == 0), "a query tile is one mask block");
  const KeyTiles<SPARSE, BN> ts(P, bh, kb, q0, q0 + C::BM);
  const int n_tiles = ts.n;
  const int hi_w = kb.hi(qw + 31);
  // e4m3: rows that keep few keys (every row of this wave at most kFewKeysP8)
  // average little of the encoding error away, so they take the residual term
  // on every tile, not only on masked ones.
  const bool few_keys = FP8 && hi_w - kb.lo(qw) < kFewKeysP8;

  if (n_tiles > 0) issue(ts.at_clamped(0) * BN, smem);
  // unconditional: a path that reached the tile loop with the Q loads pending
  // would make the compiler wait for every prefetch inside the loop
  wait_vmem();
  __syncthreads();

  // e4m3 P of a 64-key tile, written into pb: the emulated exponential of the
  // raw scores s, code = round(s * sc8 + c8) with sc8 = 8 sc and
  // c8 = 8 neg_m + 56 - kCodeShift, one byte conversion per score (negative
  // values, masked scores among them, clamp to code 0).
  static_assert(!FP8 || BN == 64, "e4m3 tiles are one 64-key chunk (pb holds the chunk's codes)");
  const float sc8 = 8.f * sc;
  float c8 = 8.f * neg_m + (56.f - kCodeShift);
  auto encode_p = [&](const f32x16 (&s)[NB]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f32x16& sb = s[j >> 2];
      const int o = (j & 3) * 4;
      unsigned w32 = (unsigned)pb[j];
#pragma unroll
      for (int u = 0; u < 4; ++u) w32 = cvt_u8(__builtin_fmaf(sb[o + u], sc8, c8), u, w32);
      pb[j] = (int)w32;
    }
  };
  // Masked tiles and rows with few keys: a second term, what the codes in pb
  // leave out of p * 112 (the hardware exponential's value, in s here),
  // rounded to nearest.
  auto encode_residual = [&](const f32x16 (&s)[NB]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f32x16& sb = s[j >> 2];
      const int o = (j & 3) * 4;
      const auto d01 = __builtin_amdgcn_cvt_pk_f32_fp8(pb[j], false);
      const auto d23 = __builtin_amdgcn_cvt_pk_f32_fp8(pb[j], true);
      int w32 = cvt_fp8x2<false>(sb[o] - d01[0], sb[o + 1] - d01[1], pb[j]);
      w32 = cvt_fp8x2<true>(sb[o + 2] - d23[0], sb[o + 3] - d23[1], w32);
      pb[j] = w32;
    }
  };
  // O^T += V^T P^T for chunk kc with the P in pb; its row sums go to l_acc.
  auto mul_pv = [&](const char* vs, int kc) __attribute__((always_inline)) {
    l_acc = mfma_fp8_16(ones_sel, pb, l_acc);
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      i32x2 a4[4];
#pragma unroll
      for (int wr = 0; wr < 4; ++wr) a4[wr] = lds_read_tr8(vs + voff[e] + (64 * kc + 16 * wr) * RB);
      acc[e] = mfma_fp8(__builtin_bit_cast(i32x8, a4), pb, acc[e]);
    }
  };

  // One key/value tile. `cur` (being read) and `nxt` (being filled by the
  // LDS-DMA prefetch) are distinct stage buffers; declaring them restrict lets
  // the compiler see that the transposing reads of `cur` cannot depend on the
  // prefetch, so it does not wait for the prefetch before them. The prefetch is
  // waited for explicitly (vmcnt + barrier) at the end of the tile.
  int key0 = ts.at_clamped(0) * BN, key1 = ts.at_clamped(1) * BN;  // tiles j and j+1 (list reads run ahead)
  auto tile = [&](int j, const char* __restrict__ cur, char* __restrict__ nxt) {
    const int key2 = ts.at_clamped(j + 2) * BN;  // read now, used by the next tile
    const bool more = j + 1 < n_tiles;
    if (more) issue(key1, nxt);
    const char* ks = cur;
    const char* vs = cur + C::TILE;
    if (key0 <= hi_w) {
      // ---- S^T = K Q^T ----
      f32x16 s[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) s[b] = f32x16{};
#pragma unroll
      for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          if constexpr (FP8) {
            if (p & 1) continue;  // one MFMA per pair of 16-byte pieces (64 fp8 values)
            const i32x4 a0 = *reinterpret_cast<const i32x4*>(ks + koff[p] + 32 * b * RB);
            const i32x4 a1 = *reinterpret_cast<const i32x4*>(ks + koff[p + 1] + 32 * b * RB);
            const i32x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            const i32x8 bq = {qf[p][0], qf[p][1], qf[p][2], qf[p][3],
                              qf[p + 1][0], qf[p + 1][1], qf[p + 1][2], qf[p + 1][3]};
            s[b] = mfma_fp8(a, bq, s[b]);
          } else {
            const f32x4 a = *reinterpret_cast<const f32x4*>(ks + koff[p] + 32 * b * RB);
            const f32x4 bq = __builtin_bit_cast(f32x4, qf[p]);
#pragma unroll
            for (int u = 0; u < 4; ++u) s[b] = mfma_f32(a[u], bq[u], s[b]);
          }
        }
      }
      // ---- mask (causal diagonal, window start, ragged tail) and tile row max ----
      const bool masked = kb.mask_tile<BN>(key0, qw);
      if (masked) {
        // key key0 + 32b + 8(v/4) + 4h + v%4 is kept iff key_lo(qrow) <= key <= key_hi(qrow);
        // compare the lane-independent part r against two per-lane limits.
        const int hi = kb.hi(qrow) - key0 - 4 * hf, lo = kb.lo(qrow) - key0 - 4 * hf;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int r = 32 * b + (v >> 2) * 8 + (v & 3);
            if (r > hi || r < lo) s[b][v] = -INFINITY;
          }
      }
      // row max: two chains of three-way maxima (each step folds two scores into
      // the running value, which maps to one max3), then the partner lane
      float m2[2] = {-INFINITY, -INFINITY};
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          float& m = m2[(v >> 3) & 1];
          m = fmaxf(fmaxf(m, s[b][v]), s[b][v + 1]);
        }
      const float mx = pair_max32(fmaxf(m2[0], m2[1])) * sc;
      // ---- conditional rescale ----
      const bool grow = mx > m_ref + tau;
      if (wave_any(grow)) {
        const float m_new = grow ? mx : m_ref;
        // rows that do not grow keep their scale (also when m_ref is still -inf: -inf - -inf is NaN)
        const float alpha = grow ? fast_exp2(m_ref - m_new) : 1.f;
        m_ref = m_new;
        // a row that has kept no key yet (m_ref = -inf, only under a window) gets p = 2^-inf = 0
        neg_m = (m_ref == -INFINITY ? 0.f : -m_ref) + (FP8 ? kLog2P8 : 0.f);
        if constexpr (FP8) {
          l_acc *= alpha;
          c8 = 8.f * neg_m + (56.f - kCodeShift);
        } else {
          l_part *= alpha;
        }
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[e] *= alpha;
      }
      // ---- O^T += V^T P^T ----
      if constexpr (FP8) {
        encode_p(s);
        mul_pv(vs, 0);
        if (masked || few_keys) {
#pragma unroll
          for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) s[b][v] = fast_exp2(__builtin_fmaf(s[b][v], sc, neg_m));
          encode_residual(s);
          mul_pv(vs, 0);
        }
      } else {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v) s[b][v] = fast_exp2(__builtin_fmaf(s[b][v], sc, neg_m));
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            l_part += s[b][v];
            const int key = 32 * b + (v >> 2) * 8 + hf * 4 + (v & 3);
#pragma unroll
            for (int e = 0; e < NE; ++e) {
              const int col = 32 * e + li;
              const float a = *reinterpret_cast<const float*>(vs + tile_off<RB>(key, col >> 2) + (col & 3) * 4);
              acc[e] = mfma_f32(a, s[b][v], acc[e]);
            }
          }
      }
    }
    if (more) wait_vmem();
    __syncthreads();
    key0 = key1;
    key1 = key2;
  };
  for (int j = 0; j < n_tiles; j += 2) {
    tile(j, smem, smem + C::STAGE);
    if (j + 1 < n_tiles) tile(j + 1, smem + C::STAGE, smem);
  }

  // ---- epilogue: O = acc / l, lse = ln(sum exp(s)) ----
  // A row that kept no key has l = 0 and m_ref = -inf: O = 0 and lse = -inf.
  const float l_tot = FP8 ? l_acc[0] : pair_sum32(l_part);
  const float inv = l_tot > 0.f ? out_mul / l_tot : 0.f;
  if (qrow < N) {
    if constexpr (C::elt == Elt::F32) {
      float* orow = reinterpret_cast<float*>(hr.o) + (size_t)qrow * P.so.r;
#pragma unroll
      for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 o4 = {acc[e][4 * g] * inv, acc[e][4 * g + 1] * inv, acc[e][4 * g + 2] * inv, acc[e][4 * g + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + 32 * e + 8 * g + 4 * hf) = o4;
        }
    } else {
      __bf16* orow = reinterpret_cast<__bf16*>(hr.o) + (size_t)qrow * P.so.r;
#pragma unroll
      for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 o4 = {(__bf16)(acc[e][4 * g] * inv), (__bf16)(acc[e][4 * g + 1] * inv),
                       (__bf16)(acc[e][4 * g + 2] * inv), (__bf16)(acc[e][4 * g + 3] * inv)};
          *reinterpret_cast<bf16x4*>(orow + 32 * e + 8 * g + 4 * hf) = o4;
        }
    }
    if (hf == 0) hr.lse[qrow] = (m_ref + __builtin_log2f(l_tot) - (FP8 ? kLog2P8 : 0.f)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// bf16 forward, software-pipelined across key tiles.
//
// Same tiling, data layout and numerics as fwd_kernel; only the order of work
// differs. Iteration j of the tile loop issues the score MFMAs of tile j+1
// (S_{j+1} = K_{j+1} Q^T) and, between them, the VALU work that turns S_j into
// P_j (exponentials, bf16 packing, row sums); it then issues the P.V MFMAs of
// tile j and, between them, the masking and row max of S_{j+1} and the
// conditional rescale. A wave's instruction stream thus alternates MFMAs with
// independent VALU work, which the SIMD executes while the MFMAs run, rather
// than a block of MFMAs followed by a block of softmax arithmetic.
//
// LDS holds two K and two V tiles; K runs one tile ahead of V:
//   iteration j reads K_{j+1} from Kb[(j+1)%2] and V_j from Vb[j%2], and its
//   LDS-DMA loads fill Kb[j%2] with K_{j+2} and Vb[(j+1)%2] with V_{j+1}, the
//   buffers read by iteration j-1 (all waves passed the barrier ending it).
// ---------------------------------------------------------------------------
template <class C, bool SAME, bool SPARSE>
__global__ void __launch_bounds__(C::NT)
__attribute__((amdgpu_waves_per_eu(C::OCC, C::OCC)))
fwd_pipe_kernel(FwdParams P) {
  static_assert(C::elt == Elt::BF16, "bf16 only");
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
  constexpr int D = C::D, BN = C::BN, NB = C::NB, NE = C::NE, RB = C::RB, NP = C::NP, TILE = C::TILE;
  constexpr int NC = BN / 16;  // 16-key chunks of a tile (P.V contraction steps)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hf = lane >> 5;

  int bh, qt;
  wg_map(P.n_qtiles, rank_major(P.cu_q != nullptr || P.kv_index != nullptr, P.causal, P.window, min(P.N, P.Nk), true), P.group, bh, qt,
         long_causal_forward(P.cu_q != nullptr || P.kv_index != nullptr, P.causal, P.window));
  const HeadRows hr = head_rows<2>(P, bh);
  const int N = hr.nq;
  const int n_qt = (N + C::BM - 1) / C::BM;
  if (P.causal) qt = n_qt - 1 - qt;
  if (qt < 0 || qt >= n_qt) return;
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
  // The workgroup's key tiles j = 0 .. n_tiles-1 (ts.at(j): dense from t_lo,
  // or the tiles of the listed key blocks) cover the keys any of its rows keeps.
  static_assert(!SPARSE || (C::BM == kBlock && kBlock % BN == 0), "a query tile is one mask block");
  const KeyTiles<SPARSE, BN> ts(P, bh, kb, q0, q0 + C::BM);
  const int n_tiles = ts.n;
  // tiles [0, n_live) hold keys this wave's queries may keep (every wave starts at the first tile:
  // rows whose window starts later see fully masked tiles first, which add nothing)
  const int n_live = ts.live_count(kb.hi(qw + 31));

  // K (V) of the tile starting at key key0 into dst
  auto issue_k = [&](int first_key, char* dst) {
#pragma unroll
    for (int i = 0; i < C::LPW; ++i)
      buf_load_lds16(rk, tl.a(i, first_key), 0, (lds_void*)(dst + (wave * C::LPW + i) * 1024));
  };
  auto issue_v = [&](int first_key, char* dst) {
#pragma unroll
    for (int i = 0; i < C::LPW; ++i)
      buf_load_lds16(rv, tl.b(i, first_key), 0, (lds_void*)(dst + (wave * C::LPW + i) * 1024));
  };

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


  char* const kb0 = smem;
  char* const kb1 = smem + TILE;
  char* const vb0 = smem + 2 * TILE;
  char* const vb1 = smem + 3 * TILE;

  // ---- S = K Q^T for one tile, optionally interleaved with P-work ----
  // VALU work on the previous scores comes in 2*NC half-chunks; half-chunk h
  // (4 keys of chunk h/2 per lane) runs next to score step (h * NP) / (2 NC).
  f32x16 sa[NB], sb[NB];  // scores of the tile being finished / being computed
  bf16x8 pb[NC];
  float l4[4];
  auto half_chunk = [&](f32x16 (&s)[NB], int h, float neg_m) {
    const int kc = h >> 1, o = (kc & 1) * 8 + (h & 1) * 4;
    f32x16& sv = s[kc >> 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[o + i] = fast_exp2(__builtin_fmaf(sv[o + i], sc, neg_m));
    if (h & 1) {
      const int o8 = (kc & 1) * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[kc][i] = (__bf16)sv[o8 + i];
      i32x4 pw = __builtin_bit_cast(i32x4, pb[kc]);
      opaque(pw);  // keeps this work here (not sunk next to its use in P.V)
      pb[kc] = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        l4[i] = dot2_bf16_sum(pw[i], l4[i]);
        opaque(l4[i]);
      }
    }
  };
  // with_s: compute scores of tile t from kt into sn; with_p: turn sp into P.
  auto scores_and_p = [&](const bool with_s, const bool with_p, const char* __restrict__ kt, f32x16 (&sn)[NB],
                          f32x16 (&sp)[NB]) __attribute__((always_inline)) {
    // a row that has kept no key yet (m_ref = -inf, only under a window) gets p = 2^-inf = 0
    const float neg_m = m_ref == -INFINITY ? 0.f : -m_ref;
    l4[0] = l4[1] = l4[2] = l4[3] = 0.f;
    if (with_s) {
      constexpr int KLA = 2;
      i32x4 ka[KLA + 1][NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) sn[b] = f32x16{};
#pragma unroll
      for (int p = 0; p < KLA; ++p)
#pragma unroll
        for (int b = 0; b < NB; ++b)
          ka[p][b] = *reinterpret_cast<const i32x4*>(kt + (kbase ^ piece_xor(p)) + 32 * b * RB);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        if (p + KLA < NP) {
#pragma unroll
          for (int b = 0; b < NB; ++b)
            ka[(p + KLA) % (KLA + 1)][b] =
                *reinterpret_cast<const i32x4*>(kt + (kbase ^ piece_xor(p + KLA)) + 32 * b * RB);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < NB; ++b)
          sn[b] = mfma_bf16(__builtin_bit_cast(bf16x8, ka[p % (KLA + 1)][b]), __builtin_bit_cast(bf16x8, qf[p]), sn[b]);
        if (with_p) {
#pragma unroll
          for (int h = 0; h < 2 * NC; ++h)
            if ((h * NP) / (2 * NC) == p) half_chunk(sp, h, neg_m);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if (with_p) {
#pragma unroll
      for (int h = 0; h < 2 * NC; ++h) half_chunk(sp, h, neg_m);
    }
    if (with_p) l_part += (l4[0] + l4[1]) + (l4[2] + l4[3]);
  };

  // ---- mask + row max of a score tile, then the conditional rescale ----
  // with_pv: P.V MFMAs of the previous tile run interleaved (vt = its V tile).
  auto pv_and_max = [&](const bool with_pv, const bool with_max, const char* __restrict__ vt, int key0,
                        f32x16 (&s)[NB], bool use_max) __attribute__((always_inline)) {
    if (with_max && use_max) {
      // key key0 + 4h + r of the tile (r = 32b + 8(v/4) + v%4) is kept iff lo <= r <= hi
      if (kb.mask_tile<BN>(key0, qw)) {
        int hi = kb.hi(qrow) - key0 - 4 * hf, lo = kb.lo(qrow) - key0 - 4 * hf;
        opaque(hi);
        opaque(lo);
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int r = 32 * b + (v >> 2) * 8 + (v & 3);
            if (r > hi || r < lo) s[b][v] = -INFINITY;
          }
      }
    }
    float m2[2] = {-INFINITY, -INFINITY};
    auto max_part = [&](int kc) {
      // keys of chunk kc: s[kc/2][(kc%2)*8 .. +8]
      const f32x16& sv = s[kc >> 1];
      const int o = (kc & 1) * 8;
#pragma unroll
      for (int v = 0; v < 8; v += 2) m2[kc & 1] = fmaxf(fmaxf(m2[kc & 1], sv[o + v]), sv[o + v + 1]);
    };
    if (with_pv) {
      s16x4 va[2][NE][2];
#pragma unroll
      for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int u = 0; u < 2; ++u) va[0][e][u] = lds_read_tr16(vt + (vbase ^ tr16_xor<RB, true>(e, u)));
#pragma unroll
      for (int kc = 0; kc < NC; ++kc) {
        if (kc + 1 < NC) {
#pragma unroll
          for (int e = 0; e < NE; ++e)
#pragma unroll
            for (int u = 0; u < 2; ++u)
              va[(kc + 1) & 1][e][u] = lds_read_tr16(vt + (vbase ^ tr16_xor<RB, true>(e, u)) + (kc + 1) * 16 * RB);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[e] = mfma_bf16(__builtin_bit_cast(bf16x8, va[kc & 1][e]), pb[kc], acc[e]);
        if (with_max) max_part(kc);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if (with_max) {
#pragma unroll
      for (int kc = 0; kc < NC; ++kc) max_part(kc);
    }
    if (with_max) {
      const float mx = pair_max32(fmaxf(m2[0], m2[1])) * sc;
      const bool grow = mx > m_ref + tau;
      if (use_max && wave_any(grow)) {
        const float m_new = grow ? mx : m_ref;
        // rows that do not grow keep their scale (also when m_ref is still -inf: -inf - -inf is NaN)
        const float alpha = grow ? fast_exp2(m_ref - m_new) : 1.f;
        m_ref = m_new;
        l_part *= alpha;
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[e] *= alpha;
      }
    }
  };

  // ---- prologue: K_0, V_0, K_1 in; S_0 and its max ----
  // first keys of tiles j+1 and j+2 of the coming iteration j (list reads run one iteration ahead)
  int key1 = ts.at_clamped(1) * BN, key2 = ts.at_clamped(2) * BN;
  if (n_tiles > 0) {
    const int key0 = ts.at_clamped(0) * BN;
    issue_k(key0, kb0);
    issue_v(key0, vb0);
  }
  if (n_tiles > 1) issue_k(key1, kb1);
  wait_vmem();
  __syncthreads();
  if (n_live > 0) {
    scores_and_p(true, false, kb0, sa, sb);
    pv_and_max(false, true, vb0, ts.at_clamped(0) * BN, sa, true);
  }
  __syncthreads();  // every wave is done with Kb[0] before K_2 overwrites it

  // One iteration; sc_ holds S_j on entry, sn_ receives S_{j+1}.
  auto iter = [&](int j, const char* __restrict__ kcur, const char* __restrict__ vcur, char* __restrict__ knxt,
                  char* __restrict__ vnxt, f32x16 (&sc_)[NB], f32x16 (&sn_)[NB]) __attribute__((always_inline)) {
    const int key3 = ts.at_clamped(j + 3) * BN;  // read now, used by the next iteration
    if (j + 1 < n_tiles) issue_v(key1, vnxt);
    if (j + 2 < n_tiles) issue_k(key2, knxt);
    opaque(kbase);
    opaque(vbase);
    if (j < n_live) {
      // the last live tile also computes (and discards) scores for the next tile
      scores_and_p(true, true, kcur, sn_, sc_);
      pv_and_max(true, true, vcur, key1, sn_, j + 1 < n_live);
    }
    if (j + 1 < n_tiles) wait_vmem();
    __syncthreads();
    key1 = key2;
    key2 = key3;
  };
  for (int j = 0; j < n_tiles; j += 2) {
    iter(j, kb1, vb0, kb0, vb1, sa, sb);
    if (j + 1 < n_tiles) iter(j + 1, kb0, vb1, kb1, vb0, sb, sa);
  }

  // ---- epilogue: O = acc / l, lse = ln(sum exp(s)); O = 0, lse = -inf for a row that kept no key ----
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

// ---------------------------------------------------------------------------
// bf16 forward with two wave groups in alternating phases.
//
// Eight waves per workgroup, two per SIMD (waves w and w + 4). Tile step j
// has an MFMA phase M(j) -- the scores S_j = K_j Q^T and the product
// O^T += V_{j-1}^T P_{j-1}^T -- and a softmax phase X(j) -- mask, row max,
// conditional rescale, exponentials, bf16 packing and row sums of S_j. Waves
// 0-3 run M(j) while waves 4-7 run X(j-1), then the groups swap, with an
// execution barrier between the phases: each SIMD's matrix core is fed by one
// wave while its partner's softmax runs on the VALU. This is the overlap that
// FA4 gets from separate softmax warps (page "FlashAttention" entity trail,
// FlashAttention-4), arranged for two waves per CDNA4 SIMD. The two waves of
// a SIMD own adjacent 32-row blocks, so under causal masking they see about
// the same number of live tiles.
//
// K and V land in two-stage rings. Step j issues K_{j+1} and V_j, which step
// j+1 reads, and every wave waits for its own copies before the step's
// closing barrier. Each wave runs 1 + 2 (n_tiles + 1) barriers, a count fixed
// by the workgroup's tile range alone.
// ---------------------------------------------------------------------------
template <int D_, int BN_>
struct FwdPPCfg {
  static constexpr int D = D_, BN = BN_, NW = 8;
  static constexpr int BM = 32 * NW;
  static constexpr int NT = 64 * NW;
  static constexpr int RB = D * 2;               // bytes per K / V row
  static constexpr int TILE = BN * RB;           // one K (or V) tile
  static constexpr int LDS = 4 * TILE;           // K and V, two stages each
  static constexpr int LPW = TILE / 1024 / NW;   // 1 KB DMA loads per wave per tile
  static constexpr int NP = RB / 32;             // 16-byte Q pieces per lane
  static constexpr int NB = BN / 32, NE = D / 32, NC = BN / 16;
  static_assert(TILE % (1024 * NW) == 0, "tile must split into whole 1 KB loads per wave");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <class C, bool SAME>
__global__ void __launch_bounds__(C::NT)
__attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_pp_kernel(FwdParams P) {
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
  constexpr int D = C::D, BN = C::BN, NB = C::NB, NE = C::NE, RB = C::RB, NP = C::NP, TILE = C::TILE, NC = C::NC;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hf = lane >> 5;
  const bool second = wave >= 4;  // the second group runs half a step behind the first

  int bh, qt;
  wg_map(P.n_qtiles, rank_major(P.cu_q != nullptr || P.kv_index != nullptr, P.causal, P.window, min(P.N, P.Nk), true), P.group, bh, qt,
         long_causal_forward(P.cu_q != nullptr || P.kv_index != nullptr, P.causal, P.window));
  const HeadRows hr = head_rows<2>(P, bh);
  const int N = hr.nq;
  const int n_qt = (N + C::BM - 1) / C::BM;
  if (P.causal) qt = n_qt - 1 - qt;
  if (qt < 0 || qt >= n_qt) return;  // whole workgroup, before any barrier
  const int q0 = qt * C::BM;
  const int qw = q0 + 32 * (2 * (wave & 3) + (wave >> 2));
  const int qrow = qw + li;

  const KeyBounds kb{N, hr.nk, P.causal, P.window};
  const auto rq = make_rsrc(hr.q, head_span(N, hr.qrs, RB));
  const auto rk = make_rsrc(hr.k, head_span(hr.nk, hr.krs, RB));
  const auto rv = make_rsrc(hr.v, head_span(hr.nk, hr.vrs, RB));
  const float sc = P.scale_log2;
  const float tau = P.rescale_log2;

  static_assert(tile_rows_affine_ok<RB, C::LPW, C::NW>(), "loader rows");
  TileLoader<C::LPW, RB, SAME> tl(wave, lane, hr.krs, hr.vrs);
  const KeyTiles<false, BN> ts(P, bh, kb, q0, q0 + C::BM);
  const int n_tiles = max(ts.n, 0);  // workgroup-uniform: it alone sets the barrier count
  const int n_live = ts.live_count(kb.hi(qw + 31));  // tiles holding keys this wave's rows may keep

  auto issue_k = [&](int first_key, char* dst) {
#pragma unroll
    for (int i = 0; i < C::LPW; ++i)
      buf_load_lds16(rk, tl.a(i, first_key), 0, (lds_void*)(dst + (wave * C::LPW + i) * 1024));
  };
  auto issue_v = [&](int first_key, char* dst) {
#pragma unroll
    for (int i = 0; i < C::LPW; ++i)
      buf_load_lds16(rv, tl.b(i, first_key), 0, (lds_void*)(dst + (wave * C::LPW + i) * 1024));
  };

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
  f32x16 s[NB];   // S_j, from M(j) to X(j)
  bf16x8 pb[NC];  // P_j, from X(j) to M(j+1)

  char* const ks0 = smem;
  char* const ks1 = smem + TILE;
  char* const vs0 = smem + 2 * TILE;
  char* const vs1 = smem + 3 * TILE;

  // ---- M(j): S_j = K_j Q^T (if tile j is live) and O^T += V_{j-1}^T P_{j-1}^T ----
  auto mma_phase = [&](int j, const char* __restrict__ kt, const char* __restrict__ vt) __attribute__((always_inline)) {
    if (j >= 1 && j - 1 < n_live) {
      s16x4 va[2][NE][2];
#pragma unroll
      for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int u = 0; u < 2; ++u) va[0][e][u] = lds_read_tr16(vt + (vbase ^ tr16_xor<RB, true>(e, u)));
#pragma unroll
      for (int kc = 0; kc < NC; ++kc) {
        if (kc + 1 < NC) {
#pragma unroll
          for (int e = 0; e < NE; ++e)
#pragma unroll
            for (int u = 0; u < 2; ++u)
              va[(kc + 1) & 1][e][u] = lds_read_tr16(vt + (vbase ^ tr16_xor<RB, true>(e, u)) + (kc + 1) * 16 * RB);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[e] = mfma_bf16(__builtin_bit_cast(bf16x8, va[kc & 1][e]), pb[kc], acc[e]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (j < n_live) {
      constexpr int KLA = 2;
      i32x4 ka[KLA + 1][NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) s[b] = f32x16{};
#pragma unroll
      for (int p = 0; p < KLA; ++p)
#pragma unroll
        for (int b = 0; b < NB; ++b)
          ka[p][b] = *reinterpret_cast<const i32x4*>(kt + (kbase ^ piece_xor(p)) + 32 * b * RB);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        if (p + KLA < NP) {
#pragma unroll
          for (int b = 0; b < NB; ++b)
            ka[(p + KLA) % (KLA + 1)][b] =
                *reinterpret_cast<const i32x4*>(kt + (kbase ^ piece_xor(p + KLA)) + 32 * b * RB);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < NB; ++b)
          s[b] = mfma_bf16(__builtin_bit_cast(bf16x8, ka[p % (KLA + 1)][b]), __builtin_bit_cast(bf16x8, qf[p]), s[b]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // ---- X(j): mask, row max, conditional rescale, P_j = exp2(S_j sc - m), row sums ----
  auto softmax_phase = [&](int j) __attribute__((always_inline)) {
    if (j < 0 || j >= n_live) return;
    const int key0 = ts.at(j) * BN;
    // key key0 + 4h + r of the tile (r = 32b + 8(v/4) + v%4) is kept iff lo <= r <= hi
    if (kb.mask_tile<BN>(key0, qw)) {
      int hi = kb.hi(qrow) - key0 - 4 * hf, lo = kb.lo(qrow) - key0 - 4 * hf;
      opaque(hi);
      opaque(lo);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = 32 * b + (v >> 2) * 8 + (v & 3);
          if (r > hi || r < lo) s[b][v] = -INFINITY;
        }
    }
    float m2[2] = {-INFINITY, -INFINITY};
#pragma unroll
    for (int kc = 0; kc < NC; ++kc) {
      const f32x16& sv = s[kc >> 1];
      const int o = (kc & 1) * 8;
#pragma unroll
      for (int v = 0; v < 8; v += 2) m2[kc & 1] = fmaxf(fmaxf(m2[kc & 1], sv[o + v]), sv[o + v + 1]);
    }
    const float mx = pair_max32(fmaxf(m2[0], m2[1])) * sc;
    const bool grow = mx > m_ref + tau;
    if (wave_any(grow)) {
      const float m_new = grow ? mx : m_ref;
      // rows that do not grow keep their scale (also when m_ref is still -inf: -inf - -inf is NaN)
      const float alpha = grow ? fast_exp2(m_ref - m_new) : 1.f;
      m_ref = m_new;
      l_part *= alpha;
#pragma unroll
      for (int e = 0; e < NE; ++e) acc[e] *= alpha;
    }
    // a row that has kept no key yet (m_ref = -inf, only under a window) gets p = 2^-inf = 0
    const float neg_m = m_ref == -INFINITY ? 0.f : -m_ref;
    float l4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < NC; ++kc) {
      f32x16& sv = s[kc >> 1];
      const int o8 = (kc & 1) * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) sv[o8 + i] = fast_exp2(__builtin_fmaf(sv[o8 + i], sc, neg_m));
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[kc][i] = (__bf16)sv[o8 + i];
      const i32x4 pw = __builtin_bit_cast(i32x4, pb[kc]);
#pragma unroll
      for (int i = 0; i < 4; ++i) l4[i] = dot2_bf16_sum(pw[i], l4[i]);
    }
    l_part += (l4[0] + l4[1]) + (l4[2] + l4[3]);
  };

  // The step loop, instantiated once per wave group so that each copy has a
  // fixed phase order (SECOND: X(j-1) then M(j); else M(j) then X(j)).
  auto run = [&](auto group) __attribute__((always_inline)) {
    constexpr bool SECOND = decltype(group)::value;
    // One step: K_{j+1} and V_j in flight, then this group's two phases.
    auto step = [&](int j, const char* __restrict__ kcur, const char* __restrict__ vprev, char* __restrict__ knxt,
                    char* __restrict__ vnxt) __attribute__((always_inline)) {
      if (j + 1 < n_tiles) issue_k(ts.at(j + 1) * BN, knxt);
      if (j < n_tiles) issue_v(ts.at(j) * BN, vnxt);
      opaque(kbase);
      opaque(vbase);
      if constexpr (SECOND) {
        softmax_phase(j - 1);
        exec_barrier();
        __builtin_amdgcn_s_setprio(1);
        mma_phase(j, kcur, vprev);
        __builtin_amdgcn_s_setprio(0);
      } else {
        __builtin_amdgcn_s_setprio(1);
        mma_phase(j, kcur, vprev);
        __builtin_amdgcn_s_setprio(0);
        exec_barrier();
        softmax_phase(j);
      }
      wait_vmem();
      __syncthreads();
    };
    if (n_tiles > 0) issue_k(ts.at(0) * BN, ks0);
    wait_vmem();
    __syncthreads();
    for (int j = 0; j <= n_tiles; j += 2) {
      step(j, ks0, vs1, ks1, vs0);
      if (j + 1 <= n_tiles) step(j + 1, ks1, vs0, ks0, vs1);
    }
  };
  if (second)
    run(BoolTag<true>{});
  else
    run(BoolTag<false>{});

  // ---- epilogue: O = acc / l, lse = ln(sum exp(s)); O = 0, lse = -inf for a row that kept no key ----
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
static hipError_t launch_fwd_pp(const FwdParams& p0, int B, int H, hipStream_t st) {
  FwdParams p = p0;
  p.n_qtiles = (p.N + C::BM - 1) / C::BM;
  const long long grid = (long long)p.n_qtiles * B * H;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (p.sk.r == p.sv.r)
    hipLaunchKernelGGL((fwd_pp_kernel<C, true>), dim3((unsigned)grid), dim3(C::NT), 0, st, p);
  else
    hipLaunchKernelGGL((fwd_pp_kernel<C, false>), dim3((unsigned)grid), dim3(C::NT), 0, st, p);
  return hipGetLastError();
}

template <class C>
static hipError_t launch_fwd_pipe(const FwdParams& p0, int B, int H, hipStream_t st) {
  FwdParams p = p0;
  p.n_qtiles = (p.N + C::BM - 1) / C::BM;
  const long long grid = (long long)p.n_qtiles * B * H;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (p.kv_index)  // block-sparse calls take contiguous layouts
    hipLaunchKernelGGL((fwd_pipe_kernel<C, true, true>), dim3((unsigned)grid), dim3(C::NT), 0, st, p);
  else if (p.sk.r == p.sv.r)
    hipLaunchKernelGGL((fwd_pipe_kernel<C, true, false>), dim3((unsigned)grid), dim3(C::NT), 0, st, p);
  else
    hipLaunchKernelGGL((fwd_pipe_kernel<C, false, false>), dim3((unsigned)grid), dim3(C::NT), 0, st, p);
  return hipGetLastError();
}

template <class C>
static hipError_t launch_fwd_direct(const FwdParams& p0, int B, int H, hipStream_t st) {
  FwdParams p = p0;
  p.n_qtiles = (p.N + C::BM - 1) / C::BM;
  const long long grid = (long long)p.n_qtiles * B * H;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (p.kv_index)
    hipLaunchKernelGGL((fwd_kernel<C, true, true>), dim3((unsigned)grid), dim3(C::NT), 0, st, p);
  else if (p.sk.r == p.sv.r)
    hipLaunchKernelGGL((fwd_kernel<C, true, false>), dim3((unsigned)grid), dim3(C::NT), 0, st, p);
  else
    hipLaunchKernelGGL((fwd_kernel<C, false, false>), dim3((unsigned)grid), dim3(C::NT), 0, st, p);
  return hipGetLastError();
}

// Parameter table: D -> (keys per tile BN, waves per workgroup, waves per SIMD).
// bf16 at D = 128 also has the phase-alternating kernel (eight waves, 64-key
// tiles) for the shapes where it is faster.
// Chosen so that two K/V stages fit LDS and, where registers allow, two
// workgroups share a CU (one wave's softmax overlaps the other's MFMAs).
hipError_t fwd_dispatch(Elt e, int D, const FwdParams& p, int B, int H, hipStream_t st) {
  switch (e) {
    case Elt::F32:
      if (D == 64) return launch_fwd_direct<FwdDCfg<Elt::F32, 64, 64, 4, 2>>(p, B, H, st);
      if (D == 128) return launch_fwd_direct<FwdDCfg<Elt::F32, 128, 32, 4, 1>>(p, B, H, st);
      if (D == 256) return launch_fwd_direct<FwdDCfg<Elt::F32, 256, 32, 4, 1>>(p, B, H, st);
      break;
    case Elt::BF16:
      if (D == 64) return launch_fwd_pipe<FwdDCfg<Elt::BF16, 64, 64, 4, 2>>(p, B, H, st);
      if (D == 128) {
        // the phase-alternating kernel where it measured faster: one query head
        // per K/V head, no window, fixed lengths and no block list (its 256-row
        // query tiles lose to 128-row ones on GQA and sliding windows)
        if (!p.kv_index && !p.cu_q && p.window < 0 && p.group == 1)
          return launch_fwd_pp<FwdPPCfg<128, 64>>(p, B, H, st);
        return launch_fwd_pipe<FwdDCfg<Elt::BF16, 128, 64, 4, 2>>(p, B, H, st);
      }
      if (D == 256) {
        // two waves per SIMD with O in AGPRs (fwd_lean.hip), except block-sparse launches
        if (!p.kv_index) return fwd_lean_dispatch(256, p, B, H, st);
        return launch_fwd_pipe<FwdDCfg<Elt::BF16, 256, 64, 4, 1>>(p, B, H, st);
      }
      break;
    case Elt::FP8:
      // e4m3 operands need few registers (121 / 166 VGPRs): four and three waves per SIMD;
      // at D = 256 the 128 accumulator registers leave two (one measured 1.7x slower)
      if (D == 64) return launch_fwd_direct<FwdDCfg<Elt::FP8, 64, 64, 4, 4>>(p, B, H, st);
      if (D == 128) return launch_fwd_direct<FwdDCfg<Elt::FP8, 128, 64, 4, 3>>(p, B, H, st);
      if (D == 256) return launch_fwd_direct<FwdDCfg<Elt::FP8, 256, 64, 4, 2>>(p, B, H, st);
      break;
  }
  return hipErrorInvalidValue;
}

bool fwd_supported(Elt e, int D) {
  return D == 64 || D == 128 || D == 256;
}

}  // namespace fa
