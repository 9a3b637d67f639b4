// Backward attention kernels for gfx950 (bf16 in/out, float32 accumulation).
//
// The probabilities are recomputed from the forward's logsumexp,
// P = exp(s - lse), instead of being stored. With D_i = sum_d dO_id O_id:
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
// Two variants, both named on the page "FlashAttention (Metal Port)"
// (README, section "Documentation"):
//   * atomic: one pass over key tiles computes dK and dV and adds each key
//     tile's dQ contribution into a float32 scratch buffer with atomics
//     (FlashAttention-2 keeps scratch memory for those atomics and partial
//     sums);
//   * deterministic: the same key-tile pass for dK and dV, plus a second pass
//     over query tiles that recomputes S and dP to form dQ -- 7 matrix
//     products instead of 5 and no atomics, parallel over both rows and
//     columns of the attention matrix. The query-tile pass runs first and
//     also writes the row statistics the key-tile pass reads (it holds each
//     query row's dO anyway), so this variant needs no preprocess kernel.
//
// CDNA4 mapping. The key-tile kernel computes S = Q K^T with 32x32 MFMAs so a
// lane holds one key's scores for 16 queries: dV^T += dO^T P and
// dK^T += Q^T dS then take P and dS straight from registers, with K^T and V^T
// held in registers for the whole pass. Q and dO tiles are copied row-major
// into LDS by LDS-DMA loads and read both directly (S, dP) and transposed
// (ds_read_b64_tr_b16 for Q^T, dO^T). The query-tile dQ kernel mirrors the
// forward: S^T = K Q^T and dP^T = V dO^T put one query per lane, so lse and D
// are per-lane scalars, and dQ^T += K^T dS^T reads K^T with transposing reads.
#include "common.hpp"
#include "launch.hpp"

namespace fa {

constexpr float kInf = __builtin_huge_valf();

// ---------------------------------------------------------------------------
// Row statistics for the passes: ld[row] = lse * log2(e) and
// ld[rows + row] = -D with D = sum_d dO O (negated so it can initialise the
// dP accumulator, which then holds dP - D for free); the atomic variant also
// zeroes dQ_accum. One thread per 8 consecutive elements of a row. (The
// deterministic variant's dQ pass computes the same values, in the same
// order, for its own rows.)
//
// Workspace row r = (b * H + h) * Np + i is query row i of head h of entry b
// (packed sequences: Bp = 1 and i runs over all packed rows, which is the
// same row as cu_q[b] + i of entry b). A row that kept no key (lse = -inf)
// gets +inf, so every recomputed probability of it is 2^-inf = 0.
// ---------------------------------------------------------------------------
// Grid: `nb` blocks of 256 / TPR rows per head, for each of the Bp * H heads in turn.
template <int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(BwdParams P, int H, int Np, int nb) {
  constexpr int TPR = D / 8;  // threads per row
  const int bh = (int)blockIdx.x / nb, h = bh % H, b = bh / H;  // wave-uniform
  const int i = ((int)blockIdx.x - bh * nb) * (256 / TPR) + (int)threadIdx.x / TPR;
  const int part = (int)threadIdx.x % TPR;
  const bool in = i < Np;
  const long long row = (long long)bh * Np + i;
  float s = 0.f;
  if (in) {
    const __bf16* o = static_cast<const __bf16*>(P.o) + (b * P.so.b + h * P.so.h + i * P.so.r) + part * 8;
    const __bf16* dO = static_cast<const __bf16*>(P.dO) + (b * P.sdo.b + h * P.sdo.h + i * P.sdo.r) + part * 8;
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(o);
    const bf16x8 y = *reinterpret_cast<const bf16x8*>(dO);
#pragma unroll
    for (int j = 0; j < 8; ++j) s += (float)x[j] * (float)y[j];
    if (P.dq_accum) {
      f32x4* z = reinterpret_cast<f32x4*>(P.dq_accum + row * D + part * 8);
      z[0] = f32x4{};
      z[1] = f32x4{};
    }
  }
#pragma unroll
  for (int o2 = TPR / 2; o2 > 0; o2 >>= 1) s += __shfl_xor(s, o2, 64);
  if (in && part == 0) {
    const float l = P.lse[b * P.lse_b + h * P.lse_h + i];
    P.ld[row] = l == -kInf ? kInf : l * kLog2e;
    P.ld[P.rows + row] = -s;
  }
}

// dQ = bf16(dQ_accum) (the scale is already applied); rows and grid as in bwd_pre_kernel.
template <int D>
__global__ void __launch_bounds__(256) bwd_dq_convert_kernel(BwdParams P, int H, int Np, int nb) {
  constexpr int TPR = D / 8;
  const int bh = (int)blockIdx.x / nb, h = bh % H, b = bh / H;
  const int i = ((int)blockIdx.x - bh * nb) * (256 / TPR) + (int)threadIdx.x / TPR;
  if (i >= Np) return;
  const int part = (int)threadIdx.x % TPR;
  const long long row = (long long)bh * Np + i;
  const f32x4 a = *reinterpret_cast<const f32x4*>(P.dq_accum + row * D + part * 8);
  const f32x4 c = *reinterpret_cast<const f32x4*>(P.dq_accum + row * D + part * 8 + 4);
  bf16x8 v;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = (__bf16)a[j];
    v[4 + j] = (__bf16)c[j];
  }
  *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(P.dq) + (b * P.sdq.b + h * P.sdq.h + i * P.sdq.r) + part * 8) = v;
}

// ---------------------------------------------------------------------------
// Key-tile pass: dK, dV (and, for the atomic variant, dQ by float atomics).
// ---------------------------------------------------------------------------
template <int D_, int NW_, int BQ_, int OCC_>
struct DkdvCfg {
  static constexpr int D = D_, NW = NW_, BQ = BQ_, OCC = OCC_;
  static constexpr int BK = 32 * NW;    // keys per workgroup (32 per wave)
  static constexpr int NT = 64 * NW;
  static constexpr int RB = D * 2;      // bytes per Q / dO / K row
  static constexpr int QTILE = BQ * RB; // one Q (or dO) tile
  static constexpr int OFF_DO = QTILE;
  static constexpr int OFF_LD = 2 * QTILE;
  static constexpr int STAGE = 2 * QTILE + 1024;  // + lse*log2e and -D rows, 2*BQ*4 <= 1 KB
  static constexpr int KTILE = BK * RB;           // K tile (atomic variant)
  static constexpr int RB_DS = BQ * 2;            // dS^T tile: [key][query] bf16
  static constexpr int DSTILE = BK * RB_DS;
  static constexpr int LPW = QTILE / 1024 / NW;   // DMA loads per wave per Q (dO) tile
  static constexpr int KLPW = KTILE / 1024 / NW;
  static constexpr int NP = RB / 32;
  static constexpr int NA = BQ / 32, NE = D / 32;
  static_assert(QTILE % (1024 * NW) == 0 && BQ * 8 <= 1024 && BQ % 32 == 0, "tile shape");
  static_assert(RB_DS == 64 || RB_DS == 128 || RB_DS % 256 == 0, "dS tile row");
};

// PLAIN: Q and dO rows are equally spaced and every query tile's workspace
// rows start at a multiple of 4 (fixed lengths with Nq % 4 == 0), so one loader
// offset serves Q and dO and the per-row values arrive in 16-byte pieces.
// SPARSE: visit only the query tiles of the blocks listed for this key block.
template <class C, bool ATOMIC, bool PLAIN, bool SPARSE>
__global__ void __launch_bounds__(C::NT)
__attribute__((amdgpu_waves_per_eu(C::OCC, C::OCC)))
bwd_dkdv_kernel(BwdParams P, int n_ktiles) {
  constexpr int D = C::D, BQ = C::BQ, NE = C::NE, NA = C::NA, RB = C::RB, NP = C::NP;
  constexpr int SMEM = 2 * C::STAGE + (ATOMIC ? C::KTILE + C::DSTILE : 0);
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps per-wave branches scalar

  // Workgroup -> (K/V head, key tile); under causal masking the first key
  // tiles see the most query tiles: rank 0 is key tile 0. The K/V head's
  // `group` query heads are consecutive (h0 .. h0 + group - 1): the pass walks
  // the query tiles of every head of the group, which sums their dK and dV
  // contributions in the accumulators.
  int bh, kt;
  wg_map(n_ktiles, rank_major(P.cu_q != nullptr || P.kv_index != nullptr, P.causal, P.window, min(P.N, P.Nk), false), 1, bh, kt);
  const int group = P.group;
  const int hkv = P.hq / group;
  const int b = bh / hkv, hk = bh % hkv, h0 = hk * group;
  const Seq sq = seq_of(P.cu_q, P.cu_k, b, P.N, P.Nk, P.total_q, P.total_k);
  const int N = sq.nq;   // query rows per head of this entry
  const int NK = sq.nk;  // keys of this entry
  const int k0 = kt * C::BK;
  if (k0 >= NK) return;  // whole workgroup: a short packed sequence has fewer key tiles
  const KeyBounds kb{N, NK, P.causal, P.window};
  const int kw = k0 + 32 * wave;
  const int key = kw + li;

  const long long bb = P.cu_q ? 0 : b;  // packed sequences start at rows tq / tk instead
  const __bf16* qg = static_cast<const __bf16*>(P.q) + (bb * P.sq.b + h0 * P.sq.h + sq.tq * P.sq.r);
  const __bf16* dog = static_cast<const __bf16*>(P.dO) + (bb * P.sdo.b + h0 * P.sdo.h + sq.tq * P.sdo.r);
  const __bf16* kh = static_cast<const __bf16*>(P.k) + (bb * P.sk.b + hk * P.sk.h + sq.tk * P.sk.r);
  const __bf16* vh = static_cast<const __bf16*>(P.v) + (bb * P.sv.b + hk * P.sv.h + sq.tk * P.sv.r);
  const uint32_t qrs = (uint32_t)(P.sq.r * 2), dors = (uint32_t)(P.sdo.r * 2);
  const uint32_t qhs = (uint32_t)(P.sq.h * 2), dohs = (uint32_t)(P.sdo.h * 2);
  const uint32_t krs = (uint32_t)(P.sk.r * 2), vrs = (uint32_t)(P.sv.r * 2);
  // Q and dO of the whole group: head g's row i is at g * (head stride) + i * (row stride)
  const auto rq = make_rsrc(qg, N > 0 ? (uint32_t)(group - 1) * qhs + head_span(N, qrs, RB) : 0u);
  const auto rdo = make_rsrc(dog, N > 0 ? (uint32_t)(group - 1) * dohs + head_span(N, dors, RB) : 0u);
  const auto rk = make_rsrc(kh, head_span(NK, krs, RB));
  const auto rv = make_rsrc(vh, head_span(NK, vrs, RB));
  // lse*log2e of workspace row r at 4r, its -D at 4(rows + r); the group's
  // head g, query i is workspace row ld_row0 + g * ld_h + i.
  const auto rld = make_rsrc(P.ld, (uint32_t)(P.rows * 8));
  const uint32_t ld_row0 = (uint32_t)(bb * P.ld_b + h0 * P.ld_h + sq.tq), ld_h = (uint32_t)P.ld_h;
  const uint32_t ld_nd = (uint32_t)(P.rows * 4);

  // K^T and V^T pieces (B operands of S = Q K^T and dP = dO V^T).
  i32x4 kf[NP], vf[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    kf[p] = buf_load16(rk, (uint32_t)key * krs + 32 * p + 16 * hf);
    vf[p] = buf_load16(rv, (uint32_t)key * vrs + 32 * p + 16 * hf);
  }

  static_assert(tile_rows_affine_ok<RB, C::LPW, C::NW>(), "loader rows");
  TileLoader<C::LPW, RB, PLAIN> tl(wave, lane, qrs, dors);
  // Query tile of head g of the group starting at query i0.
  auto issue = [&](int g, int i0, char* st) {
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      const int m = wave * C::LPW + i;
      buf_load_lds16(rq, tl.a(i, i0) + (uint32_t)g * qhs, 0, (lds_void*)(st + m * 1024));
      buf_load_lds16(rdo, tl.b(i, i0) + (uint32_t)g * dohs, 0, (lds_void*)(st + C::OFF_DO + m * 1024));
    }
    if constexpr (PLAIN) {
      // lanes 0..BQ/4-1 bring lse*log2e of the tile's rows (4 per lane), the next BQ/4 lanes their -D
      if (wave == 0 && lane < BQ / 2) {
        const int half = lane >= BQ / 4, j = lane - half * (BQ / 4);
        const uint32_t r = ld_row0 + (uint32_t)g * ld_h + (uint32_t)i0;
        buf_load_lds16(rld, (half ? ld_nd : 0u) + 4 * r + 16 * j, 0, (lds_void*)(st + C::OFF_LD));
      }
    } else {
      // lanes 0..BQ-1 (of the first 2*BQ/64 waves) bring lse*log2e of the tile's rows, lanes BQ..2BQ-1 their -D
      if (wave < 2 * BQ / 64) {
        const int L = wave * 64 + lane, half = L >= BQ, j = L - half * BQ;
        const uint32_t r = ld_row0 + (uint32_t)g * ld_h + (uint32_t)(i0 + j);
        buf_load_lds4(rld, (half ? ld_nd : 0u) + 4 * r, (lds_void*)(st + C::OFF_LD + wave * 256));
      }
    }
  };

  char* kt_lds = smem + 2 * C::STAGE;
  char* ds_lds = kt_lds + C::KTILE;
  if constexpr (ATOMIC) {
#pragma unroll
    for (int i = 0; i < C::KLPW; ++i) {
      const int m = wave * C::KLPW + i;
      int row, ch;
      tile_pos<RB>(m * 64 + lane, row, ch);
      buf_load_lds16(rk, (uint32_t)(k0 + row) * krs + ch * 16, 0, (lds_void*)(kt_lds + m * 1024));
    }
  }

  // Per-lane LDS offsets, one base register per operand kind: piece p of a
  // row-major Q/dO operand sits at qbase ^ piece_xor(p), transposed piece
  // (e, u) at tbase ^ tr16_xor(e, u).
  static_assert(piece_xor_ok<RB, NP>() && tr16_xor_ok<RB, true, NE>(), "offset XOR form");
  uint32_t qbase = tile_off<RB>(li, hf);
  uint32_t tbase = tr16_off<RB, true>(lane, 0, 0);

  f32x16 adk[NE], adv[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    adk[e] = f32x16{};
    adv[e] = f32x16{};
  }

  // query tiles [qt0, nq) hold every query that keeps a key of this workgroup
  const int qt0 = kb.qlo(k0) / BQ;
  const int nq = kb.qhi(min(k0 + C::BK, NK) - 1) / BQ + 1;
  const float sl2 = P.scale_log2;

  // Query tiles visited, head by head of the group (dense: tiles [qt0, nq) of
  // each head; sparse: the tiles of the listed query blocks). A window can
  // leave the first keys with no query at all: then dK = dV = 0.
  static_assert(!SPARSE || C::BK == kBlock, "a key tile is one mask block");
  QueryTiles<SPARSE, BQ> qts(P, bb * P.hq + h0, kt, qt0, nq, group);
  if (qts.valid()) issue(qts.g, qts.row(), smem);
  wait_vmem();  // unconditional: no path reaches the tile loop with the register loads above pending
  __syncthreads();

  // One query tile. `cur` is read while the LDS-DMA prefetch fills `nxt`; the
  // restrict qualifiers (also on the dS^T and K tiles) tell the compiler these
  // regions are disjoint, so it does not wait for the prefetch before reading
  // them. The prefetch is waited for explicitly at the end of the tile.
  auto tile = [&](const char* __restrict__ cur, char* __restrict__ nxt, char* __restrict__ dsb,
                  const char* __restrict__ ktb) {
    const int q0 = qts.row();
    const int qh = qts.g;  // this tile's query head within the group
    QueryTiles<SPARSE, BQ> nx = qts;
    nx.advance();
    const bool more = nx.valid();
    if (more) issue(nx.g, nx.row(), nxt);
    const char* qs = cur;
    const char* dos = qs + C::OFF_DO;
    const float* lds_ld = reinterpret_cast<const float*>(qs + C::OFF_LD);
    opaque(qbase);
    opaque(tbase);

    const bool live = q0 + BQ - 1 >= kb.qlo(kw) && q0 <= kb.qhi(kw + 31);
    bf16x8 pb[BQ / 16], db[BQ / 16];  // P and dS as bf16 B operands, 16 queries per piece
    if (live) {
      f32x16 s[NA], dp[NA];
      // S = Q K^T and dP = dO V^T. The Q/dO pieces are read LA pieces ahead into
      // a register ring; scheduling barriers keep the reads ahead of the MFMAs
      // they feed, so LDS latency hides behind the MFMAs in between.
      constexpr int LA = D >= 128 ? 1 : 2;
#pragma unroll
      for (int a = 0; a < NA; ++a) {
        s[a] = f32x16{};
        // dP accumulator starts at -D of each row, so it ends as dP - D
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 nd = *reinterpret_cast<const f32x4*>(lds_ld + BQ + 32 * a + 8 * g + 4 * hf);
#pragma unroll
          for (int t = 0; t < 4; ++t) dp[a][4 * g + t] = nd[t];
        }
        i32x4 xq[LA + 1], xd[LA + 1];
        auto rd = [&](int p) {
          const uint32_t o = (qbase ^ piece_xor(p)) + 32 * a * RB;
          xq[p % (LA + 1)] = *reinterpret_cast<const i32x4*>(qs + o);
          xd[p % (LA + 1)] = *reinterpret_cast<const i32x4*>(dos + o);
        };
#pragma unroll
        for (int p = 0; p < LA; ++p) rd(p);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          if (p + LA < NP) rd(p + LA);
          __builtin_amdgcn_sched_barrier(0);
          s[a] = mfma_bf16(__builtin_bit_cast(bf16x8, xq[p % (LA + 1)]), __builtin_bit_cast(bf16x8, kf[p]), s[a]);
          dp[a] = mfma_bf16(__builtin_bit_cast(bf16x8, xd[p % (LA + 1)]), __builtin_bit_cast(bf16x8, vf[p]), dp[a]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // P = 2^(s*sl2 - lse*log2e); accumulator rows are queries 32a + 8g + 4h + t.
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 l2 = *reinterpret_cast<const f32x4*>(lds_ld + 32 * a + 8 * g + 4 * hf);
#pragma unroll
          for (int t = 0; t < 4; ++t) s[a][4 * g + t] = fast_exp2(__builtin_fmaf(s[a][4 * g + t], sl2, -l2[t]));
        }
      // Masked tiles only, as wave-uniform branches (opaque() on the bound keeps
      // the compiler from flattening them into selects run on every tile).
      // Element (a, v) is query q0 + 4h + r with r = 32a + 8(v/4) + v%4.
      const int off = kb.nk - kb.nq;  // the diagonal of query i is key i + off
      if (P.causal && q0 < kw + 31 - off) {  // causal diagonal: keep query >= key - off
        int lo = key - off - q0 - 4 * hf;
        opaque(lo);
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (32 * a + 8 * (v >> 2) + (v & 3) < lo) s[a][v] = 0.f;
      }
      if (q0 + BQ > N) {  // ragged tail: keep query < N
        int hi = N - q0 - 4 * hf;
        opaque(hi);
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (32 * a + 8 * (v >> 2) + (v & 3) >= hi) s[a][v] = 0.f;
      }
      if (kb.window >= 0 && q0 + BQ - 1 > kw - off + kb.window) {  // window: keep query <= key - off + window
        int hw = key - off + kb.window - q0 - 4 * hf;
        opaque(hw);
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (32 * a + 8 * (v >> 2) + (v & 3) > hw) s[a][v] = 0.f;
      }
      // dS = P (dP - D); both to bf16 pieces
#pragma unroll
      for (int kc = 0; kc < BQ / 16; ++kc)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float pv = s[kc >> 1][(kc & 1) * 8 + i];
          pb[kc][i] = (__bf16)pv;
          db[kc][i] = (__bf16)(pv * dp[kc >> 1][(kc & 1) * 8 + i]);
        }

      // dV^T += dO^T P ; dK^T += Q^T dS, over 16-query chunks kc and 32-column
      // blocks e; the transposed dO/Q pieces are read one step ahead.
      constexpr int NS = BQ / 16 * NE;
      s16x4 tx[2][2], ty[2][2];
      auto rdt = [&](int st) {
        const int kc = st / NE, e = st % NE;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const uint32_t o = (tbase ^ tr16_xor<RB, true>(e, u)) + kc * 16 * RB;
          tx[st & 1][u] = lds_read_tr16(dos + o);
          ty[st & 1][u] = lds_read_tr16(qs + o);
        }
      };
      rdt(0);
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const int kc = st / NE, e = st % NE;
        if (st + 1 < NS) rdt(st + 1);
        __builtin_amdgcn_sched_barrier(0);
        adv[e] = mfma_bf16(__builtin_bit_cast(bf16x8, tx[st & 1]), pb[kc], adv[e]);
        adk[e] = mfma_bf16(__builtin_bit_cast(bf16x8, ty[st & 1]), db[kc], adk[e]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    if constexpr (ATOMIC) {
      // dS^T (bf16) -> LDS [key][query]; each lane writes its 16 queries as 4 x 8 bytes.
      const int kr = 32 * wave + li;
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 x4;
#pragma unroll
          for (int t = 0; t < 4; ++t) x4[t] = live ? db[2 * a + (g >> 1)][4 * (g & 1) + t] : (__bf16)0.f;
          *reinterpret_cast<bf16x4*>(dsb + tile_off<C::RB_DS>(kr, 4 * a + g) + 8 * hf) = x4;
        }
      __syncthreads();
      // dQ tile (BQ x D) += dS K over this workgroup's BK keys; one 32x32 block per wave per step.
      for (int blk = wave; blk < NA * NE; blk += C::NW) {
        const int a = blk / NE, e = blk % NE;
        f32x16 c = f32x16{};
#pragma unroll
        for (int kc = 0; kc < C::BK / 16; ++kc) {
          const s16x4 x[2] = {lds_read_tr16(dsb + tr16_off<C::RB_DS, false>(lane, a, 0) + kc * 16 * C::RB_DS),
                              lds_read_tr16(dsb + tr16_off<C::RB_DS, false>(lane, a, 1) + kc * 16 * C::RB_DS)};
          const s16x4 y[2] = {lds_read_tr16(ktb + tr16_off<RB, false>(lane, e, 0) + kc * 16 * RB),
                              lds_read_tr16(ktb + tr16_off<RB, false>(lane, e, 1) + kc * 16 * RB)};
          c = mfma_bf16(__builtin_bit_cast(bf16x8, x), __builtin_bit_cast(bf16x8, y), c);
        }
        float* dst = P.dq_accum + ((size_t)ld_row0 + (size_t)qh * ld_h) * D + 32 * e + li;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int q = q0 + 32 * a + (v >> 2) * 8 + 4 * hf + (v & 3);
          if (q < N) atomicAdd(dst + (size_t)q * D, c[v] * P.scale);
        }
      }
    }

    if (more) wait_vmem();
    __syncthreads();
    qts = nx;
  };
  while (qts.valid()) {
    tile(smem, smem + C::STAGE, ds_lds, kt_lds);
    if (qts.valid()) tile(smem + C::STAGE, smem, ds_lds, kt_lds);
  }

  if (key < NK) {
    __bf16* dk = static_cast<__bf16*>(P.dk) + (bb * P.sdk.b + hk * P.sdk.h + (sq.tk + key) * P.sdk.r);
    __bf16* dv = static_cast<__bf16*>(P.dv) + (bb * P.sdv.b + hk * P.sdv.h + (sq.tk + key) * P.sdv.r);
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * e + 8 * g + 4 * hf;
        bf16x4 a4, b4;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          a4[t] = (__bf16)(adk[e][4 * g + t] * P.scale);
          b4[t] = (__bf16)adv[e][4 * g + t];
        }
        *reinterpret_cast<bf16x4*>(dk + d) = a4;
        *reinterpret_cast<bf16x4*>(dv + d) = b4;
      }
  }
}

// ---------------------------------------------------------------------------
// Query-tile pass: dQ without atomics (deterministic variant).
// ---------------------------------------------------------------------------
template <int D_, int NW_, int BN_, int OCC_>
struct DqCfg {
  static constexpr int D = D_, NW = NW_, BN = BN_, OCC = OCC_;
  static constexpr int BM = 32 * NW;
  static constexpr int NT = 64 * NW;
  static constexpr int RB = D * 2;
  static constexpr int TILE = BN * RB;
  static constexpr int STAGE = 2 * TILE;  // K tile, then V tile
  static constexpr int LPW = TILE / 1024 / NW;
  static constexpr int NP = RB / 32;
  static constexpr int NB = BN / 32, NE = D / 32;
  static_assert(TILE % (1024 * NW) == 0 && BN % 32 == 0, "tile shape");
};

// SAME: K and V rows are equally spaced. SPARSE: walk only the key tiles of
// the blocks listed for this query block.
template <class C, bool SAME, bool SPARSE>
__global__ void __launch_bounds__(C::NT)
__attribute__((amdgpu_waves_per_eu(C::OCC, C::OCC)))
bwd_dq_kernel(BwdParams P, int n_qtiles) {
  constexpr int D = C::D, BN = C::BN, NB = C::NB, NE = C::NE, RB = C::RB, NP = C::NP;
  __shared__ __attribute__((aligned(1024))) char smem[2 * C::STAGE];
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps per-wave branches scalar

  int bh, qt;
  wg_map(n_qtiles, rank_major(P.cu_q != nullptr || P.kv_index != nullptr, P.causal, P.window, min(P.N, P.Nk), false), P.group, bh, qt);
  const int b = bh / P.hq, h = bh % P.hq, hk = h / P.group;
  const Seq sq = seq_of(P.cu_q, P.cu_k, b, P.N, P.Nk, P.total_q, P.total_k);
  const int N = sq.nq;
  const int n_qt = (N + C::BM - 1) / C::BM;
  if (P.causal) qt = n_qt - 1 - qt;
  if (qt < 0 || qt >= n_qt) return;  // whole workgroup
  const int q0 = qt * C::BM;
  const int qw = q0 + 32 * wave;
  const int qrow = qw + li;

  const KeyBounds kb{N, sq.nk, P.causal, P.window};
  const long long bb = P.cu_q ? 0 : b;
  const __bf16* qh = static_cast<const __bf16*>(P.q) + (bb * P.sq.b + h * P.sq.h + sq.tq * P.sq.r);
  const __bf16* doh = static_cast<const __bf16*>(P.dO) + (bb * P.sdo.b + h * P.sdo.h + sq.tq * P.sdo.r);
  const __bf16* kh = static_cast<const __bf16*>(P.k) + (bb * P.sk.b + hk * P.sk.h + sq.tk * P.sk.r);
  const __bf16* vh = static_cast<const __bf16*>(P.v) + (bb * P.sv.b + hk * P.sv.h + sq.tk * P.sv.r);
  const uint32_t qrs = (uint32_t)(P.sq.r * 2), dors = (uint32_t)(P.sdo.r * 2);
  const uint32_t krs = (uint32_t)(P.sk.r * 2), vrs = (uint32_t)(P.sv.r * 2);
  const auto rq = make_rsrc(qh, head_span(N, qrs, RB));
  const auto rdo = make_rsrc(doh, head_span(N, dors, RB));
  const auto rk = make_rsrc(kh, head_span(sq.nk, krs, RB));
  const auto rv = make_rsrc(vh, head_span(sq.nk, vrs, RB));

  i32x4 qf[NP], dof[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    qf[p] = buf_load16(rq, (uint32_t)qrow * qrs + 32 * p + 16 * hf);
    dof[p] = buf_load16(rdo, (uint32_t)qrow * dors + 32 * p + 16 * hf);
  }
  // Row statistics of this lane's query row, written to the workspace for the
  // key-tile pass that runs after this one: lse * log2(e) and D = <dO, O>,
  // summed as bwd_pre_kernel sums them (8-element pieces, then pairs of
  // pieces 8, 4, 2, 1 apart; piece 2p + hf is this lane's piece p), so both
  // paths give bitwise the same values.
  const __bf16* oh = static_cast<const __bf16*>(P.o) + (bb * P.so.b + h * P.so.h + sq.tq * P.so.r);
  const uint32_t ors = (uint32_t)(P.so.r * 2);
  const auto ro = make_rsrc(oh, head_span(N, ors, RB));
  float dpart[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const bf16x8 ov = __builtin_bit_cast(bf16x8, buf_load16(ro, (uint32_t)qrow * ors + 32 * p + 16 * hf));
    const bf16x8 dv8 = __builtin_bit_cast(bf16x8, dof[p]);
    float t = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) t += (float)ov[j] * (float)dv8[j];
    dpart[p] = t;
  }
#pragma unroll
  for (int m = NP / 2; m >= 1; m >>= 1) {
    float t[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) t[p] = dpart[p] + dpart[p ^ m];
#pragma unroll
    for (int p = 0; p < NP; ++p) dpart[p] = t[p];
  }
  const float dlt = pair_sum32(dpart[0]);
  float lse_l2 = kInf;
  if (qrow < N) {
    const size_t r = (size_t)(bb * P.ld_b + h * P.ld_h + sq.tq) + qrow;  // workspace row
    const float l = P.lse[bb * P.lse_b + h * P.lse_h + sq.tq + qrow];
    lse_l2 = l == -kInf ? kInf : l * kLog2e;
    if (hf == 0) {
      P.ld[r] = lse_l2;
      P.ld[(size_t)P.rows + r] = -dlt;
    }
  }
  const float sl2 = P.scale_log2;

  static_assert(tile_rows_affine_ok<RB, C::LPW, C::NW>(), "loader rows");
  TileLoader<C::LPW, RB, SAME> tl(wave, lane, krs, vrs);
  auto issue = [&](int first_key, char* dst) {
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      const int m = wave * C::LPW + i;
      buf_load_lds16(rk, tl.a(i, first_key), 0, (lds_void*)(dst + m * 1024));
      buf_load_lds16(rv, tl.b(i, first_key), 0, (lds_void*)(dst + C::TILE + m * 1024));
    }
  };
  // One base register per operand kind (see the key-tile pass).
  static_assert(piece_xor_ok<RB, NP>() && tr16_xor_ok<RB, true, NE>(), "offset XOR form");
  uint32_t kbase = tile_off<RB>(li, hf);
  uint32_t tbase = tr16_off<RB, true>(lane, 0, 0);  // K^T operands, key order of the S^T accumulator

  f32x16 acc[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) acc[e] = f32x16{};

  // the workgroup's key tiles j = 0 .. n_tiles-1 (dense: every tile holding a
  // key one of its rows keeps; sparse: the tiles of the listed key blocks)
  static_assert(!SPARSE || (C::BM == kBlock && kBlock % BN == 0), "a query tile is one mask block");
  const KeyTiles<SPARSE, BN> ts(P, bh, kb, q0, q0 + C::BM);
  const int n_tiles = ts.n;

  if (n_tiles > 0) issue(ts.at_clamped(0) * BN, smem);
  wait_vmem();  // unconditional: no path reaches the tile loop with the register loads above pending
  __syncthreads();

  // One key tile; see the key-tile pass for the restrict qualifiers.
  int key0 = ts.at_clamped(0) * BN, key1 = ts.at_clamped(1) * BN;  // tiles j and j+1 (list reads run ahead)
  auto tile = [&](int j, const char* __restrict__ cur, char* __restrict__ nxt) {
    const int key2 = ts.at_clamped(j + 2) * BN;  // read now, used by the next tile
    const bool more = j + 1 < n_tiles;
    if (more) issue(key1, nxt);
    const char* ks = cur;
    const char* vs = ks + C::TILE;
    opaque(kbase);
    opaque(tbase);
    if (key0 <= kb.hi(qw + 31) && key0 + BN - 1 >= kb.lo(qw)) {
      // S^T = K Q^T and dP^T - D = V dO^T - D, K/V pieces read one piece ahead.
      f32x16 s[NB], dp[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        s[b] = f32x16{};
#pragma unroll
        for (int v = 0; v < 16; ++v) dp[b][v] = -dlt;
      }
      constexpr int LA = 1;
      i32x4 xk[LA + 1][NB], xv[LA + 1][NB];
      auto rd = [&](int p) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const uint32_t o = (kbase ^ piece_xor(p)) + 32 * b * RB;
          xk[p % (LA + 1)][b] = *reinterpret_cast<const i32x4*>(ks + o);
          xv[p % (LA + 1)][b] = *reinterpret_cast<const i32x4*>(vs + o);
        }
      };
#pragma unroll
      for (int p = 0; p < LA; ++p) rd(p);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        if (p + LA < NP) rd(p + LA);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < NB; ++b)
          s[b] = mfma_bf16(__builtin_bit_cast(bf16x8, xk[p % (LA + 1)][b]), __builtin_bit_cast(bf16x8, qf[p]), s[b]);
#pragma unroll
        for (int b = 0; b < NB; ++b)
          dp[b] = mfma_bf16(__builtin_bit_cast(bf16x8, xv[p % (LA + 1)][b]), __builtin_bit_cast(bf16x8, dof[p]), dp[b]);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[b][v] = fast_exp2(__builtin_fmaf(s[b][v], sl2, -lse_l2));
      // Masked tiles (causal diagonal, window start, ragged tail) only, as a
      // wave-uniform branch (see the key-tile pass). Element (b, v) is key
      // key0 + 4h + r with r = 32b + 8(v/4) + v%4, kept iff
      // key_lo(qrow) <= key <= key_hi(qrow).
      if (kb.mask_tile<BN>(key0, qw)) {
        int hi = kb.hi(qrow) - key0 - 4 * hf, lo = kb.lo(qrow) - key0 - 4 * hf;
        opaque(hi);
        opaque(lo);
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int r = 32 * b + 8 * (v >> 2) + (v & 3);
            if (r > hi || r < lo) s[b][v] = 0.f;
          }
      }
      // dS^T = P^T (dP^T - D) as bf16 pieces of 16 keys
      bf16x8 db[BN / 16];
#pragma unroll
      for (int kc = 0; kc < BN / 16; ++kc)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int b = kc >> 1, v = (kc & 1) * 8 + i;
          db[kc][i] = (__bf16)(s[b][v] * dp[b][v]);
        }
      // dQ^T += K^T dS^T over 16-key chunks kc and 32-column blocks e; the
      // transposed K pieces are read LB steps ahead.
      constexpr int NS = BN / 16 * NE, LB = 2;
      s16x4 tk[LB + 1][2];
      auto rdt = [&](int st) {
        const int kc = st / NE, e = st % NE;
#pragma unroll
        for (int u = 0; u < 2; ++u)
          tk[st % (LB + 1)][u] = lds_read_tr16(ks + (tbase ^ tr16_xor<RB, true>(e, u)) + kc * 16 * RB);
      };
#pragma unroll
      for (int st = 0; st < LB; ++st) rdt(st);
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        if (st + LB < NS) rdt(st + LB);
        __builtin_amdgcn_sched_barrier(0);
        acc[st % NE] = mfma_bf16(__builtin_bit_cast(bf16x8, tk[st % (LB + 1)]), db[st / NE], acc[st % NE]);
        __builtin_amdgcn_sched_barrier(0);
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

  if (qrow < N) {
    __bf16* dq = static_cast<__bf16*>(P.dq) + (bb * P.sdq.b + h * P.sdq.h + (sq.tq + qrow) * P.sdq.r);
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 a4;
#pragma unroll
        for (int t = 0; t < 4; ++t) a4[t] = (__bf16)(acc[e][4 * g + t] * P.scale);
        *reinterpret_cast<bf16x4*>(dq + 32 * e + 8 * g + 4 * hf) = a4;
      }
  }
}

// Workspace rows of the preprocess and the dQ convert: Bp entries of Np rows
// per head (packed sequences: one entry of all packed rows).
// Row blocks per head of the preprocess and dQ-convert grids.
template <int D>
static int row_blocks(int Np) {
  constexpr int RPB = 256 / (D / 8);  // rows per block
  return (Np + RPB - 1) / RPB;
}

template <int D>
static hipError_t launch_pre(const BwdParams& p, int H, hipStream_t st) {
  const int Np = p.cu_q ? p.total_q : p.N, nb = row_blocks<D>(Np);
  const long long grid = (long long)nb * (p.rows / Np);
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3((unsigned)grid), dim3(256), 0, st, p, H, Np, nb);
  return hipGetLastError();
}

template <class KCA, class KCD, class QC>
static hipError_t launch_bwd(int variant, const BwdParams& p, int B, int H, hipStream_t st) {
  const int HKV = H / p.group;  // the key-tile passes run over K/V heads
  // Q/dO equally spaced and workspace rows of every query tile 16-byte aligned
  const bool plain = p.sq.r == p.sdo.r && !p.cu_q && p.N % 4 == 0;
  // every grid is checked before anything is launched
  const int nka = (p.Nk + KCA::BK - 1) / KCA::BK, nkd = (p.Nk + KCD::BK - 1) / KCD::BK;
  const int nq = (p.N + QC::BM - 1) / QC::BM;
  const long long gka = (long long)nka * B * HKV, gkd = (long long)nkd * B * HKV, gq = (long long)nq * B * H;
  if ((variant == 0 ? gka : gkd) > 0x7fffffffLL || (variant == 1 && gq > 0x7fffffffLL))
    return hipErrorInvalidConfiguration;
  hipError_t e;
  if (variant == 1) {
    // dQ pass first: it also writes the row statistics the key-tile pass reads
    if (p.kv_index)  // block-sparse calls take contiguous layouts
      hipLaunchKernelGGL((bwd_dq_kernel<QC, true, true>), dim3((unsigned)gq), dim3(QC::NT), 0, st, p, nq);
    else if (p.sk.r == p.sv.r)
      hipLaunchKernelGGL((bwd_dq_kernel<QC, true, false>), dim3((unsigned)gq), dim3(QC::NT), 0, st, p, nq);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<QC, false, false>), dim3((unsigned)gq), dim3(QC::NT), 0, st, p, nq);
  } else if ((e = launch_pre<KCD::D>(p, H, st)) != hipSuccess) {
    return e;
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (variant == 0) {
    if (p.q_index)  // block-sparse
      hipLaunchKernelGGL((bwd_dkdv_kernel<KCA, true, false, true>), dim3((unsigned)gka), dim3(KCA::NT), 0, st, p, nka);
    else if (plain)
      hipLaunchKernelGGL((bwd_dkdv_kernel<KCA, true, true, false>), dim3((unsigned)gka), dim3(KCA::NT), 0, st, p, nka);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<KCA, true, false, false>), dim3((unsigned)gka), dim3(KCA::NT), 0, st, p, nka);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int Np = p.cu_q ? p.total_q : p.N, nb = row_blocks<KCA::D>(Np);
    hipLaunchKernelGGL(bwd_dq_convert_kernel<KCA::D>, dim3((unsigned)((long long)nb * (p.rows / Np))), dim3(256), 0,
                       st, p, H, Np, nb);
    return hipGetLastError();
  }
  if (p.q_index)  // block-sparse
    hipLaunchKernelGGL((bwd_dkdv_kernel<KCD, false, false, true>), dim3((unsigned)gkd), dim3(KCD::NT), 0, st, p, nkd);
  else if (plain)
    hipLaunchKernelGGL((bwd_dkdv_kernel<KCD, false, true, false>), dim3((unsigned)gkd), dim3(KCD::NT), 0, st, p, nkd);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<KCD, false, false, false>), dim3((unsigned)gkd), dim3(KCD::NT), 0, st, p, nkd);
  return hipGetLastError();
}

bool bwd_supported(int D) { return D == 64 || D == 128 || D == 256; }

// Parameter table for the backward: D -> key pass with atomic dQ (waves,
// query tile, waves per SIMD), key pass without, and the dQ pass (waves, key
// tile, waves per SIMD). The atomic pass holds a K tile and a dS^T tile in LDS
// on top of the stages, so it runs one workgroup per CU with larger query tiles;
// the plain key pass uses 32-query tiles, which fit three waves per SIMD at
// D=64 and two at D=128; the D=64 dQ pass likewise takes 32-key tiles to run
// three waves per SIMD.
hipError_t bwd_dispatch(int D, int variant, const BwdParams& p, int B, int H, hipStream_t st) {
  if (D == 64)
    return launch_bwd<DkdvCfg<64, 4, 64, 2>, DkdvCfg<64, 4, 32, 3>, DqCfg<64, 4, 32, 3>>(variant, p, B, H, st);
  if (D == 128)
    return launch_bwd<DkdvCfg<128, 4, 64, 1>, DkdvCfg<128, 4, 32, 2>, DqCfg<128, 4, 64, 2>>(variant, p, B, H, st);
  if (D == 256)
    return launch_bwd<DkdvCfg<256, 4, 32, 1>, DkdvCfg<256, 4, 32, 1>, DqCfg<256, 4, 32, 1>>(variant, p, B, H, st);
  return hipErrorInvalidValue;
}

}  // namespace fa
