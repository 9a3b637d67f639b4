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
// from the score registers. V is stored transposed in LDS (with the key
// permutation of perm16/perm64) so every MFMA operand is one contiguous LDS
// read. Q stays in registers for the whole loop.
#include "common.hpp"
#include "launch.hpp"

namespace fa {

template <Elt E, int D_, int BN_, int NW_, int OCC_>
struct FwdCfg {
  static constexpr Elt elt = E;
  static constexpr int D = D_, BN = BN_, NW = NW_, OCC = OCC_;
  static constexpr int ESZ = EltInfo<E>::bytes;
  static constexpr int BM = 32 * NW;   // query rows per workgroup
  static constexpr int NT = 64 * NW;   // threads per workgroup
  static constexpr int RB_K = D * ESZ; // bytes per K row (global and LDS)
  static constexpr bool V_T = (E != Elt::F32);  // V transposed in LDS?
  static constexpr int RB_V = V_T ? BN * ESZ : D * ESZ;
  static constexpr int K_BYTES = BN * RB_K;
  static constexpr int V_BYTES = V_T ? D * RB_V : BN * RB_V;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int CPR = RB_K / 16;            // 16-byte chunks per global row
  static constexpr int CPT = BN * CPR / NT;        // chunks per thread per tile (K, and V)
  static constexpr int NP = RB_K / 32;             // 16-byte Q pieces per lane
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert((BN * CPR) % NT == 0, "tile must split evenly over threads");
  static_assert(E != Elt::FP8 || BN % 64 == 0, "fp8 contracts 64 keys per MFMA");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <class C>
__device__ __forceinline__ void load_kv_tile(const __amdgpu_buffer_rsrc_t& rk, const __amdgpu_buffer_rsrc_t& rv,
                                             int key0, int tid, i32x4* kr, i32x4* vr) {
#pragma unroll
  for (int r = 0; r < C::CPT; ++r) {
    const int c = tid + C::NT * r;
    const int row = c / C::CPR, ch = c % C::CPR;
    const uint32_t off = (uint32_t)(key0 + row) * C::RB_K + ch * 16;
    kr[r] = buf_load16(rk, off);
    vr[r] = buf_load16(rv, off);
  }
}

template <class C>
__device__ __forceinline__ void store_kv_tile(char* stage, int tid, const i32x4* kr, const i32x4* vr) {
  char* ks = stage;
  char* vs = stage + C::K_BYTES;
#pragma unroll
  for (int r = 0; r < C::CPT; ++r) {
    const int c = tid + C::NT * r;
    const int row = c / C::CPR, ch = c % C::CPR;
    *reinterpret_cast<i32x4*>(ks + lds_off<C::RB_K>(row, ch)) = kr[r];
    if constexpr (!C::V_T) {
      *reinterpret_cast<i32x4*>(vs + lds_off<C::RB_V>(row, ch)) = vr[r];
    } else if constexpr (C::elt == Elt::BF16) {
      // 8 values of row `row` (key), columns d = 8ch .. 8ch+7 -> Vt[d][perm16(key)]
      const int p = perm16(row);
      const unsigned short* e = reinterpret_cast<const unsigned short*>(&vr[r]);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<unsigned short*>(vs + lds_off<C::RB_V>(8 * ch + i, p >> 3) + (p & 7) * 2) = e[i];
    } else {
      const int p = perm64(row);
      const unsigned char* e = reinterpret_cast<const unsigned char*>(&vr[r]);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        *reinterpret_cast<unsigned char*>(vs + lds_off<C::RB_V>(16 * ch + i, p >> 4) + (p & 15)) = e[i];
    }
  }
}

template <class C>
__global__ void __launch_bounds__(C::NT)
__attribute__((amdgpu_waves_per_eu(C::OCC, C::OCC)))
fwd_kernel_staged(FwdParams P) {
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  constexpr int D = C::D, BN = C::BN, NB = BN / 32, NE = D / 32;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, hf = lane >> 5;

  // Workgroup -> (head, query tile). Consecutive workgroups go to different
  // XCDs (round-robin), so regroup: each XCD gets a contiguous run of heads
  // (K/V of a head stay in one L2); within a head, causal runs the longest
  // (last) query tiles first.
  const int G = gridDim.x;
  int w = blockIdx.x;
  if ((G & 7) == 0) w = (w & 7) * (G >> 3) + (w >> 3);
  const int bh = w / P.n_qtiles;
  int qt = w % P.n_qtiles;
  if (P.causal) qt = P.n_qtiles - 1 - qt;
  const int N = P.N;
  const int q0 = qt * C::BM;
  const int qw = q0 + 32 * wave;   // first query row of this wave
  const int qrow = qw + li;        // this lane's query row

  const size_t head_elems = (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)(head_elems * C::ESZ);
  const char* qh = reinterpret_cast<const char*>(P.q) + (size_t)bh * head_elems * C::ESZ;
  const char* kh = reinterpret_cast<const char*>(P.k) + (size_t)bh * head_elems * C::ESZ;
  const char* vh = reinterpret_cast<const char*>(P.v) + (size_t)bh * head_elems * C::ESZ;
  const auto rq = make_rsrc(qh, head_bytes);
  const auto rk = make_rsrc(kh, head_bytes);
  const auto rv = make_rsrc(vh, head_bytes);

  float sc = P.scale_log2;  // score -> base-2 exponent
  float tau = P.rescale_log2;
  float out_mul = 1.f;
  if constexpr (C::elt == Elt::FP8) {
    const float dq = P.q_descale ? *P.q_descale : 1.f;
    const float dk = P.k_descale ? *P.k_descale : 1.f;
    const float dv = P.v_descale ? *P.v_descale : 1.f;
    sc *= dq * dk;
    out_mul = dv * (1.f / 448.f);
    tau = 0.f;
  }

  // Q^T pieces (B operand of S^T = K Q^T): lane-half h holds bytes 32p+16h.
  i32x4 qf[C::NP];
#pragma unroll
  for (int p = 0; p < C::NP; ++p) qf[p] = buf_load16(rq, (uint32_t)qrow * C::RB_K + 32 * p + 16 * hf);

  f32x16 acc[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) acc[e] = f32x16{};
  float m_ref = -INFINITY, l_part = 0.f;

  const int kv_end = P.causal ? min(N, q0 + C::BM) : N;
  const int n_tiles = (kv_end + BN - 1) / BN;

  i32x4 kr[C::CPT], vr[C::CPT];
  load_kv_tile<C>(rk, rv, 0, tid, kr, vr);
  store_kv_tile<C>(smem, tid, kr, vr);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int key0 = t * BN;
    const bool more = (t + 1) < n_tiles;
    if (more) load_kv_tile<C>(rk, rv, key0 + BN, tid, kr, vr);
    const char* ks = smem + (t & 1) * C::STAGE;
    const char* vs = ks + C::K_BYTES;

    const bool wave_live = !P.causal || key0 <= qw + 31;
    if (wave_live) {
      // ---- S^T = K Q^T (fp32 accumulate) ----
      f32x16 s[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        s[b] = f32x16{};
        const int krow = 32 * b + li;
        if constexpr (C::elt == Elt::BF16) {
#pragma unroll
          for (int p = 0; p < C::NP; ++p) {
            const i32x4 a = *reinterpret_cast<const i32x4*>(ks + lds_off<C::RB_K>(krow, 2 * p + hf));
            s[b] = mfma_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qf[p]), s[b]);
          }
        } else if constexpr (C::elt == Elt::FP8) {
#pragma unroll
          for (int p = 0; p < C::NP; p += 2) {
            const i32x4 a0 = *reinterpret_cast<const i32x4*>(ks + lds_off<C::RB_K>(krow, 2 * p + hf));
            const i32x4 a1 = *reinterpret_cast<const i32x4*>(ks + lds_off<C::RB_K>(krow, 2 * p + 2 + hf));
            const i32x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            const i32x8 bq = {qf[p][0], qf[p][1], qf[p][2], qf[p][3], qf[p + 1][0], qf[p + 1][1], qf[p + 1][2], qf[p + 1][3]};
            s[b] = mfma_fp8(a, bq, s[b]);
          }
        } else {
#pragma unroll
          for (int p = 0; p < C::NP; ++p) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(ks + lds_off<C::RB_K>(krow, 2 * p + hf));
            const f32x4 bq = __builtin_bit_cast(f32x4, qf[p]);
#pragma unroll
            for (int u = 0; u < 4; ++u) s[b] = mfma_f32(a[u], bq[u], s[b]);
          }
        }
      }

      // ---- mask (causal diagonal / ragged tail) and tile row max ----
      const bool need_mask = (key0 + BN > N) || (P.causal && key0 + BN - 1 > qw);
      if (need_mask) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = key0 + 32 * b + (v >> 2) * 8 + hf * 4 + (v & 3);
            if (key >= N || (P.causal && key > qrow)) s[b][v] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[b][v]);
      mx = fmaxf(mx, xor32(mx)) * sc;

      // ---- conditional rescale: move the reference max only when it grew by > tau ----
      const bool grow = mx > m_ref + tau;
      if (wave_any(grow)) {
        const float m_new = grow ? mx : m_ref;
        const float alpha = fast_exp2(m_ref - m_new);
        m_ref = m_new;
        l_part *= alpha;
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[e] *= alpha;
      }

      // ---- probabilities p = 2^(s*sc - m_ref) and partial row sum ----
      const float neg_m = -m_ref;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = fast_exp2(__builtin_fmaf(s[b][v], sc, neg_m));
          s[b][v] = p;
          l_part += p;
        }

      // ---- O^T += V^T P^T ----
      if constexpr (C::elt == Elt::BF16) {
#pragma unroll
        for (int kc = 0; kc < BN / 16; ++kc) {
          const f32x16& sb = s[kc >> 1];
          const int o8 = (kc & 1) * 8;
          bf16x8 pb;
#pragma unroll
          for (int i = 0; i < 8; ++i) pb[i] = (__bf16)sb[o8 + i];
#pragma unroll
          for (int e = 0; e < NE; ++e) {
            const i32x4 a = *reinterpret_cast<const i32x4*>(vs + lds_off<C::RB_V>(32 * e + li, 2 * kc + hf));
            acc[e] = mfma_bf16(__builtin_bit_cast(bf16x8, a), pb, acc[e]);
          }
        }
      } else if constexpr (C::elt == Elt::FP8) {
#pragma unroll
        for (int kc = 0; kc < BN / 64; ++kc) {
          i32x8 pb;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const f32x16& sb = s[2 * kc + (j >> 2)];
            const int o = (j & 3) * 4;
            int w32 = cvt_fp8x2<false>(sb[o] * 448.f, sb[o + 1] * 448.f, 0);
            w32 = cvt_fp8x2<true>(sb[o + 2] * 448.f, sb[o + 3] * 448.f, w32);
            pb[j] = w32;
          }
#pragma unroll
          for (int e = 0; e < NE; ++e) {
            const i32x4 a0 = *reinterpret_cast<const i32x4*>(vs + lds_off<C::RB_V>(32 * e + li, 4 * kc + 2 * hf));
            const i32x4 a1 = *reinterpret_cast<const i32x4*>(vs + lds_off<C::RB_V>(32 * e + li, 4 * kc + 2 * hf + 1));
            const i32x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            acc[e] = mfma_fp8(a, pb, acc[e]);
          }
        }
      } else {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = 32 * b + (v >> 2) * 8 + hf * 4 + (v & 3);
#pragma unroll
            for (int e = 0; e < NE; ++e) {
              const int col = 32 * e + li;
              const float a = *reinterpret_cast<const float*>(vs + lds_off<C::RB_V>(key, col >> 2) + (col & 3) * 4);
              acc[e] = mfma_f32(a, s[b][v], acc[e]);
            }
          }
      }
    }

    if (more) store_kv_tile<C>(smem + ((t + 1) & 1) * C::STAGE, tid, kr, vr);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, lse = ln(sum exp(s)) ----
  const float l_tot = l_part + xor32(l_part);
  const float inv = out_mul / l_tot;
  if (qrow < N) {
    const size_t row_base = ((size_t)bh * N + qrow) * D;
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * e + 8 * g + 4 * hf;
        if constexpr (C::elt == Elt::F32) {
          f32x4 o4 = {acc[e][4 * g] * inv, acc[e][4 * g + 1] * inv, acc[e][4 * g + 2] * inv, acc[e][4 * g + 3] * inv};
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(P.o) + row_base + d) = o4;
        } else {
          bf16x4 o4 = {(__bf16)(acc[e][4 * g] * inv), (__bf16)(acc[e][4 * g + 1] * inv),
                       (__bf16)(acc[e][4 * g + 2] * inv), (__bf16)(acc[e][4 * g + 3] * inv)};
          *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(P.o) + row_base + d) = o4;
        }
      }
    if (hf == 0) P.lse[(size_t)bh * N + qrow] = (m_ref + __builtin_log2f(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Forward with direct global->LDS tile loads (float32 and bf16).
//
// K and V tiles are copied row-major into swizzled LDS tiles by LDS-DMA
// buffer loads (no register staging, no LDS store instructions). S^T = K Q^T
// reads K rows as MFMA A operands; for bf16 the P.V product reads V^T
// operands with transposing LDS reads (ds_read_b64_tr_b16), so V needs no
// transposed copy. The tile loop is unrolled by two so the stage base of
// every LDS read is an immediate.
// ---------------------------------------------------------------------------
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
  static_assert(E == Elt::F32 || E == Elt::BF16, "direct-load kernel is for f32 / bf16");
  static_assert(TILE % (1024 * NW) == 0, "tile must split into whole 1 KB loads per wave");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <int S> struct StageTag { static constexpr int value = S; };

template <class C>
__global__ void __launch_bounds__(C::NT)
__attribute__((amdgpu_waves_per_eu(C::OCC, C::OCC)))
fwd_kernel(FwdParams P) {
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
  constexpr int D = C::D, BN = C::BN, NB = C::NB, NE = C::NE, RB = C::RB, NP = C::NP;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, hf = lane >> 5;

  // Workgroup -> (head, query tile); see the staged kernel for the XCD regrouping.
  const int G = gridDim.x;
  int w = blockIdx.x;
  if ((G & 7) == 0) w = (w & 7) * (G >> 3) + (w >> 3);
  const int bh = w / P.n_qtiles;
  int qt = w % P.n_qtiles;
  if (P.causal) qt = P.n_qtiles - 1 - qt;
  const int N = P.N;
  const int q0 = qt * C::BM;
  const int qw = q0 + 32 * wave;
  const int qrow = qw + li;

  const size_t head_elems = (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)(head_elems * C::ESZ);
  const char* qh = reinterpret_cast<const char*>(P.q) + (size_t)bh * head_elems * C::ESZ;
  const char* kh = reinterpret_cast<const char*>(P.k) + (size_t)bh * head_elems * C::ESZ;
  const char* vh = reinterpret_cast<const char*>(P.v) + (size_t)bh * head_elems * C::ESZ;
  const auto rq = make_rsrc(qh, head_bytes);
  const auto rk = make_rsrc(kh, head_bytes);
  const auto rv = make_rsrc(vh, head_bytes);
  const float sc = P.scale_log2;
  const float tau = P.rescale_log2;

  // Loader: 16-byte slot `lane` of 1 KB block m of a tile comes from tile_pos(slot).
  uint32_t goff[C::LPW];
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) {
    int row, ch;
    tile_pos<RB>((wave * C::LPW + i) * 64 + lane, row, ch);
    goff[i] = (uint32_t)(row * RB + ch * 16);
  }
  auto issue = [&](int key0, int stage) {
    char* kb = smem + stage * C::STAGE;
    const uint32_t base = (uint32_t)key0 * RB;
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      const int m = wave * C::LPW + i;
      buf_load_lds16(rk, goff[i] + base, 0, (lds_void*)(kb + m * 1024));
      buf_load_lds16(rv, goff[i] + base, 0, (lds_void*)(kb + C::TILE + m * 1024));
    }
  };

  // Q^T pieces (B operand of S^T = K Q^T): lane-half h holds bytes 32p + 16h.
  i32x4 qf[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) qf[p] = buf_load16(rq, (uint32_t)qrow * RB + 32 * p + 16 * hf);

  // Per-lane LDS read offsets (tile-relative); blocks and key chunks add whole rows.
  uint32_t koff[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) koff[p] = tile_off<RB>(li, 2 * p + hf);
  uint32_t voff[NE][2];
  if constexpr (C::elt == Elt::BF16) {
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        voff[e][u] = tr16_off<RB, true>(lane, e, u);
  }

  f32x16 acc[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) acc[e] = f32x16{};
  float m_ref = -INFINITY, l_part = 0.f;

  const int kv_end = P.causal ? min(N, q0 + C::BM) : N;
  const int n_tiles = (kv_end + BN - 1) / BN;

  issue(0, 0);
  wait_vmem();
  __syncthreads();

  auto tile = [&](int t, auto stage_tag) {
    constexpr int S = decltype(stage_tag)::value;
    const int key0 = t * BN;
    const bool more = (t + 1) < n_tiles;
    if (more) issue(key0 + BN, S ^ 1);
    const char* ks = smem + S * C::STAGE;
    const char* vs = ks + C::TILE;
    if (!P.causal || key0 <= qw + 31) {
      // ---- S^T = K Q^T ----
      f32x16 s[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        s[b] = f32x16{};
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          if constexpr (C::elt == Elt::BF16) {
            const i32x4 a = *reinterpret_cast<const i32x4*>(ks + koff[p] + 32 * b * RB);
            s[b] = mfma_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qf[p]), s[b]);
          } else {
            const f32x4 a = *reinterpret_cast<const f32x4*>(ks + koff[p] + 32 * b * RB);
            const f32x4 bq = __builtin_bit_cast(f32x4, qf[p]);
#pragma unroll
            for (int u = 0; u < 4; ++u) s[b] = mfma_f32(a[u], bq[u], s[b]);
          }
        }
      }
      // ---- mask (causal diagonal / ragged tail) and tile row max ----
      if ((key0 + BN > N) || (P.causal && key0 + BN - 1 > qw)) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = key0 + 32 * b + (v >> 2) * 8 + hf * 4 + (v & 3);
            if (key >= N || (P.causal && key > qrow)) s[b][v] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[b][v]);
      mx = fmaxf(mx, xor32(mx)) * sc;
      // ---- conditional rescale ----
      const bool grow = mx > m_ref + tau;
      if (wave_any(grow)) {
        const float m_new = grow ? mx : m_ref;
        const float alpha = fast_exp2(m_ref - m_new);
        m_ref = m_new;
        l_part *= alpha;
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[e] *= alpha;
      }
      const float neg_m = -m_ref;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[b][v] = fast_exp2(__builtin_fmaf(s[b][v], sc, neg_m));
      // ---- O^T += V^T P^T ----
      if constexpr (C::elt == Elt::BF16) {
#pragma unroll
        for (int kc = 0; kc < BN / 16; ++kc) {
          const f32x16& sb = s[kc >> 1];
          const int o8 = (kc & 1) * 8;
          bf16x8 pb;
#pragma unroll
          for (int i = 0; i < 8; ++i) pb[i] = (__bf16)sb[o8 + i];
          const i32x4 pw = __builtin_bit_cast(i32x4, pb);
#pragma unroll
          for (int i = 0; i < 4; ++i) l_part = dot2_bf16_sum(pw[i], l_part);
#pragma unroll
          for (int e = 0; e < NE; ++e) {
            const s16x4 lo = lds_read_tr16(vs + voff[e][0] + kc * 16 * RB);
            const s16x4 hi = lds_read_tr16(vs + voff[e][1] + kc * 16 * RB);
            const s16x4 a8[2] = {lo, hi};
            acc[e] = mfma_bf16(__builtin_bit_cast(bf16x8, a8), pb, acc[e]);
          }
        }
      } else {
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
  };
  for (int t = 0; t < n_tiles; t += 2) {
    tile(t, StageTag<0>{});
    if (t + 1 < n_tiles) tile(t + 1, StageTag<1>{});
  }

  // ---- epilogue: O = acc / l, lse = ln(sum exp(s)) ----
  const float l_tot = l_part + xor32(l_part);
  const float inv = 1.f / l_tot;
  if (qrow < N) {
    const size_t row_base = ((size_t)bh * N + qrow) * D;
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * e + 8 * g + 4 * hf;
        if constexpr (C::elt == Elt::F32) {
          f32x4 o4 = {acc[e][4 * g] * inv, acc[e][4 * g + 1] * inv, acc[e][4 * g + 2] * inv, acc[e][4 * g + 3] * inv};
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(P.o) + row_base + d) = o4;
        } else {
          bf16x4 o4 = {(__bf16)(acc[e][4 * g] * inv), (__bf16)(acc[e][4 * g + 1] * inv),
                       (__bf16)(acc[e][4 * g + 2] * inv), (__bf16)(acc[e][4 * g + 3] * inv)};
          *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(P.o) + row_base + d) = o4;
        }
      }
    if (hf == 0) P.lse[(size_t)bh * N + qrow] = (m_ref + __builtin_log2f(l_tot)) * kLn2;
  }
}

template <class C>
static hipError_t launch_fwd_direct(const FwdParams& p0, int B, int H, hipStream_t st) {
  FwdParams p = p0;
  p.n_qtiles = (p.N + C::BM - 1) / C::BM;
  const long long grid = (long long)p.n_qtiles * B * H;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fwd_kernel<C>, dim3((unsigned)grid), dim3(C::NT), 0, st, p);
  return hipGetLastError();
}

template <class C>
static hipError_t launch_fwd(const FwdParams& p0, int B, int H, hipStream_t st) {
  FwdParams p = p0;
  p.n_qtiles = (p.N + C::BM - 1) / C::BM;
  const long long grid = (long long)p.n_qtiles * B * H;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fwd_kernel_staged<C>, dim3((unsigned)grid), dim3(C::NT), 0, st, p);
  return hipGetLastError();
}

// Parameter table: D -> (keys per tile BN, waves per workgroup, waves per SIMD).
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
      if (D == 64) return launch_fwd_direct<FwdDCfg<Elt::BF16, 64, 64, 4, 2>>(p, B, H, st);
      if (D == 128) return launch_fwd_direct<FwdDCfg<Elt::BF16, 128, 64, 4, 2>>(p, B, H, st);
      if (D == 256) return launch_fwd_direct<FwdDCfg<Elt::BF16, 256, 32, 4, 1>>(p, B, H, st);
      break;
    case Elt::FP8:
      if (D == 64) return launch_fwd<FwdCfg<Elt::FP8, 64, 64, 4, 2>>(p, B, H, st);
      if (D == 128) return launch_fwd<FwdCfg<Elt::FP8, 128, 64, 4, 2>>(p, B, H, st);
      break;
  }
  return hipErrorInvalidValue;
}

bool fwd_supported(Elt e, int D) {
  if (e == Elt::FP8) return D == 64 || D == 128;
  return D == 64 || D == 128 || D == 256;
}

}  // namespace fa
