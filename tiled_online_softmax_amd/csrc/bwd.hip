// Backward attention kernels for gfx950 (bf16 in/out, float32 accumulation).
//
// The probabilities are recomputed from the forward's logsumexp,
// P = exp(s - lse), instead of being stored. With D_i = sum_d dO_id O_id:
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
// Two variants, both named on the page "FlashAttention (Metal Port)"
// (README, section "Documentation"):
//   * atomic: one pass over key tiles computes dK and dV and adds each key
//     tile's dQ contribution into a float32 scratch buffer with atomics
//     (FlashAttention-2's "scratch space for atomics and partial sums");
//   * deterministic: the same key-tile pass for dK and dV, plus a second pass
//     over query tiles that recomputes S and dP to form dQ -- 7 matrix
//     products instead of 5 and no atomics, parallel over both rows and
//     columns of the attention matrix.
//
// CDNA4 mapping. The key-tile kernel computes S = Q K^T with 32x32 MFMAs so a
// lane holds one key's scores for 16 queries: dV^T += dO^T P and
// dK^T += Q^T dS then take P and dS straight from registers, with K^T and V^T
// held in registers for the whole pass and Q, dO (row-major and transposed)
// streamed through double-buffered LDS. The query-tile dQ kernel mirrors the
// forward: S^T = K Q^T and dP^T = V dO^T put one query per lane, so lse and D
// are per-lane scalars, and dQ^T += K^T dS^T reads a transposed K tile.
#include "common.hpp"
#include "launch.hpp"

namespace fa {

constexpr float kInf = __builtin_huge_valf();

// ---------------------------------------------------------------------------
// D_i = sum_d dO_id O_id (float32); the atomic variant also zeroes dQ_accum.
// One thread per 8 consecutive elements of a row.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(const __bf16* __restrict__ o, const __bf16* __restrict__ dO,
                                                      float* __restrict__ delta, float* __restrict__ dq_accum,
                                                      long long rows) {
  constexpr int TPR = D / 8;  // threads per row
  const long long gt = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = gt / TPR;
  const int part = (int)(gt % TPR);
  float s = 0.f;
  if (row < rows) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(o + row * D + part * 8);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(dO + row * D + part * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) s += (float)a[i] * (float)b[i];
    if (dq_accum) {
      f32x4* z = reinterpret_cast<f32x4*>(dq_accum + row * D + part * 8);
      z[0] = f32x4{};
      z[1] = f32x4{};
    }
  }
#pragma unroll
  for (int o2 = TPR / 2; o2 > 0; o2 >>= 1) s += __shfl_xor(s, o2, 64);
  if (row < rows && part == 0) delta[row] = s;
}

// dQ = bf16(dQ_accum) (the scale is already applied).
__global__ void __launch_bounds__(256) bwd_dq_convert_kernel(const float* __restrict__ acc, __bf16* __restrict__ dq,
                                                             long long n8) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *reinterpret_cast<const f32x4*>(acc + 8 * i);
  const f32x4 b = *reinterpret_cast<const f32x4*>(acc + 8 * i + 4);
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[j] = (__bf16)a[j];
    r[4 + j] = (__bf16)b[j];
  }
  *reinterpret_cast<bf16x8*>(dq + 8 * i) = r;
}

// Writes the 8 bf16 of a 16-byte global chunk (row `row`, columns 8ch..8ch+7)
// into a transposed LDS tile T[col][perm16(row)] of RB bytes per column row.
template <int RB>
__device__ __forceinline__ void store_transposed_bf16(char* base, int row, int ch, const i32x4& data) {
  const int p = perm16(row);
  const unsigned short* e = reinterpret_cast<const unsigned short*>(&data);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<unsigned short*>(base + lds_off<RB>(8 * ch + i, p >> 3) + (p & 7) * 2) = e[i];
}

// ---------------------------------------------------------------------------
// Key-tile pass: dK, dV (and atomic dQ).
// ---------------------------------------------------------------------------
template <int D_, int NW_, int BQ_, int OCC_>
struct DkdvCfg {
  static constexpr int D = D_, NW = NW_, BQ = BQ_, OCC = OCC_;
  static constexpr int BK = 32 * NW;    // keys per workgroup (32 per wave)
  static constexpr int NT = 64 * NW;
  static constexpr int RB = D * 2;      // bytes per row-major Q / dO row
  static constexpr int RBT = BQ * 2;    // bytes per transposed row (BQ queries)
  static constexpr int Q_BYTES = BQ * RB;
  static constexpr int QT_BYTES = D * RBT;
  static constexpr int OFF_QT = Q_BYTES;
  static constexpr int OFF_DO = OFF_QT + QT_BYTES;
  static constexpr int OFF_DOT = OFF_DO + Q_BYTES;
  static constexpr int OFF_LSE = OFF_DOT + QT_BYTES;
  static constexpr int OFF_DELTA = OFF_LSE + BQ * 4;
  static constexpr int STAGE = OFF_DELTA + BQ * 4;
  static constexpr int RB_KT = BK * 2;  // transposed K rows (atomic variant)
  static constexpr int KT_BYTES = D * RB_KT;
  static constexpr int RB_DS = BK * 2;  // dS tile [BQ queries][BK keys]
  static constexpr int DS_BYTES = BQ * RB_DS;
  static constexpr int CPR = RB / 16;
  static constexpr int CPT = BQ * CPR / NT;  // 16-byte chunks per thread per Q (and dO) tile
  static constexpr int NP = RB / 32;         // K^T / V^T register pieces per lane
  static_assert((BQ * CPR) % NT == 0 && BQ % 32 == 0 && D % 32 == 0, "tile shape");
};

template <class C>
__device__ __forceinline__ void dkdv_load(const __amdgpu_buffer_rsrc_t& rq, const __amdgpu_buffer_rsrc_t& rdo,
                                          int q0, int tid, i32x4* qr, i32x4* dor) {
#pragma unroll
  for (int r = 0; r < C::CPT; ++r) {
    const int c = tid + C::NT * r;
    const uint32_t off = (uint32_t)(q0 + c / C::CPR) * C::RB + (c % C::CPR) * 16;
    qr[r] = buf_load16(rq, off);
    dor[r] = buf_load16(rdo, off);
  }
}

template <class C>
__device__ __forceinline__ void dkdv_store(char* st, int tid, const i32x4* qr, const i32x4* dor, float lse_l2,
                                           float dlt) {
#pragma unroll
  for (int r = 0; r < C::CPT; ++r) {
    const int c = tid + C::NT * r;
    const int row = c / C::CPR, ch = c % C::CPR;
    *reinterpret_cast<i32x4*>(st + lds_off<C::RB>(row, ch)) = qr[r];
    *reinterpret_cast<i32x4*>(st + C::OFF_DO + lds_off<C::RB>(row, ch)) = dor[r];
    store_transposed_bf16<C::RBT>(st + C::OFF_QT, row, ch, qr[r]);
    store_transposed_bf16<C::RBT>(st + C::OFF_DOT, row, ch, dor[r]);
  }
  if (tid < C::BQ) {
    reinterpret_cast<float*>(st + C::OFF_LSE)[tid] = lse_l2;
    reinterpret_cast<float*>(st + C::OFF_DELTA)[tid] = dlt;
  }
}

template <class C, bool ATOMIC>
__global__ void __launch_bounds__(C::NT)
__attribute__((amdgpu_waves_per_eu(C::OCC, C::OCC)))
bwd_dkdv_kernel(BwdParams P, int n_ktiles) {
  constexpr int D = C::D, BQ = C::BQ, NE = D / 32, NA = BQ / 32;
  constexpr int SMEM = 2 * C::STAGE + (ATOMIC ? C::KT_BYTES + C::DS_BYTES : 0);
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 31, hf = lane >> 5;

  const int G = gridDim.x;
  int w = blockIdx.x;
  if ((G & 7) == 0) w = (w & 7) * (G >> 3) + (w >> 3);
  const int bh = w / n_ktiles;
  const int kt = w % n_ktiles;  // ascending: under causal masking the first key tiles have the most work
  const int N = P.N;
  const int k0 = kt * C::BK;
  const int kw = k0 + 32 * wave;
  const int key = kw + li;

  const size_t head = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)((size_t)N * D * 2);
  const auto rq = make_rsrc(reinterpret_cast<const __bf16*>(P.q) + head, head_bytes);
  const auto rk = make_rsrc(reinterpret_cast<const __bf16*>(P.k) + head, head_bytes);
  const auto rv = make_rsrc(reinterpret_cast<const __bf16*>(P.v) + head, head_bytes);
  const auto rdo = make_rsrc(reinterpret_cast<const __bf16*>(P.dO) + head, head_bytes);
  const float* lse_h = P.lse + (size_t)bh * N;
  const float* dl_h = P.delta + (size_t)bh * N;

  // K^T and V^T pieces (B operands of S = Q K^T and dP = dO V^T).
  i32x4 kf[C::NP], vf[C::NP];
#pragma unroll
  for (int p = 0; p < C::NP; ++p) {
    kf[p] = buf_load16(rk, (uint32_t)key * C::RB + 32 * p + 16 * hf);
    vf[p] = buf_load16(rv, (uint32_t)key * C::RB + 32 * p + 16 * hf);
  }
  char* kt_lds = smem + 2 * C::STAGE;
  char* ds_lds = kt_lds + C::KT_BYTES;
  if constexpr (ATOMIC) {
    // K tile transposed: KT[d][perm16(key - k0)]
    constexpr int CH = C::BK * C::CPR;
    for (int c = tid; c < CH; c += C::NT) {
      const int row = c / C::CPR, ch = c % C::CPR;
      const i32x4 x = buf_load16(rk, (uint32_t)(k0 + row) * C::RB + ch * 16);
      store_transposed_bf16<C::RB_KT>(kt_lds, row, ch, x);
    }
  }

  f32x16 adk[NE], adv[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    adk[e] = f32x16{};
    adv[e] = f32x16{};
  }

  const int qt0 = P.causal ? k0 / BQ : 0;
  const int nq = (N + BQ - 1) / BQ;
  const float sl2 = P.scale_log2;

  i32x4 qr[C::CPT], dor[C::CPT];
  float lse_n = 0.f, dl_n = 0.f;
  auto fetch_rows = [&](int q0) {
    dkdv_load<C>(rq, rdo, q0, tid, qr, dor);
    if (tid < BQ) {
      const int q = q0 + tid;
      lse_n = q < N ? lse_h[q] * kLog2e : kInf;
      dl_n = q < N ? dl_h[q] : 0.f;
    }
  };
  fetch_rows(qt0 * BQ);
  dkdv_store<C>(smem, tid, qr, dor, lse_n, dl_n);
  __syncthreads();

  for (int it = qt0; it < nq; ++it) {
    const int q0 = it * BQ;
    const bool more = it + 1 < nq;
    if (more) fetch_rows(q0 + BQ);
    const char* st = smem + ((it - qt0) & 1) * C::STAGE;
    const float* lse_s = reinterpret_cast<const float*>(st + C::OFF_LSE);
    const float* dl_s = reinterpret_cast<const float*>(st + C::OFF_DELTA);

    const bool live = !P.causal || q0 + BQ - 1 >= kw;
    f32x16 s[NA], dp[NA];
    if (live) {
#pragma unroll
      for (int a = 0; a < NA; ++a) {
        s[a] = f32x16{};
        dp[a] = f32x16{};
#pragma unroll
        for (int p = 0; p < C::NP; ++p) {
          const i32x4 x = *reinterpret_cast<const i32x4*>(st + lds_off<C::RB>(32 * a + li, 2 * p + hf));
          s[a] = mfma_bf16(__builtin_bit_cast(bf16x8, x), __builtin_bit_cast(bf16x8, kf[p]), s[a]);
          const i32x4 y = *reinterpret_cast<const i32x4*>(st + C::OFF_DO + lds_off<C::RB>(32 * a + li, 2 * p + hf));
          dp[a] = mfma_bf16(__builtin_bit_cast(bf16x8, y), __builtin_bit_cast(bf16x8, vf[p]), dp[a]);
        }
      }
      // P = 2^(s*sl2 - lse*log2e) and dS = P (dP - D); rows are queries 32a + 8g + 4h + t.
      const bool mask = P.causal && q0 < kw + 31;
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int qb = 32 * a + 8 * g + 4 * hf;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse_s + qb);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(dl_s + qb);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int v = 4 * g + t;
            float pv = fast_exp2(__builtin_fmaf(s[a][v], sl2, -l4[t]));
            if (mask && key > q0 + qb + t) pv = 0.f;
            s[a][v] = pv;
            dp[a][v] = pv * (dp[a][v] - d4[t]);
          }
        }
      // dV^T += dO^T P ; dK^T += Q^T dS (contraction over 16-query chunks)
#pragma unroll
      for (int kc = 0; kc < BQ / 16; ++kc) {
        bf16x8 pb, db;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          pb[i] = (__bf16)s[kc >> 1][(kc & 1) * 8 + i];
          db[i] = (__bf16)dp[kc >> 1][(kc & 1) * 8 + i];
        }
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          const i32x4 x = *reinterpret_cast<const i32x4*>(st + C::OFF_DOT + lds_off<C::RBT>(32 * e + li, 2 * kc + hf));
          adv[e] = mfma_bf16(__builtin_bit_cast(bf16x8, x), pb, adv[e]);
          const i32x4 y = *reinterpret_cast<const i32x4*>(st + C::OFF_QT + lds_off<C::RBT>(32 * e + li, 2 * kc + hf));
          adk[e] = mfma_bf16(__builtin_bit_cast(bf16x8, y), db, adk[e]);
        }
      }
    }

    if constexpr (ATOMIC) {
      // dS (bf16) -> LDS as [query][perm16(key)], then dQ_tile += dS K over this
      // workgroup's BK keys, added into the float32 scratch with atomics.
      const int kp = perm16(32 * wave + li);
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int qr_ = 32 * a + (v >> 2) * 8 + 4 * hf + (v & 3);
          const __bf16 x = live ? (__bf16)dp[a][v] : (__bf16)0.f;
          *reinterpret_cast<__bf16*>(ds_lds + lds_off<C::RB_DS>(qr_, kp >> 3) + (kp & 7) * 2) = x;
        }
      __syncthreads();
      constexpr int NBLK = NA * NE;  // 32x32 blocks of the BQ x D dQ tile
      for (int blk = wave; blk < NBLK; blk += C::NW) {
        const int a = blk / NE, e = blk % NE;
        f32x16 c = f32x16{};
#pragma unroll
        for (int kc = 0; kc < C::BK / 16; ++kc) {
          const i32x4 x = *reinterpret_cast<const i32x4*>(ds_lds + lds_off<C::RB_DS>(32 * a + li, 2 * kc + hf));
          const i32x4 y = *reinterpret_cast<const i32x4*>(kt_lds + lds_off<C::RB_KT>(32 * e + li, 2 * kc + hf));
          c = mfma_bf16(__builtin_bit_cast(bf16x8, x), __builtin_bit_cast(bf16x8, y), c);
        }
        float* dst = P.dq_accum + ((size_t)bh * N) * D + 32 * e + li;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int q = q0 + 32 * a + (v >> 2) * 8 + 4 * hf + (v & 3);
          if (q < N) atomicAdd(dst + (size_t)q * D, c[v] * P.scale);
        }
      }
    }

    if (more) {
      float l = lse_n, d = dl_n;
      dkdv_store<C>(smem + ((it - qt0 + 1) & 1) * C::STAGE, tid, qr, dor, l, d);
    }
    __syncthreads();
  }

  if (key < N) {
    __bf16* dk = reinterpret_cast<__bf16*>(P.dk) + head + (size_t)key * D;
    __bf16* dv = reinterpret_cast<__bf16*>(P.dv) + head + (size_t)key * D;
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
  static constexpr int RBT = BN * 2;
  static constexpr int K_BYTES = BN * RB;
  static constexpr int OFF_V = K_BYTES;
  static constexpr int OFF_KT = 2 * K_BYTES;
  static constexpr int STAGE = OFF_KT + D * RBT;
  static constexpr int CPR = RB / 16;
  static constexpr int CPT = BN * CPR / NT;
  static constexpr int NP = RB / 32;
  static_assert((BN * CPR) % NT == 0 && BN % 32 == 0, "tile shape");
};

template <class C>
__global__ void __launch_bounds__(C::NT)
__attribute__((amdgpu_waves_per_eu(C::OCC, C::OCC)))
bwd_dq_kernel(BwdParams P, int n_qtiles) {
  constexpr int D = C::D, BN = C::BN, NB = BN / 32, NE = D / 32;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 31, hf = lane >> 5;

  const int G = gridDim.x;
  int w = blockIdx.x;
  if ((G & 7) == 0) w = (w & 7) * (G >> 3) + (w >> 3);
  const int bh = w / n_qtiles;
  int qt = w % n_qtiles;
  if (P.causal) qt = n_qtiles - 1 - qt;
  const int N = P.N;
  const int q0 = qt * C::BM;
  const int qw = q0 + 32 * wave;
  const int qrow = qw + li;

  const size_t head = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)((size_t)N * D * 2);
  const auto rq = make_rsrc(reinterpret_cast<const __bf16*>(P.q) + head, head_bytes);
  const auto rk = make_rsrc(reinterpret_cast<const __bf16*>(P.k) + head, head_bytes);
  const auto rv = make_rsrc(reinterpret_cast<const __bf16*>(P.v) + head, head_bytes);
  const auto rdo = make_rsrc(reinterpret_cast<const __bf16*>(P.dO) + head, head_bytes);

  i32x4 qf[C::NP], dof[C::NP];
#pragma unroll
  for (int p = 0; p < C::NP; ++p) {
    qf[p] = buf_load16(rq, (uint32_t)qrow * C::RB + 32 * p + 16 * hf);
    dof[p] = buf_load16(rdo, (uint32_t)qrow * C::RB + 32 * p + 16 * hf);
  }
  const float lse_l2 = qrow < N ? P.lse[(size_t)bh * N + qrow] * kLog2e : kInf;
  const float dlt = qrow < N ? P.delta[(size_t)bh * N + qrow] : 0.f;
  const float sl2 = P.scale_log2;

  f32x16 acc[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) acc[e] = f32x16{};

  const int kv_end = P.causal ? min(N, q0 + C::BM) : N;
  const int n_tiles = (kv_end + BN - 1) / BN;

  i32x4 kr[C::CPT], vr[C::CPT];
  auto load = [&](int key0) {
#pragma unroll
    for (int r = 0; r < C::CPT; ++r) {
      const int c = tid + C::NT * r;
      const uint32_t off = (uint32_t)(key0 + c / C::CPR) * C::RB + (c % C::CPR) * 16;
      kr[r] = buf_load16(rk, off);
      vr[r] = buf_load16(rv, off);
    }
  };
  auto store = [&](char* st) {
#pragma unroll
    for (int r = 0; r < C::CPT; ++r) {
      const int c = tid + C::NT * r;
      const int row = c / C::CPR, ch = c % C::CPR;
      *reinterpret_cast<i32x4*>(st + lds_off<C::RB>(row, ch)) = kr[r];
      *reinterpret_cast<i32x4*>(st + C::OFF_V + lds_off<C::RB>(row, ch)) = vr[r];
      store_transposed_bf16<C::RBT>(st + C::OFF_KT, row, ch, kr[r]);
    }
  };
  load(0);
  store(smem);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int key0 = t * BN;
    const bool more = t + 1 < n_tiles;
    if (more) load(key0 + BN);
    const char* st = smem + (t & 1) * C::STAGE;
    if (!P.causal || key0 <= qw + 31) {
      f32x16 s[NB], dp[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        s[b] = f32x16{};
        dp[b] = f32x16{};
#pragma unroll
        for (int p = 0; p < C::NP; ++p) {
          const i32x4 x = *reinterpret_cast<const i32x4*>(st + lds_off<C::RB>(32 * b + li, 2 * p + hf));
          s[b] = mfma_bf16(__builtin_bit_cast(bf16x8, x), __builtin_bit_cast(bf16x8, qf[p]), s[b]);
          const i32x4 y = *reinterpret_cast<const i32x4*>(st + C::OFF_V + lds_off<C::RB>(32 * b + li, 2 * p + hf));
          dp[b] = mfma_bf16(__builtin_bit_cast(bf16x8, y), __builtin_bit_cast(bf16x8, dof[p]), dp[b]);
        }
      }
      const bool need_mask = (key0 + BN > N) || (P.causal && key0 + BN - 1 > qw);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float pv = fast_exp2(__builtin_fmaf(s[b][v], sl2, -lse_l2));
          if (need_mask) {
            const int kk = key0 + 32 * b + (v >> 2) * 8 + 4 * hf + (v & 3);
            if (kk >= N || (P.causal && kk > qrow)) pv = 0.f;
          }
          dp[b][v] = pv * (dp[b][v] - dlt);
        }
#pragma unroll
      for (int kc = 0; kc < BN / 16; ++kc) {
        bf16x8 db;
#pragma unroll
        for (int i = 0; i < 8; ++i) db[i] = (__bf16)dp[kc >> 1][(kc & 1) * 8 + i];
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          const i32x4 x = *reinterpret_cast<const i32x4*>(st + C::OFF_KT + lds_off<C::RBT>(32 * e + li, 2 * kc + hf));
          acc[e] = mfma_bf16(__builtin_bit_cast(bf16x8, x), db, acc[e]);
        }
      }
    }
    if (more) store(smem + ((t + 1) & 1) * C::STAGE);
    __syncthreads();
  }

  if (qrow < N) {
    __bf16* dq = reinterpret_cast<__bf16*>(P.dq) + head + (size_t)qrow * D;
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

template <int D>
static hipError_t launch_pre(const BwdParams& p, long long rows, hipStream_t st) {
  const long long threads = rows * (D / 8);
  hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<const __bf16*>(p.o), reinterpret_cast<const __bf16*>(p.dO), p.delta, p.dq_accum,
                     rows);
  return hipGetLastError();
}

template <class KC, class QC>
static hipError_t launch_bwd(int variant, const BwdParams& p, int B, int H, hipStream_t st) {
  const long long rows = (long long)B * H * p.N;
  hipError_t e = launch_pre<KC::D>(p, rows, st);
  if (e != hipSuccess) return e;
  const int nk = (p.N + KC::BK - 1) / KC::BK;
  const long long gk = (long long)nk * B * H;
  if (gk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (variant == 0) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<KC, true>), dim3((unsigned)gk), dim3(KC::NT), 0, st, p, nk);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const long long n8 = rows * KC::D / 8;
    hipLaunchKernelGGL(bwd_dq_convert_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, p.dq_accum,
                       reinterpret_cast<__bf16*>(p.dq), n8);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((bwd_dkdv_kernel<KC, false>), dim3((unsigned)gk), dim3(KC::NT), 0, st, p, nk);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int nq = (p.N + QC::BM - 1) / QC::BM;
  const long long gq = (long long)nq * B * H;
  hipLaunchKernelGGL(bwd_dq_kernel<QC>, dim3((unsigned)gq), dim3(QC::NT), 0, st, p, nq);
  return hipGetLastError();
}

bool bwd_supported(int D) { return D == 64 || D == 128; }

// Parameter table for the backward: D -> (waves, query tile of the key pass,
// key tile of the dQ pass, waves per SIMD).
hipError_t bwd_dispatch(int D, int variant, const BwdParams& p, int B, int H, hipStream_t st) {
  if (D == 64) return launch_bwd<DkdvCfg<64, 4, 64, 1>, DqCfg<64, 4, 64, 2>>(variant, p, B, H, st);
  if (D == 128) return launch_bwd<DkdvCfg<128, 4, 32, 1>, DqCfg<128, 4, 64, 1>>(variant, p, B, H, st);
  return hipErrorInvalidValue;
}

}  // namespace fa
