// Shared device helpers for the gfx950 attention kernels: vector types,
// bounds-checked buffer loads, the LDS swizzle, MFMA wrappers and the
// wave-level reductions. CDNA4 only (wave64, MFMA, 160 KB LDS per CU).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

enum class Elt { F32, BF16, FP8 };

// Rows (and columns) of a block of a block-sparse mask.
constexpr int kBlock = 128;

template <Elt E> struct EltInfo;
template <> struct EltInfo<Elt::F32> { static constexpr int bytes = 4; };
template <> struct EltInfo<Elt::BF16> { static constexpr int bytes = 2; };
template <> struct EltInfo<Elt::FP8> { static constexpr int bytes = 1; };

// ---------------------------------------------------------------------------
// Buffer resources: loads past `bytes` return zero instead of faulting, which
// is how ragged tails (rows >= N) are read without branches.
// ---------------------------------------------------------------------------
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ i32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

__device__ __forceinline__ float buf_load4f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

// ---------------------------------------------------------------------------
// Row-major LDS tiles written by direct global->LDS loads.
//
// A tile holds rows of RB bytes, viewed as 256-byte lines (64 banks x 4 B)
// and 16-byte chunks. The chunk position inside a line is XOR-swizzled with
// a bijection of the row so that
//   * 16 lanes reading the same chunk of 16 consecutive rows (an MFMA operand
//     read with ds_read_b128) hit 16 different bank groups, and
//   * a ds_read_b64_tr_b16 over 4 consecutive rows x 64 bytes by 32 lanes
//     covers 64 different banks (rows differing in the two low bits land in
//     different 64-byte groups of the line).
// tile_off(row, chunk) is the byte offset of logical chunk `chunk` of `row`;
// tile_pos(phys16) inverts it for the loader, which writes lane-linear 16-byte
// positions.
// ---------------------------------------------------------------------------
__device__ __forceinline__ constexpr int swz16(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ constexpr int swz8(int x) { return ((x & 1) << 2) | ((x >> 1) & 3); }

template <int RB>
__device__ __forceinline__ constexpr uint32_t tile_off(int row, int chunk) {
  static_assert(RB == 64 || RB == 128 || RB % 256 == 0, "row size");
  if constexpr (RB >= 256) {
    constexpr int LPR = RB / 256;  // lines per row
    return (uint32_t)((row * LPR + (chunk >> 4)) * 256 + (((chunk & 15) ^ swz16(row & 15)) << 4));
  } else if constexpr (RB == 128) {
    return (uint32_t)((row >> 1) * 256 + (((row & 1) << 3) + ((chunk & 7) ^ swz8((row >> 1) & 7))) * 16);
  } else {
    return (uint32_t)((row >> 2) * 256 + (((row & 3) << 2) + ((chunk & 3) ^ ((row >> 2) & 3))) * 16);
  }
}

// Inverse of tile_off: physical 16-byte slot -> (row, logical chunk).
template <int RB>
__device__ __forceinline__ constexpr void tile_pos(int phys, int& row, int& chunk) {
  const int line = phys >> 4, pos = phys & 15;
  if constexpr (RB >= 256) {
    constexpr int LPR = RB / 256;
    row = line / LPR;
    chunk = (line % LPR) * 16 + (pos ^ swz16(row & 15));
  } else if constexpr (RB == 128) {
    row = 2 * line + (pos >> 3);
    chunk = (pos & 7) ^ swz8(line & 7);
  } else {
    row = 4 * line + (pos >> 2);
    chunk = (pos & 3) ^ (line & 3);
  }
}

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// 16 bytes per lane from a buffer straight into LDS at lds_base + 16 * lane.
__device__ __forceinline__ void buf_load_lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                               lds_void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 16, (int)voff, (int)soff, 0, 0);
}

// 4 bytes per lane from a buffer straight into LDS at lds_base + 4 * lane.
__device__ __forceinline__ void buf_load_lds4(__amdgpu_buffer_rsrc_t r, uint32_t voff, lds_void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 4, (int)voff, 0, 0, 0);
}

// Bytes from the first byte of row 0 to the last byte of row n-1 of a head
// whose rows are `rs` bytes apart and `row` bytes long (0 for no rows); the
// extent of the buffer resource over that head, so rows >= n read as zero.
__device__ __forceinline__ uint32_t head_span(int n, uint32_t rs, uint32_t row) {
  return n > 0 ? (uint32_t)(n - 1) * rs + row : 0u;
}

// One batch entry's query and key lengths and first packed rows. Without
// packed sequences (cu_q null) every entry has the launch's lengths. Packed
// offsets are clamped into [0, total] and the lengths to the launch's longest
// ones, so a malformed offset array cannot move an access outside the tensors.
struct Seq {
  int nq, nk, tq, tk;
};
__device__ __forceinline__ Seq seq_of(const int* cu_q, const int* cu_k, int b, int Nq, int Nk, int total_q,
                                      int total_k) {
  if (!cu_q) return {Nq, Nk, 0, 0};
  const int q0 = min(max(cu_q[b], 0), total_q), k0 = min(max(cu_k[b], 0), total_k);
  const int q1 = min(max(cu_q[b + 1], q0), total_q), k1 = min(max(cu_k[b + 1], k0), total_k);
  return {min(q1 - q0, Nq), min(k1 - k0, Nk), q0, k0};
}

// Transposing 8-byte LDS read of 16-bit elements (gfx950). Within each group
// of 16 lanes, lane j supplies the address of 4 consecutive elements M[j][0..3];
// lane j' receives M[4i + j'/4][j' % 4] for i = 0..3.
__device__ __forceinline__ s16x4 lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// Tile offset of the 8 bytes this lane reads with lds_read_tr16 when building
// the A operand X^T of a 32x32x16 MFMA from a row-major tile X (RB bytes per
// row): output rows are the 32 columns 32e.. of X, the contraction runs over 16
// rows of X, and slots 4u..4u+3 come from one read. CL selects the row order
// of those slots: CL = true gives X rows 8u + 4h + i (the order in which a 32x32
// accumulator lane holds its rows, h = lane / 32), CL = false gives 8h + 4u + i.
// Further 16-row contraction chunks add 16 * RB bytes.
template <int RB, bool CL>
__device__ __forceinline__ constexpr uint32_t tr16_off(int lane, int e, int u) {
  const int j = lane & 15, g = lane >> 4, h = g >> 1;
  const int row = CL ? (8 * u + 4 * h + (j >> 2)) : (8 * h + 4 * u + (j >> 2));
  const int chunk = 4 * e + 2 * (g & 1) + ((j & 3) >> 1);
  return tile_off<RB>(row, chunk) + 8 * (j & 1);
}

// XOR forms of per-lane operand offsets. The swizzle only permutes 16-byte
// chunks within a 256-byte line, so for the row sizes used here the offset of
// operand piece p (or of column block e, slot group u) is the offset of piece 0
// XOR a constant that is the same for every lane. A kernel can then keep one
// base register per operand kind and fold the constant in at each read rather
// than hold one offset register per piece. The *_ok() checks prove the identity
// for every lane at compile time.
//
// Row-major operand pieces: lane (row li < 32, half hf) reads logical chunk
// 2p + hf of row li.
__device__ __forceinline__ constexpr uint32_t piece_xor(int p) { return (uint32_t)p << 5; }
template <int RB, int NP>
__device__ __forceinline__ constexpr bool piece_xor_ok() {
  for (int li = 0; li < 32; ++li)
    for (int hf = 0; hf < 2; ++hf)
      for (int p = 0; p < NP; ++p)
        if (tile_off<RB>(li, 2 * p + hf) != (tile_off<RB>(li, hf) ^ piece_xor(p))) return false;
  return true;
}
// Transposed pieces read with lds_read_tr16.
template <int RB, bool CL>
__device__ __forceinline__ constexpr uint32_t tr16_xor(int e, int u) {
  return tr16_off<RB, CL>(0, e, u) ^ tr16_off<RB, CL>(0, 0, 0);
}
template <int RB, bool CL, int NE>
__device__ __forceinline__ constexpr bool tr16_xor_ok() {
  for (int lane = 0; lane < 64; ++lane)
    for (int e = 0; e < NE; ++e)
      for (int u = 0; u < 2; ++u)
        if (tr16_off<RB, CL>(lane, e, u) != (tr16_off<RB, CL>(lane, 0, 0) ^ tr16_xor<RB, CL>(e, u))) return false;
  return true;
}

// Hides a value's origin from the optimiser, so expressions computed from it
// inside a loop are not hoisted out of the loop into registers of their own.
template <class T>
__device__ __forceinline__ void opaque(T& x) {
  asm volatile("" : "+v"(x));
}
// The same for a wave-uniform value held in a scalar register.
template <class T>
__device__ __forceinline__ void opaque_s(T& x) {
  asm volatile("" : "+s"(x));
}

// Transposing 8-byte LDS read of 8-bit elements (gfx950). Within each group
// of 16 lanes, lane j supplies the address of 8 consecutive bytes M[j][0..7];
// lane j' receives M[2i + j'/8][j' % 8] for i = 0..7.
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
__device__ __forceinline__ i32x2 lds_read_tr8(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p));
}

// Tile offset of the 8 bytes this lane reads with lds_read_tr8 for the A
// operand V^T of a 32x32x64 fp8 MFMA from a row-major tile V (RB bytes per
// row): output rows are the 32 columns 32e.. of V, and read w (0..3) fills
// slots 8w..8w+7, which hold V rows 16w + 8(i/4) + 4h + i%4 (i = 0..7) -- the
// order in which two 32x32 accumulator blocks hold their rows. Further reads
// w add 16 * RB bytes, further 64-row chunks 64 * RB.
template <int RB>
__device__ __forceinline__ uint32_t tr8_off(int lane, int e) {
  const int j = lane & 15, g = lane >> 4, h = g >> 1;
  const int row = 8 * (j >> 3) + 4 * h + ((j >> 1) & 3);
  return tile_off<RB>(row, 2 * e + (g & 1)) + 8 * (j & 1);
}

// Workgroup -> (head, tile rank). blockIdx values are dealt round-robin to the
// 8 XCDs in dispatch order. Where every tile costs about the same: each XCD
// gets a contiguous run of workgroups (whole heads when the tile count
// allows), so the K/V of a head stay in one L2. Where costs are uneven
// (`uneven`, chosen by rank_major): under causal masking the tiles of a head
// cost from one to n_tiles units, and a head-by-head order leaves long
// workgroups for the end of the launch; there the order is rank-major
// (rank 0, the costliest tile, of every head first), which schedules the
// longest workgroups first. The `group` consecutive heads that share one K/V
// head stay on one XCD (whole groups u with u % 8 = x on XCD x) when the head
// count is a multiple of 8 * group, so their K/V tiles are fetched into one L2.
// (Giving each XCD a contiguous block of heads instead raised the backward
// key-tile pass's L2 misses by about half, with no change in its time.)
// Whether a launch takes wg_map's rank-major order. Packed sequences and
// block-sparse launches (`irregular`) always do: with the head-by-head order
// each XCD gets a contiguous run of whole heads or sequences, and tiles of
// very different cost end up bunched. Rank-major was 3x faster on 16 packed
// sequences of 17-4096 rows, non-causal (forward and backward) and 2.4x on a
// windowed packed forward. On a non-causal block-sparse backward it was 1.7x
// faster, with the forward within 1%. Otherwise causal launches do, except
// a forward whose window keeps every row to at most a quarter of the n keys:
// all its query tiles but a short ramp at the start cost the same, so the
// head-by-head order keeps each head's K/V in one L2 without a long tail (1-3%
// faster). The backward passes measured slower that way and keep the
// rank-major order under windows.
__device__ __forceinline__ bool rank_major(bool irregular, int causal, int window, int n, bool forward) {
  if (irregular) return true;
  if (!causal) return false;
  return !(forward && window >= 0 && 4LL * window <= n);
}

// Long causal forwards (`long_fwd`: dense, no window, at least kXcdHeadsMinTiles
// query tiles per head, K/V-group count a multiple of 8) take a third order:
// XCD x runs its K/V groups u = x, x + 8, ... one after another, each with
// its heads' tiles in rank-major order (costliest first). The workgroups live
// on an XCD then belong to one or two K/V groups and walk the same keys at
// about the same time, so their K/V tiles come from L2: on the e4m3 workload
// B1 H32 N32768 D128 the fetches past L2 fell from 4.3 to 0.85 GB per launch,
// the clock rose by 3% and the launch ran 1-2% faster. With fewer tiles per
// head the order loses balance (128 tiles of 64-dim e4m3 heads: 5% slower;
// 8 tiles, B4 H16 N2048: 39% slower), hence the bound.
constexpr int kXcdHeadsMinTiles = 256;

__device__ __forceinline__ bool long_causal_forward(bool irregular, int causal, int window) {
  return !irregular && causal && window < 0;
}

__device__ __forceinline__ void wg_map(int n_tiles, bool uneven, int group, int& bh, int& rank,
                                       bool long_fwd = false) {
  const int G = gridDim.x, g = blockIdx.x;
  if (uneven && long_fwd && n_tiles >= kXcdHeadsMinTiles && (G / n_tiles) % (8 * group) == 0) {
    const int x = g & 7, k = g >> 3;         // XCD, position in its dispatch sequence
    const int per = group * n_tiles;         // workgroups of one K/V group
    const int u = x + 8 * (k / per), r = k % per;
    bh = u * group + r % group;
    rank = r / group;
    return;
  }
  if (uneven) {
    const int BH = G / n_tiles;
    const int i = g % BH;
    if (BH % (8 * group) == 0) {
      const int j = i >> 3;
      bh = ((i & 7) + 8 * (j / group)) * group + j % group;
    } else {
      bh = i;
    }
    rank = g / BH;
  } else {
    const int w = (G & 7) == 0 ? (g & 7) * (G >> 3) + (g >> 3) : g;
    bh = w / n_tiles;
    rank = w % n_tiles;
  }
}

// Offsets of the LDS-DMA loads that fill a row-major tile of two tensors
// with the same tile shape (K and V, or Q and dO) whose rows are `ars` and
// `brs` bytes apart in memory. Slot i of a lane (1 KB block wave*LPW + i of the
// tile) reads tile row row0 + i * (1024 / RB) at chunk ch_i, so the second
// tensor's offset is the first one's plus row * (brs - ars) (32-bit modular
// arithmetic): one register per slot and one per lane serve both tensors.
template <int RB, int LPW, int NW>
__device__ __forceinline__ constexpr bool tile_rows_affine_ok() {
  for (int w = 0; w < NW; ++w)
    for (int lane = 0; lane < 64; ++lane) {
      int r0 = 0, c0 = 0;
      tile_pos<RB>(w * LPW * 64 + lane, r0, c0);
      for (int i = 0; i < LPW; ++i) {
        int r = 0, c = 0;
        tile_pos<RB>((w * LPW + i) * 64 + lane, r, c);
        if (r != r0 + i * (1024 / RB)) return false;
      }
    }
  return true;
}

// SAME: both tensors have the same row spacing (ars == brs); the second
// tensor then uses the first one's offsets.
template <int LPW, int RB, bool SAME>
struct TileLoader {
  static_assert(1024 % RB == 0, "a 1 KB block holds whole rows");
  uint32_t off[LPW];  // row_i * ars + 16 * ch_i
  uint32_t dlt;       // row0 * (brs - ars)
  uint32_t ars, brs;
  __device__ __forceinline__ TileLoader(int wave, int lane, uint32_t ars_, uint32_t brs_) : ars(ars_), brs(brs_) {
    dlt = 0;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      int row, ch;
      tile_pos<RB>((wave * LPW + i) * 64 + lane, row, ch);
      off[i] = (uint32_t)row * ars + (uint32_t)ch * 16;
      if (i == 0 && !SAME) dlt = (uint32_t)row * (brs - ars);
    }
  }
  // Byte offset of slot i of the first (a) or second (b) tensor for a tile
  // starting at row r0. The tile's scalar base goes through opaque_s (and the
  // per-lane delta through opaque, in place), so the compiler cannot split off
  // a loop-invariant part of the sum and hoist per-slot partial sums out of the
  // tile loop into registers of their own.
  __device__ __forceinline__ uint32_t a(int i, int r0) const {
    uint32_t base = (uint32_t)r0 * ars;
    opaque_s(base);
    return off[i] + base;
  }
  __device__ __forceinline__ uint32_t b(int i, int r0) {
    if constexpr (SAME) {
      return a(i, r0);
    } else {
      uint32_t base = (uint32_t)r0 * brs + (uint32_t)(i * (1024 / RB)) * (brs - ars);
      opaque_s(base);
      opaque(dlt);
      return off[i] + dlt + base;
    }
  }
};

// Keys that query row i keeps: key_lo(i) <= j <= key_hi(i). The causal
// diagonal of row i is key i + (nk - nq), so the last query row lines up with
// the last key (bottom-right alignment); a left window w >= 0 keeps only keys
// from i + (nk - nq) - w on. Both bounds are non-decreasing in i. Query rows
// past the end of a head get the bounds of the same formulas (their results
// are never stored). key_lo may exceed key_hi only for such rows.
struct KeyBounds {
  int nq, nk, causal, window;
  __device__ __forceinline__ int lo(int i) const { return window >= 0 ? max(0, i + nk - nq - window) : 0; }
  __device__ __forceinline__ int hi(int i) const { return causal ? min(nk - 1, i + nk - nq) : nk - 1; }
  // Queries that key row j is kept by: qlo(j) <= i <= qhi(j).
  __device__ __forceinline__ int qlo(int j) const { return causal ? max(0, j - (nk - nq)) : 0; }
  __device__ __forceinline__ int qhi(int j) const { return window >= 0 ? min(nq - 1, j - (nk - nq) + window) : nq - 1; }
  // Does the key tile [key0, key0 + bn) need masking for the 32 query rows qw .. qw + 31 (ragged
  // tail, causal diagonal or window start)? The terms are combined without short-circuit
  // evaluation: a chain of branches placed right after an MFMA chain gave the compiler a join
  // block reached by two paths, and on the shorter one it left too few wait states before the
  // VALU read of the MFMA result (stale accumulator values for the fp32 D = 256 forward).
  template <int BN>
  __device__ __forceinline__ bool mask_tile(int key0, int qw) const {
    return (key0 + BN > nk) | ((causal != 0) & (key0 + BN - 1 > hi(qw))) | ((window >= 0) & (key0 < lo(qw + 31)));
  }
};

// vmcnt(0): all of this wave's vector-memory operations (incl. LDS DMA) done.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup execution barrier without a memory fence. It waits for no
// outstanding memory operation (a fenced barrier waits for every LDS-DMA
// copy still in flight) and only keeps the compiler from moving memory
// accesses across it; for phase changes that read nothing written since the
// last fenced barrier.
__device__ __forceinline__ void exec_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float dot2_bf16_sum(int packed_pair, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed_pair), one, acc, false);
}

// ---------------------------------------------------------------------------
// MFMA wrappers (gfx950).
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// e4m3 x e4m3, K = 64, unit block scales (e8m0 127 = 2^0).
__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// e4m3 x e4m3, 16x16x128, unit block scales.
__device__ __forceinline__ f32x4 mfma_fp8_16(const i32x8& a, const i32x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
__device__ __forceinline__ f32x16 mfma_f32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Combine a value with the one held by the lane 32 away (the other half of a
// 32x32 accumulator column), with v_permlane32_swap: swapping the upper half
// of one copy with the lower half of another leaves, in every lane, its own
// value in one result and its partner's in the other.
__device__ __forceinline__ float pair_max32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bool wave_any(bool p) {
  return __builtin_amdgcn_ballot_w64(p) != 0;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two floats -> two e4m3 codes (round to nearest even) in the low (HI=false)
// or high 16 bits of `old`.
template <bool HI>
__device__ __forceinline__ int cvt_fp8x2(float a, float b, int old) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

// Float -> unsigned byte (rounded to nearest, clamped to [0, 255]) written
// into byte `sel` of `old`; the other bytes are kept (v_cvt_pk_u8_f32).
__device__ __forceinline__ unsigned cvt_u8(float a, unsigned sel, unsigned old) {
  return __builtin_amdgcn_cvt_pk_u8_f32(a, sel, old);
}

}  // namespace fa
