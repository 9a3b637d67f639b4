/*
 * libfa -- exact FlashAttention-style attention for AMD MI355X (gfx950).
 *
 * The operation. For each batch b and head h, with q_i, k_j, v_j the rows of
 * Q, K, V ([N, D] slices of [B, H, N, D] tensors):
 *     s_ij  = scale * <q_i, k_j>             (causal: only keys j <= i are kept)
 *     O_i   = sum_j softmax_j(s_ij) v_j
 *     lse_i = ln sum_j exp(s_ij)              (natural log)
 * computed without materialising the N x N score matrix: K/V are walked in
 * tiles, a running row max and sum are kept, and the output is normalised
 * once at the end. The pages give tiling with an online softmax as the
 * FA1 baseline (page "r/mlscaling", FA1 bullet), with query-tile ownership and
 * deferred normalisation (FA2 bullet), ping-pong tile buffers and an FP8
 * forward (FA3 bullet), and conditional rescaling (FA4 bullet), all keeping
 * the exact attention result (closing sentence of that list). The backward
 * recomputes the probabilities from lse instead of storing them; the pages
 * name both the atomics-based backward of FlashAttention-2 and an
 * atomics-free alternative that spends more matrix multiplies ("FlashAttention
 * (Metal Port)" README, section "Documentation").
 *
 * Layout: Q, K, V, O, dO, dQ, dK, dV are contiguous row-major [B, H, N, D];
 * lse is contiguous float32 [B, H, N]. Query and key lengths are equal except
 * in the _general, _strided and _varlen entry points, and K/V heads may be
 * fewer than query heads in all of those and the _gqa ones. The _strided entry
 * points take any element strides for the batch, head and row dimensions (the
 * head dimension D contiguous); the _varlen ones take packed variable-length
 * batches.
 *
 * Rows that keep no key (causal with Nk < Nq leaves the first Nq - Nk rows
 * so; a packed sequence may have no keys): O = 0, lse = -inf, and their
 * gradients are 0 -- the sum over their keys is empty.
 *
 * Ownership: the caller allocates and owns every buffer (device memory).
 * The library never allocates, frees or synchronises, and keeps no state
 * except a per-thread error string. Every call is asynchronous on `stream`
 * (a hipStream_t passed as void*; NULL is the default stream). Device-side
 * faults surface at the caller's next synchronisation, as with any HIP call.
 *
 * Errors: every entry point returns an fa_status. Arguments are validated
 * before any HIP call (so validation works without a GPU); on failure
 * fa_last_error() describes the problem. FA_ERR_INVALID_ARG: null pointer,
 * B/H/N/D < 1, scale not > 0 or not finite, causal not 0/1, a pointer not
 * 16-byte aligned, or one head larger than 2^31 bytes. FA_ERR_UNSUPPORTED: D
 * not in the parameter table or a dtype/pass pair that is not built.
 * FA_ERR_WORKSPACE: workspace too small. FA_ERR_HIP: a HIP launch error
 * (hipGetErrorString text in fa_last_error()).
 */
#ifndef LIBFA_FA_H
#define LIBFA_FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_F32 = 0, FA_BF16 = 1, FA_FP8_E4M3 = 2 } fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1,
  FA_ERR_UNSUPPORTED = 2,
  FA_ERR_WORKSPACE = 3,
  FA_ERR_HIP = 4
} fa_status;

/* Backward variants (see fa_bwd). */
enum { FA_BWD_ATOMIC = 0, FA_BWD_DETERMINISTIC = 1 };

/*
 * Forward pass.
 *   q, k, v : [B, H, N, D] of `dtype` (FA_F32: float; FA_BF16: bfloat16;
 *             FA_FP8_E4M3: OCP e4m3 codes with unit scales -- use
 *             fa_fwd_fp8 for per-tensor scales).
 *   o       : [B, H, N, D] output; float for FA_F32, bfloat16 otherwise.
 *   lse     : [B, H, N] float output, natural-log logsumexp of the scaled
 *             scores of each query row (what fa_bwd consumes).
 *   D       : head dimension: 64, 128 or 256 (every dtype).
 *   causal  : 1 keeps key j only for query i >= j.
 *   scale   : factor on q.k, > 0 and finite (usually 1/sqrt(D)).
 * Rows are rescaled when their running max grows by more than 8 in base-2
 * units (FA_FP8_E4M3: by more than 2), which is exact in exact arithmetic.
 * Inputs must be finite: a NaN or infinite element gives undefined rows (the
 * e4m3 forward, for one, encodes a NaN score as probability 0 on most tiles
 * rather than propagating it).
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int D, int causal, float scale, int dtype,
           void* stream);

/*
 * Grouped-query forward: K and V have Hkv heads, each shared by H / Hkv
 * consecutive query heads -- query head h (0 <= h < H) attends with K/V head
 * h / (H / Hkv) of the same batch entry. Hkv = H is fa_fwd; Hkv = 1 is
 * multi-query attention. (Grouped-query attention is the variant the
 * "FlashAttention" entity trail page, section "Corpus findings", reports
 * attention kernels being carried over to, AVO entry.)
 *   q, o   : [B, H, N, D];  k, v : [B, Hkv, N, D];  lse : [B, H, N].
 *   dtype  : FA_F32 or FA_BF16 (D as for fa_fwd), or FA_FP8_E4M3 with unit
 *            scales. FA_ERR_INVALID_ARG if Hkv < 1 or Hkv does not divide H.
 * Other arguments, numerics and errors as for fa_fwd.
 */
int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int Hkv, int N, int D, int causal, float scale,
               int dtype, void* stream);

/*
 * General forward: grouped K/V heads (as fa_fwd_gqa), query and key lengths
 * that differ, and an optional left window.
 *   q, o   : [B, H, Nq, D];  k, v : [B, Hkv, Nk, D];  lse : [B, H, Nq].
 *   causal : 1 keeps key j for query i only if j <= i + (Nk - Nq): the causal
 *            diagonal is aligned at the bottom right, so the last query sees
 *            every key, as when new queries extend a cached prefix of keys
 *            (the KV-cache prefill of the FlashPrefill V2 entry on the
 *            "FlashAttention" entity trail page, section "Corpus findings").
 *            With Nk < Nq the first Nq - Nk rows keep no key (O = 0,
 *            lse = -inf).
 *   window : -1, or w >= 0 to keep only keys j >= i + (Nk - Nq) - w -- with
 *            causal, a sliding window of the w + 1 keys ending at the
 *            diagonal (the local sliding-window attention of the WAND entry
 *            on the "attention mechanism" tag page). Tiles wholly outside a
 *            row's keys are skipped.
 * Nq = Nk = N with window = -1 is fa_fwd_gqa. Other arguments as for
 * fa_fwd; FA_ERR_INVALID_ARG also for Nk < 1 or window < -1.
 */
int fa_fwd_general(const void* q, const void* k, const void* v, void* o,
                   float* lse, int B, int H, int Hkv, int Nq, int Nk, int D,
                   int causal, int window, float scale, int dtype, void* stream);

/*
 * Strided forward: fa_fwd_general on tensors with any element strides, e.g.
 * [B, N, H, D] (the layout of a projection output viewed per head) or views of
 * a packed QKV tensor. The pages name general strides only as part of the
 * KV-cache prefill and batching work (FlashPrefill V2 entry, "FlashAttention"
 * entity trail page, section "Corpus findings"); the layout is the caller's.
 *   strides : host array of 14 element strides -- q (batch, head, row),
 *             k (batch, head, row), v (batch, head, row), o (batch, head, row),
 *             lse (batch, head). Element (b, h, i, d) of q is
 *             q[b*s0 + h*s1 + i*s2 + d]; lse rows are contiguous. Read during
 *             the call only.
 * FA_ERR_INVALID_ARG if strides is NULL, a stride is negative, a row stride
 * is < D, or a batch/head/row stride of q, k, v, o is not a multiple of 16
 * bytes; FA_ERR_UNSUPPORTED if one head's rows (plus a tile of padding rows)
 * span 2^31 bytes or more. Other arguments as for fa_fwd_general.
 */
int fa_fwd_strided(const void* q, const void* k, const void* v, void* o,
                   float* lse, int B, int H, int Hkv, int Nq, int Nk, int D,
                   int causal, int window, float scale, int dtype,
                   const long long* strides, void* stream);

/*
 * Variable-length forward over a packed batch: B independent sequences whose
 * rows are concatenated (the continuous batching of the FlashPrefill V2 entry
 * on the "FlashAttention" entity trail page, section "Corpus findings").
 *   q, o          : [total_q, H, D];  k, v : [total_k, Hkv, D];
 *   lse           : [H, total_q] float.
 *   cu_seqlens_q  : device int32 [B + 1]: sequence b is rows
 *                   cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of q, o and lse;
 *                   cu_seqlens_k likewise for k and v. Offsets must be
 *                   non-decreasing from 0 to total; the kernels clamp them into
 *                   [0, total] (so no access leaves the tensors) but rows of
 *                   malformed sequences are then not defined.
 *   max_seqlen_q, max_seqlen_k : upper bounds of the lengths (they size the
 *                   launch; rows past them are not computed).
 * causal and window apply inside each sequence with its own lengths (the
 * bottom-right diagonal of fa_fwd_general). Other arguments as for
 * fa_fwd_general; FA_ERR_INVALID_ARG also for a NULL or misaligned offset
 * array or total_q, total_k < 1.
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o,
                  float* lse, const int* cu_seqlens_q, const int* cu_seqlens_k,
                  int B, int H, int Hkv, int total_q, int total_k,
                  int max_seqlen_q, int max_seqlen_k, int D, int causal,
                  int window, float scale, int dtype, void* stream);

/*
 * Block lists of a block-sparse mask. Block sparsity keeps or drops whole
 * 128 x 128 blocks of the score matrix: score (i, j) is kept only when the
 * mask byte of (query block i / 128, key block j / 128) is non-zero, on top of
 * causal and window (the block-sparsity customisation named in the
 * "FlashAttention (Metal Port)" README, section "Documentation"). The kernels
 * walk lists of the blocks that can hold a kept score; this call builds them
 * once per mask, for reuse by every fa_fwd_sparse / fa_bwd_sparse call with
 * the same mask, B, H, Nq, Nk, causal and window.
 *   mask         : device bytes; element (b, h, qb, kb) at
 *                  b*s0 + h*s1 + qb*s2 + kb with mask_strides = {s0, s1, s2}
 *                  (host array, >= 0; 0 broadcasts), qb < ceil(Nq / 128),
 *                  kb < ceil(Nk / 128), h over the H query heads.
 *   kv_count     : device int32 [B, H, nqb] (nqb = ceil(Nq / 128)): how many
 *                  key blocks are listed for each query block;
 *   kv_index     : device int32 [B, H, nqb, nkb] (nkb = ceil(Nk / 128)): the
 *                  listed key blocks, ascending, in the first kv_count entries;
 *   q_count, q_index : the same for the query blocks of each key block
 *                  ([B, H, nkb] and [B, H, nkb, nqb]).
 * A block is listed when its mask byte is non-zero and it meets the causal /
 * window band of fa_fwd_general. One small kernel on `stream`.
 * FA_ERR_INVALID_ARG: a NULL or misaligned pointer, a negative stride,
 * B/H/Nq/Nk < 1, causal not 0/1, window < -1.
 */
int fa_block_lists(const void* mask, const long long* mask_strides, int B,
                   int H, int Nq, int Nk, int causal, int window,
                   int* kv_count, int* kv_index, int* q_count, int* q_index,
                   void* stream);

/*
 * Block-sparse forward: fa_fwd_general restricted to the blocks listed in
 * kv_count / kv_index (from fa_block_lists with the same B, H, Nq, Nk, causal
 * and window). Contiguous layouts as for fa_fwd_general; every dtype. Rows
 * whose blocks are all dropped keep no key: O = 0, lse = -inf. Lists not made
 * by fa_block_lists give undefined results (list reads and tile loads stay
 * inside their buffers).
 */
int fa_fwd_sparse(const void* q, const void* k, const void* v, void* o,
                  float* lse, int B, int H, int Hkv, int Nq, int Nk, int D,
                  int causal, int window, float scale, int dtype,
                  const int* kv_count, const int* kv_index, void* stream);

/*
 * fa_fwd with an explicit conditional-rescale threshold `rescale_log2`
 * (>= 0, in base-2 units of the score): a row's reference max is moved --
 * and its accumulator rescaled -- only when a new tile's max exceeds it by
 * more than this. 0 rescales on every increase. Ignored for FA_FP8_E4M3,
 * which fixes it at 2: probabilities up to 4 are encoded as e4m3(p * 112),
 * which stays within e4m3's largest value 448.
 * The result is the same attention for every threshold (the conditional
 * rescaling of page "r/mlscaling", FA4 bullet, and of the FlashAttention-4
 * entry on the page "FlashAttention" entity trail, section "Corpus findings").
 */
int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int N, int D, int causal, float scale, int dtype,
              float rescale_log2, void* stream);

/*
 * FP8 forward with per-tensor scales (page "r/mlscaling", FA3 bullet names an
 * FP8 forward path; the scaling recipe is per-tensor amax, see
 * fa_quantize_fp8).
 *   q, k, v  : [B, H, N, D] e4m3 codes; the value of an element is
 *              decode(code) * descale of its tensor.
 *   q_descale, k_descale, v_descale : device pointers to one float each, or
 *              NULL for 1.0 (read by the kernel, so they may be produced by
 *              fa_quantize_fp8 on the same stream without a host sync).
 *   o        : [B, H, N, D] bfloat16; lse: [B, H, N] float.
 *   D        : 64, 128 or 256.
 * Both products use fp8 MFMA, with the descales folded into the score scale
 * and the output. The probabilities are encoded as e4m3(p * 112) (p <= 4:
 * the rescale threshold is 2) for the P.V product, and the row sums that
 * normalise O and enter lse add the same encoded values, on the matrix core.
 * On key tiles that need masking (the causal diagonal, a ragged tail) --
 * which hold every key of the shortest rows -- a second e4m3 term carries the
 * rounding residual of the first, so those products see about 2^-8 relative
 * error in P instead of up to 2^-4.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int D, int causal, float scale,
               const float* q_descale, const float* k_descale,
               const float* v_descale, void* stream);

/*
 * FP8 forward with per-tensor scales on the general layouts: fa_fwd_general's
 * grouped K/V heads, query and key lengths and window (fa_fwd_fp8_general),
 * and fa_fwd_varlen's packed sequences (fa_fwd_fp8_varlen), with e4m3 codes
 * and the descale pointers of fa_fwd_fp8 (grouped-query attention and
 * prefill with a cached prefix are how the FP8 forward of the "r/mlscaling"
 * page's FA3 bullet is used in serving). O is bfloat16. Arguments, layouts
 * and errors as for those calls and fa_fwd_fp8; fa_fwd_fp8 is
 * fa_fwd_fp8_general with Hkv = H, Nq = Nk = N and window = -1.
 */
int fa_fwd_fp8_general(const void* q, const void* k, const void* v, void* o,
                       float* lse, int B, int H, int Hkv, int Nq, int Nk, int D,
                       int causal, int window, float scale,
                       const float* q_descale, const float* k_descale,
                       const float* v_descale, void* stream);
int fa_fwd_fp8_varlen(const void* q, const void* k, const void* v, void* o,
                      float* lse, const int* cu_seqlens_q,
                      const int* cu_seqlens_k, int B, int H, int Hkv,
                      int total_q, int total_k, int max_seqlen_q,
                      int max_seqlen_k, int D, int causal, int window,
                      float scale, const float* q_descale,
                      const float* k_descale, const float* v_descale,
                      void* stream);

/*
 * Per-tensor FP8 quantisation (the operand preparation of the FP8 forward):
 *   amax    = max |x_i| over all n elements,
 *   codes_i = e4m3 round-to-nearest-even of x_i * (448 / amax) (float32
 *             product, saturating at +-448),
 *   *descale = amax / 448 (1 when amax is 0).
 *   x       : n floats (device); codes: n bytes (device); descale: one float
 *             (device) which is also used as the amax accumulator.
 * Three kernels on `stream`; n >= 1 and n < 2^40.
 */
int fa_quantize_fp8(const float* x, size_t n, void* codes, float* descale,
                    void* stream);

/*
 * Workspace bytes fa_bwd needs: two floats per row, lse_i * log2(e) and
 * -D_i with D_i = sum_d dO_id O_id (each [B, H, N]), plus a float dQ
 * accumulator [B, H, N, D] for FA_BWD_ATOMIC. 0 on invalid input.
 */
size_t fa_bwd_workspace_size(int B, int H, int N, int D, int dtype, int variant);

/*
 * Backward pass: gradients of sum(dO * O) with respect to Q, K, V, with the
 * probabilities recomputed from lse (P = exp(s - lse)) rather than stored.
 *   q, k, v, o, dO : [B, H, N, D] bfloat16 (dtype must be FA_BF16); o and lse
 *                    are what fa_fwd returned for the same q, k, v.
 *   lse            : [B, H, N] float.
 *   dq, dk, dv     : [B, H, N, D] bfloat16 outputs.
 *   D              : 64, 128 or 256.
 *   variant        : FA_BWD_ATOMIC -- one pass over key tiles computing dK, dV
 *                    and accumulating dQ with float atomics in the workspace
 *                    (the FlashAttention-2 scheme with scratch for atomics);
 *                    FA_BWD_DETERMINISTIC -- dK/dV over key tiles plus a
 *                    separate pass over query tiles for dQ that recomputes
 *                    the scores (7 matrix products instead of 5, no atomics,
 *                    bitwise reproducible), as in the "FlashAttention (Metal
 *                    Port)" README, section "Documentation".
 *   workspace      : device buffer of at least fa_bwd_workspace_size bytes,
 *                    16-byte aligned; the library initialises what it needs.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const void* dO, const float* lse, void* dq, void* dk, void* dv,
           int B, int H, int N, int D, int causal, float scale, int dtype,
           int variant, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Grouped-query backward (the gradients of fa_fwd_gqa): K/V head j's dK and
 * dV are the sums of the contributions of its H / Hkv query heads.
 *   q, o, dO, dq : [B, H, N, D];  k, v, dk, dv : [B, Hkv, N, D];
 *   lse          : [B, H, N];  workspace: fa_bwd_workspace_size(B, H, N, D,
 *                  dtype, variant) bytes (H = query heads).
 * FA_ERR_INVALID_ARG if Hkv < 1 or Hkv does not divide H; FA_ERR_UNSUPPORTED
 * if the H / Hkv query heads of a group span 2^32 bytes or more. Other
 * arguments, variants and errors as for fa_bwd.
 */
int fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o,
               const void* dO, const float* lse, void* dq, void* dk, void* dv,
               int B, int H, int Hkv, int N, int D, int causal, float scale,
               int dtype, int variant, void* workspace, size_t workspace_bytes,
               void* stream);

/*
 * General backward: the gradients of fa_fwd_general.
 *   q, o, dO, dq : [B, H, Nq, D];  k, v, dk, dv : [B, Hkv, Nk, D];
 *   lse          : [B, H, Nq];  workspace: fa_bwd_workspace_size(B, H, Nq, D,
 *                  dtype, variant) bytes.
 * Keys that no query keeps (possible under a window) get dK = dV = 0. Other
 * arguments, variants and errors as for fa_bwd_gqa and fa_fwd_general.
 */
int fa_bwd_general(const void* q, const void* k, const void* v, const void* o,
                   const void* dO, const float* lse, void* dq, void* dk,
                   void* dv, int B, int H, int Hkv, int Nq, int Nk, int D,
                   int causal, int window, float scale, int dtype, int variant,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Strided backward: the gradients of fa_fwd_strided.
 *   strides : host array of 26 element strides -- (batch, head, row) of q, k,
 *             v, o, dO, dq, dk, dv in that order, then lse (batch, head).
 *   workspace : fa_bwd_workspace_size(B, H, Nq, D, dtype, variant) bytes.
 * Errors as for fa_fwd_strided and fa_bwd_general; the span limit applies to
 * the rows of the H / Hkv query heads that share a K/V head, which one pass
 * reads together.
 */
int fa_bwd_strided(const void* q, const void* k, const void* v, const void* o,
                   const void* dO, const float* lse, void* dq, void* dk,
                   void* dv, int B, int H, int Hkv, int Nq, int Nk, int D,
                   int causal, int window, float scale, int dtype, int variant,
                   void* workspace, size_t workspace_bytes,
                   const long long* strides, void* stream);

/*
 * Block-sparse backward: the gradients of fa_fwd_sparse. The dQ pass walks
 * kv_count / kv_index, the key-tile pass q_count / q_index (all four from one
 * fa_block_lists call). Other arguments, variants and errors as for
 * fa_bwd_general.
 */
int fa_bwd_sparse(const void* q, const void* k, const void* v, const void* o,
                  const void* dO, const float* lse, void* dq, void* dk,
                  void* dv, int B, int H, int Hkv, int Nq, int Nk, int D,
                  int causal, int window, float scale, int dtype, int variant,
                  const int* kv_count, const int* kv_index, const int* q_count,
                  const int* q_index, void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * Variable-length backward: the gradients of fa_fwd_varlen.
 *   q, o, dO, dq : [total_q, H, D];  k, v, dk, dv : [total_k, Hkv, D];
 *   lse          : [H, total_q];  workspace: fa_bwd_workspace_size(1, H,
 *                  total_q, D, dtype, variant) bytes.
 * Key rows outside every sequence are not written. Other arguments and errors
 * as for fa_fwd_varlen and fa_bwd_general.
 */
int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                  const void* dO, const float* lse, void* dq, void* dk,
                  void* dv, const int* cu_seqlens_q, const int* cu_seqlens_k,
                  int B, int H, int Hkv, int total_q, int total_k,
                  int max_seqlen_q, int max_seqlen_k, int D, int causal,
                  int window, float scale, int dtype, int variant,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * dK and dV only: the preprocess and the key-tile pass of fa_bwd, without any
 * dQ work, for callers that need no gradient with respect to Q. Arguments as
 * for fa_bwd (dq is not taken); the workspace is the FA_BWD_DETERMINISTIC
 * size. The results are bitwise those of fa_bwd with FA_BWD_DETERMINISTIC.
 */
int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* o,
                const void* dO, const float* lse, void* dk, void* dv,
                int B, int H, int N, int D, int causal, float scale, int dtype,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): fa_bwd with
 * its workspace taken from a static device array of FA_NOALLOC_SCRATCH_BYTES
 * that the library holds on every GPU it runs on, from load until the process
 * ends. Nothing is allocated or freed. Arguments, variants, results and
 * errors as for fa_bwd; a problem whose fa_bwd_workspace_size exceeds
 * FA_NOALLOC_SCRATCH_BYTES is refused with FA_ERR_WORKSPACE before any HIP
 * call. Every call on a GPU uses that GPU's one array, which keeps the last
 * call's contents (the kernels initialise what they read): calls that overlap
 * on one GPU (other streams, other threads) race and must be serialised by the
 * caller. The first call on a device looks the array up (hipGetSymbolAddress);
 * a failure there returns FA_ERR_HIP.
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const void* dO, const float* lse, void* dq, void* dk,
                   void* dv, int B, int H, int N, int D, int causal,
                   float scale, int dtype, int variant, void* stream);

/* Static text for a status code. */
const char* fa_status_string(int status);

/* Message for the last non-OK return on the calling thread ("" if none). */
const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBFA_FA_H */
