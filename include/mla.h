/*
 * mla.h — C ABI of the INT2 rotated-latent MLA decode library (libmla.so,
 * AMD Instinct MI355X / gfx950).
 *
 * What the library computes comes from three pages:
 *  [OSCAR-MLA]  OSCAR issue #10 "MLA model support (GLM-5.1 / DeepSeek-style)",
 *               maintainer reply, part "How the rotation adapts to the latent":
 *               one rotation per MLA layer fitted on the shared latent c_kv
 *               (eigh of c_kv^T c_kv over calibration tokens, eigenvectors by
 *               ascending eigenvalue), clip thresholds fitted on the rotated
 *               latent, the cache holds the rotated INT2 latent, and the
 *               kv_b_proj up-projection runs on the dequantised latent.
 *  [SHARD-MLA]  shard PR #5 "GLM-5.2 speculative drafting ... + opt-in
 *               MLA-latent KV cache", TL;DR item 2: DeepSeek "absorb" — cache
 *               the latent plus one shared rope key, attend in latent space.
 *  [LLMH-SIZE]  llm-helper PR #64 "hf: size GLM-5.3-Flash's KV cache from its
 *               latent layers only", PR description: a latent layer stores
 *               kv_lora_rank + qk_rope_head_dim (+ index_head_dim) per token.
 *
 * Conventions for every call
 *  - Pointers marked "device" are device memory of the current HIP device;
 *    "host" pointers are ordinary host memory.  The caller owns every buffer.
 *    append and decode allocate no device memory.
 *  - bf16 and fp16 values travel as uint16_t bit patterns.
 *  - Arguments are checked on the host before anything is launched; on
 *    failure the call returns a non-zero status, writes nothing and
 *    mla_last_error() describes the problem.
 *  - Calls marked "asynchronous" enqueue work on `stream` (a hipStream_t;
 *    NULL = the legacy default stream) and return; a device-side fault shows
 *    up as MLA_ERR_HIP on a later call or at the caller's synchronisation.
 *  - No C++ exception crosses this interface.  Calls are not re-entrant on
 *    one stream from several host threads.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 3

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,  /* bad pointer, size, shape or dims */
  MLA_ERR_UNSUPPORTED = 2,  /* valid, but no kernel for this shape */
  MLA_ERR_WORKSPACE = 3,    /* workspace too small */
  MLA_ERR_NUMERIC = 4,      /* non-finite input or solver failure */
  MLA_ERR_HIP = 5           /* a HIP runtime call failed */
} mla_status;

typedef enum mla_dtype { MLA_DTYPE_BF16 = 0, MLA_DTYPE_FP32 = 1 } mla_dtype;

/* Shapes of one MLA layer.  Requirements checked by every call:
 * kv_lora_rank (r) > 0, r % group_size == 0, r % 16 == 0, group_size in
 * {16, 32}; 0 < qk_rope_head_dim (d_r) <= 256 and even; qk_nope_head_dim
 * (d_n), v_head_dim (d_v) in 1..1024; num_heads (H) >= 1;
 * index_head_dim (d_idx) >= 0 (0 = no indexer key); rope_bits 0 or 4, and
 * with 4, d_r a multiple of 16.
 *
 * rope_bits selects how the cache stores the shared rope key:
 *  0  bf16, d_r values (2 d_r bytes);
 *  4  the rope-key variant [OSCAR issue #10, the maintainer's later reply,
 *     which names two designs for the rope and non-rope parts without
 *     describing them].  The reading implemented: the rope key stays out of
 *     the rotation and is quantised on its own, in groups of 16 dims, with
 *     4-bit codes by the latent quantiser without clipping (15 levels):
 *     mid = 0.5(mx+mn), half = 0.5(mx-mn), lo = mid - half, hi = mid + half,
 *     scale = fp16((hi-lo)/15), zero = fp16(lo), code = min(15, max(0,
 *     rint((x - zero)/scale))) (0 when scale == 0), in fp32 without fused
 *     multiply-add.  Entry: d_r/2 code bytes (dim 2k in bits 0..3 of byte k,
 *     dim 2k+1 in bits 4..7), then per group its fp16 scale and fp16 zero:
 *     d_r/2 + d_r/4 bytes (48 at d_r = 64, against 128 in bf16). */
typedef struct mla_dims {
  int32_t kv_lora_rank;
  int32_t qk_rope_head_dim;
  int32_t qk_nope_head_dim;
  int32_t v_head_dim;
  int32_t num_heads;
  int32_t group_size;
  int32_t index_head_dim;
  int32_t rope_bits;
} mla_dims;

/* The INT2 latent cache: structure-of-arrays over token slots
 * [LLMH-SIZE: per token, the latent plus the rotary key (plus the indexer
 * key)].  Slot s holds
 *   codes[s*r/4 .. +r/4)        2-bit codes; channel 4k+i at bits 2i..2i+1 of
 *                               byte k (channels of the rotated latent)
 *   scale_zero[s*(r/G)*2 ..]    per group g: [2g] = scale, [2g+1] = zero, fp16
 *   k_rope                      shared rope key: rope_bits 0: bf16 at
 *                               k_rope[s*d_r ..]; rope_bits 4: the quantised
 *                               entry (see mla_dims) at byte s*(d_r/2 + d_r/4)
 *   idx_key[s*d_idx ..]         indexer key, bf16 (NULL when d_idx == 0)
 * i.e. r/4 + 4r/G + rope (2d_r, or d_r/2 + d_r/4) (+ 2d_idx) bytes per
 * token, no padding.
 * Dequantised value: z_hat = zero + scale * code.  All pointers device. */
typedef struct mla_cache {
  uint8_t *codes;
  uint16_t *scale_zero;
  uint16_t *k_rope;
  uint16_t *idx_key;
  int64_t capacity; /* number of slots */
} mla_cache;

/* ------------------------------------------------------------------------
 * mla_calibrate_rotation — per-layer latent rotation  [OSCAR-MLA]
 *
 * Sigma = c^T c / n_cal over the calibration latents (fp64, no centring),
 * symmetric eigendecomposition in fp64, eigenvectors ordered by ascending
 * eigenvalue, each eigenvector's largest-magnitude entry made positive (ties:
 * lowest row).  The covariance is formed on the GPU; the r x r fp64
 * eigensolver (Householder tridiagonalisation + implicit symmetric QR) runs
 * on the host inside the library.
 *   c_cal    device [n_cal][r], dtype bf16 or fp32, row-major
 *   R_out    device [r][r] fp32 row-major: R_out[i*r + j] = component i of
 *            the eigenvector of the j-th smallest eigenvalue
 *   eig_out  host [r] fp64 eigenvalues of Sigma, ascending (may be NULL)
 * Synchronous: returns after R_out is written.
 * Errors: INVALID_ARG (n_cal < 1, NULL pointers, dims), NUMERIC (non-finite
 * covariance or no convergence), HIP.
 * ---------------------------------------------------------------------- */
mla_status mla_calibrate_rotation(const mla_dims *dims, const void *c_cal,
                                  mla_dtype dtype, int64_t n_cal, float *R_out,
                                  double *eig_out, void *stream);

/* ------------------------------------------------------------------------
 * mla_calibrate_rotation_weighted — up-projection-aware rotation
 *
 * [OSCAR issue #10, maintainer reply, closing paragraph]: the open
 * refinement is a latent rotation aware of the kv_b_proj up-projection, so
 * that the INT2 error lands in the latent directions that matter least
 * after reconstruction.  The page gives no formula; this entry point
 * implements one reading: with G = sum_h (W_UK[h]^T W_UK[h] +
 * W_UV[h]^T W_UV[h]) (the metric in which the up-projection counts latent
 * errors, scaled to trace r) and Sigma the uncentred latent covariance as
 * in mla_calibrate_rotation, R holds the eigenvectors of
 * (G + 1e-8 I)^(-1/2) Sigma (G + 1e-8 I)^(-1/2) by ascending eigenvalue,
 * signed as there: directions the up-projection amplifies share the first,
 * finest INT2 groups.  R is orthogonal, so mla_prepare_rotation,
 * mla_fit_clip, mla_fold_absorb_weights, the cache format and decode are
 * used unchanged; for G proportional to the identity R equals
 * mla_calibrate_rotation's.
 *   c_cal    device [n_cal][r], bf16 or fp32 (dtype)
 *   w_uk     device [H][d_n][r] bf16 (un-folded W_UK)
 *   w_uv     device [H][d_v][r] bf16 (un-folded W_UV)
 *   R_out    device [r][r] fp32, layout as in mla_calibrate_rotation
 *   eig_out  host [r] fp64 eigenvalues of the weighted covariance, ascending
 *            (may be NULL)
 * Synchronous: returns after R_out is written.  Allocates device scratch.
 * Errors: INVALID_ARG (n_cal < 1, NULL pointers, dims), NUMERIC (zero or
 * non-finite weights, non-finite covariance, no convergence), HIP.
 * ---------------------------------------------------------------------- */
mla_status mla_calibrate_rotation_weighted(const mla_dims *dims, const void *c_cal,
                                           mla_dtype dtype, int64_t n_cal,
                                           const uint16_t *w_uk, const uint16_t *w_uv,
                                           float *R_out, double *eig_out, void *stream);

/* ------------------------------------------------------------------------
 * mla_prepare_rotation — the rotation as applied: R_apply = bf16(R)
 *
 * Writes R_apply_t[j*r + i] = bf16_round_nearest_even(R[i*r + j]) (the
 * transpose, so row j holds eigenvector j).  Every consumer (append, clip
 * fit, weight folding) uses this one matrix.
 *   R          device [r][r] fp32 (as written by mla_calibrate_rotation)
 *   R_apply_t  device [r][r] bf16
 * Asynchronous.
 * ---------------------------------------------------------------------- */
mla_status mla_prepare_rotation(const mla_dims *dims, const float *R,
                                uint16_t *R_apply_t, void *stream);

/* ------------------------------------------------------------------------
 * mla_fit_clip — per-group clip ratios on the rotated latent  [OSCAR-MLA]
 *
 * For each group g and each ratio a in alpha_grid: rotate every calibration
 * latent with R_apply (z = c R_apply, rounded to fp32), quantise group g with
 * thresholds mid -+ a*half of each token's group range (the append
 * quantiser), and sum (z - z_hat)^2 over tokens and channels in fp64.
 * alpha_out[g] = the ratio with the smallest sum; exact ties -> larger ratio.
 *   c_cal       device [n_cal][r] bf16 or fp32
 *   R_apply_t   device [r][r] bf16 (mla_prepare_rotation)
 *   alpha_grid  host [n_grid] fp32, each in (0, 1]; 1 <= n_grid <= 64
 *   alpha_out   device [r/G] fp32
 *   sse_out     host [r/G][n_grid] fp64 (may be NULL)
 * Synchronous.
 * ---------------------------------------------------------------------- */
mla_status mla_fit_clip(const mla_dims *dims, const void *c_cal,
                        mla_dtype dtype, int64_t n_cal,
                        const uint16_t *R_apply_t, const float *alpha_grid,
                        int32_t n_grid, float *alpha_out, double *sse_out,
                        void *stream);

/* ------------------------------------------------------------------------
 * mla_fold_absorb_weights — fold the un-rotation into kv_b_proj
 *
 * The cache holds z = c R_apply; attention needs c_hat = R_apply z_hat
 * [OSCAR-MLA: up-projection on the dequantised latent].  Folding
 * W~[h] = W[h] R_apply once per layer lets decode work on z_hat directly:
 *   w_uk_f[h][j][a] = sum_i w_uk[h][a][i] R_apply[i][j]   (fp32 sum -> fp16)
 *   w_uv_f[h][v][j] = sum_i w_uv[h][v][i] R_apply[i][j]
 * (the K-side fold is stored transposed per head, latent channel-major, so
 * the absorb kernel reads contiguous runs of the nope dimension)
 *   w_uk   device [H][d_n][r] bf16 (the K half of kv_b_proj per head)
 *   w_uv   device [H][d_v][r] bf16 (the V half)
 *   w_uk_f device [H][r][d_n] fp16;  w_uv_f device [H][d_v][r] fp16
 * Asynchronous.
 * ---------------------------------------------------------------------- */
mla_status mla_fold_absorb_weights(const mla_dims *dims, const uint16_t *w_uk,
                                   const uint16_t *w_uv,
                                   const uint16_t *R_apply_t, uint16_t *w_uk_f,
                                   uint16_t *w_uv_f, void *stream);

/* ------------------------------------------------------------------------
 * mla_append_quant — quantise-on-append  [OSCAR-MLA; SHARD-MLA]
 *
 * For each token i < n with 0 <= slot_mapping[i] < capacity (other slots are
 * skipped): z = latent[i] R_apply (fp32 accumulation), then per group of G
 * channels, in fp32 without fused multiply-add:
 *   mid = 0.5(mx+mn); half = 0.5(mx-mn); lo = mid - a*half; hi = mid + a*half
 *   scale = fp16((hi-lo)/3); zero = fp16(lo)
 *   code = min(3, max(0, rint((z - zero)/scale)))   (0 when scale == 0)
 * and write codes, (scale, zero), k_rope[i] (bf16, or with rope_bits = 4
 * its quantised entry) and idx_key[i] to the slot.
 *   latent        device [n][r] bf16 or fp32
 *   k_rope        device [n][d_r] bf16
 *   idx_key       device [n][d_idx] bf16 (NULL iff d_idx == 0)
 *   slot_mapping  device [n] int64
 *   R_apply_t     device [r][r] bf16;  alpha  device [r/G] fp32
 *   cache         host struct of device pointers
 * Slots that repeat within one call race.  Asynchronous.
 * ---------------------------------------------------------------------- */
mla_status mla_append_quant(const mla_dims *dims, const void *latent,
                            mla_dtype dtype, const uint16_t *k_rope,
                            const uint16_t *idx_key,
                            const int64_t *slot_mapping, int64_t n,
                            const uint16_t *R_apply_t, const float *alpha,
                            const mla_cache *cache, void *stream);

/* Bytes of workspace mla_decode_absorbed needs for `batch` sequences of `tq`
 * queries on the current device (0 for invalid arguments). */
size_t mla_decode_workspace_size(const mla_dims *dims, int32_t batch,
                                 int32_t tq);

/* ------------------------------------------------------------------------
 * mla_decode_absorbed — absorbed MLA decode over the INT2 cache
 * [SHARD-MLA absorb form; OSCAR-MLA up-projection on z_hat]
 *
 * For sequence b, query t, head h, with L = seq_len[b] cache slots
 * seq_base[b] .. seq_base[b]+L-1 (the tq queries are the last tq positions):
 *   q~[j] = sum_a w_uk_f[h][j][a] q_nope[b,t,h][a]
 *   s_tau = softmax_scale (q~ . z_hat_tau + q_rope[b,t,h] . k_rope_tau)
 *   p = softmax over visible tau (causal != 0: tau <= L - tq + t; else all L)
 *   out[b,t,h] = w_uv_f[h] sum_tau p_tau z_hat_tau
 *   lse[b,t,h] = log sum_tau exp(s_tau)   (natural log)
 * Work is split over token chunks (split-K) and merged by log-sum-exp.  A
 * row with no visible token gets out = 0 and lse = -inf.
 *   q_nope [B][tq][H][d_n] bf16; q_rope [B][tq][H][d_r] bf16   (device)
 *   w_uk_f [H][r][d_n] fp16; w_uv_f [H][d_v][r] fp16   (device, folded)
 *   seq_base [B] int64; seq_len [B] int32   (device)
 *   workspace  device, >= mla_decode_workspace_size(dims, batch, tq) bytes
 *   out [B][tq][H][d_v] fp32 (device); lse [B][tq][H] fp32 (device or NULL)
 * Requirements: 1 <= tq <= 64; batch >= 0 (0 = nothing to do);
 * kv_lora_rank <= 512 (UNSUPPORTED otherwise); the caller keeps
 * seq_base[b] + seq_len[b] <= capacity (not checkable on the host).
 * Operand range: the MFMA path (kv_lora_rank 512, qk_rope_head_dim 64,
 * group_size 16 or 32, qk_nope_head_dim a multiple of 16) multiplies fp16
 * operands with fp32 accumulation, so |q_nope|, |q~ * softmax_scale * log2(e)|,
 * |q_rope * softmax_scale * log2(e)|, |k_rope| and |z_hat| must stay below
 * 65504 (the fp16 maximum); beyond it an operand overflows to infinity and
 * the rows it touches come out undefined.  No range check is made.  Each
 * operand carries one fp16 rounding (relative 2^-11; z_hat = zero + scale *
 * code is rounded once, so where |zero| >> scale that rounding can exceed
 * the code step).  The vector-ALU path works in fp32.
 * Asynchronous; no host synchronisation.
 * ---------------------------------------------------------------------- */
mla_status mla_decode_absorbed(const mla_dims *dims, const uint16_t *q_nope,
                               const uint16_t *q_rope, const uint16_t *w_uk_f,
                               const uint16_t *w_uv_f, const mla_cache *cache,
                               const int64_t *seq_base, const int32_t *seq_len,
                               int32_t batch, int32_t tq, int32_t causal,
                               float softmax_scale, void *workspace,
                               size_t workspace_bytes, float *out, float *lse,
                               void *stream);

/* ------------------------------------------------------------------------
 * mla_decode_absorbed_noalloc — mla_decode_absorbed without a caller
 * workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same operands, outputs, kernels and results as mla_decode_absorbed; the
 * workspace is instead a static device array of the library (48 MiB, one
 * copy per GPU, held until the process ends; its address is looked up once
 * per device on that device's first call).  The call allocates nothing.
 * Nothing in the array needs to start at zero: every launch writes what the
 * later launches of the same call read (work list, query operands,
 * partials).  All calls on one GPU share the array, so calls that overlap
 * on one GPU (several streams, several host threads) race: serialise them.
 * Errors: as mla_decode_absorbed; WORKSPACE when this decode needs more
 * than mla_decode_noalloc_max_workspace() bytes (mla_decode_workspace_size
 * gives the need), with nothing launched.
 * ---------------------------------------------------------------------- */
size_t mla_decode_noalloc_max_workspace(void);
mla_status mla_decode_absorbed_noalloc(const mla_dims *dims,
                                       const uint16_t *q_nope,
                                       const uint16_t *q_rope,
                                       const uint16_t *w_uk_f,
                                       const uint16_t *w_uv_f,
                                       const mla_cache *cache,
                                       const int64_t *seq_base,
                                       const int32_t *seq_len, int32_t batch,
                                       int32_t tq, int32_t causal,
                                       float softmax_scale, float *out,
                                       float *lse, void *stream);

/* ------------------------------------------------------------------------
 * mla_decode_step — one decode step: quantise-on-append of the step's new
 * tokens, then absorbed decode over the cache that now holds them
 * [OSCAR-MLA; SHARD-MLA absorb form]
 *
 * The result (cache bytes, out, lse) is exactly that of mla_append_quant(dims,
 * latent, dtype, k_rope, idx_key, slot_mapping, n, R_apply_t, alpha, cache)
 * followed by mla_decode_absorbed(dims, q_nope, ..., lse) on the same stream;
 * the arguments mean what they mean there.  When the decode takes its MFMA
 * path and the append is small (bf16 latents, kv_lora_rank 512, n <= 1024)
 * the append runs in the query-absorb launch, next to the absorb blocks;
 * otherwise the two run one after the other.  n == 0 skips the append;
 * batch == 0 skips the decode.  All arguments are checked before anything
 * is launched.  Asynchronous.
 * ---------------------------------------------------------------------- */
mla_status mla_decode_step(const mla_dims *dims, const void *latent,
                           mla_dtype dtype, const uint16_t *k_rope,
                           const uint16_t *idx_key,
                           const int64_t *slot_mapping, int64_t n,
                           const uint16_t *R_apply_t, const float *alpha,
                           const uint16_t *q_nope, const uint16_t *q_rope,
                           const uint16_t *w_uk_f, const uint16_t *w_uv_f,
                           const mla_cache *cache, const int64_t *seq_base,
                           const int32_t *seq_len, int32_t batch, int32_t tq,
                           int32_t causal, float softmax_scale,
                           void *workspace, size_t workspace_bytes,
                           float *out, float *lse, void *stream);

/* ------------------------------------------------------------------------
 * Sparse decode through the cached indexer key
 * [LLMH-SIZE: GLM-5.3-Flash's latent layers carry a sparse-attention indexer
 * and cache its key]
 *
 * The pages name the indexer and its cached key, not its scoring rule.  The
 * rule implemented here is one reading: one index query vector per sequence,
 *   score_tau = q_idx[b] . idx_key[seq_base[b] + tau]
 * accumulated in fp32 in channel order (bf16 x bf16 products are exact in
 * fp32), and the selection is the top_k tokens by score with equal scores
 * going to the lower token index (fewer than top_k tokens: all of them).
 * ---------------------------------------------------------------------- */

/* Bytes of workspace mla_index_topk needs (0 for invalid arguments): one fp32
 * score per cache slot plus per-sequence histograms and counts. */
size_t mla_index_topk_workspace_size(const mla_dims *dims, int32_t batch,
                                     int64_t capacity);

/* mla_index_topk — select the tokens a query attends to.
 *   q_idx [B][index_head_dim] bf16 (device): the index query vectors
 *   cache: idx_key must be set (index_head_dim 64 or 128, else UNSUPPORTED)
 *   seq_base [B] int64, seq_len [B] int32 (device), as for decode
 *   sel [B][top_k] int32 (device, out): the selected token indices of
 *     sequence b (0-based within the sequence), ascending, in
 *     sel[b*top_k .. b*top_k + n_sel[b] - 1]; the rest is left untouched
 *   n_sel [B] int32 (device, out): min(top_k, seq_len[b])
 * Exact: the selection is decided on the fp32 scores with no approximate
 * step (radix select on the scores, ties resolved by token index).
 * Asynchronous; no host
 * synchronisation.  The caller keeps seq_base[b] + seq_len[b] <= capacity. */
mla_status mla_index_topk(const mla_dims *dims, const uint16_t *q_idx,
                          const mla_cache *cache, const int64_t *seq_base,
                          const int32_t *seq_len, int32_t batch, int32_t top_k,
                          void *workspace, size_t workspace_bytes,
                          int32_t *sel, int32_t *n_sel, void *stream);

/* mla_decode_sparse — mla_decode_absorbed for one query token per sequence
 * (tq = 1) over the selected tokens only: token t < n_sel[b] of sequence b is
 * cache slot seq_base[b] + sel[b*top_k + t] (sel, n_sel as written by
 * mla_index_topk, or any indices the caller keeps inside the sequence).
 * Same operands, workspace (mla_decode_workspace_size(dims, batch, 1)),
 * outputs and error behaviour as mla_decode_absorbed; a sequence with
 * n_sel[b] = 0 gets out = 0 and lse = -inf. */
mla_status mla_decode_sparse(const mla_dims *dims, const uint16_t *q_nope,
                             const uint16_t *q_rope, const uint16_t *w_uk_f,
                             const uint16_t *w_uv_f, const mla_cache *cache,
                             const int64_t *seq_base, const int32_t *sel,
                             const int32_t *n_sel, int32_t batch, int32_t top_k,
                             float softmax_scale, void *workspace,
                             size_t workspace_bytes, float *out, float *lse,
                             void *stream);

/* ------------------------------------------------------------------------
 * OSCAR for full-attention (grouped-query) layers
 *
 * [OSCAR issue #10, "MLA model support (GLM-5.1 / DeepSeek-style)",
 * maintainer reply, part "How the rotation adapts to the latent", first
 * point]: on full-attention models the method fits two rotations per layer,
 * each per KV head: one for K from the query covariance and one for V from a
 * score-weighted value covariance.  Each KV head's K and V rows are rotated
 * and INT2 group-quantised by the latent quantiser (mla_append_quant's
 * arithmetic and entry format, without side keys), and decode runs on the
 * rotated entries: each query is rotated once (q R_k), the merged output
 * un-rotated once (o_z R_v^T).  The page gives no formulas; the readings
 * implemented:
 *  - the calibration data is one sequence of n_cal tokens under causal
 *    self-attention (query i sees keys 0..i) with the given softmax scale;
 *  - K rotation of head h (gqa_dims.k_rotation):
 *      GQA_K_QUERY_COVARIANCE (0, the default, the plain reading of "a
 *      query-covariance rotation for K"): eigenvectors, by ascending
 *      eigenvalue, of Sigma_q, the uncentred covariance of the queries that
 *      read the head (its G query heads, all positions).  A key error e
 *      costs the score error q . e, of mean square e^T Sigma_q e, which in
 *      this basis weights each rotated channel's error by its eigenvalue, so
 *      channels of equal weight share the INT2 groups;
 *      GQA_K_QUERY_METRIC (1, a refinement that also follows where the keys
 *      vary): eigenvectors, by ascending eigenvalue, of
 *      (M + 1e-8 I)^(-1/2) Sigma_k (M + 1e-8 I)^(-1/2), with Sigma_k the
 *      uncentred covariance of the head's keys and M = Sigma_q scaled to
 *      mean eigenvalue 1;
 *  - V rotation of head h: eigenvectors, by ascending eigenvalue, of
 *    sum_t w_t v_t v_t^T / sum_t w_t, with w_t the attention mass key t
 *    receives (summed over the head's query heads and the positions i >= t);
 *  - signs as mla_calibrate_rotation.
 * Layout: query head g reads KV head g / G, G = num_q_heads / num_kv_heads.
 * ---------------------------------------------------------------------- */
#define GQA_K_QUERY_COVARIANCE 0
#define GQA_K_QUERY_METRIC 1
typedef struct gqa_dims {
  int32_t head_dim;     /* d: a multiple of group_size and of 8, 16..256 */
  int32_t num_q_heads;  /* H_q, a multiple of num_kv_heads, <= 4096 */
  int32_t num_kv_heads; /* H_kv >= 1 */
  int32_t group_size;   /* INT2 group along d: 16 or 32 */
  int32_t k_rotation;   /* GQA_K_QUERY_COVARIANCE or GQA_K_QUERY_METRIC (gqa_calibrate only) */
} gqa_dims;

/* K and V entries per KV head in the latent entry format (codes packed four
 * per byte, channel 4i + e in bits 2e..2e+1 of byte i; fp16 scale then zero
 * per group).  Entry (h, slot) is row h * capacity + slot of
 *   k_codes [H_kv * capacity][d/4] u8,  k_scale_zero [H_kv * capacity][d/G][2] fp16,
 *   v_codes, v_scale_zero likewise.  Device memory, caller-owned. */
typedef struct gqa_cache {
  uint8_t *k_codes;
  uint16_t *k_scale_zero;
  uint8_t *v_codes;
  uint16_t *v_scale_zero;
  int64_t capacity; /* slots per KV head */
} gqa_cache;

/* gqa_calibrate — both rotations of every KV head.
 *   q_cal [H_q][n_cal][d], k_cal and v_cal [H_kv][n_cal][d]: device bf16,
 *     n_cal in 1..65536 (the attention masses cost n_cal^2 d per query head),
 *     head-major (one calibration sequence, position-ordered)
 *   softmax_scale: the layer's score scale (for the attention weights)
 *   R_k, R_v: device [H_kv][d][d] fp32, per head laid out as
 *     mla_calibrate_rotation's R (column j = eigenvector j)
 *   eig_k, eig_v: host [H_kv][d] fp64 eigenvalues, ascending (may be NULL)
 * The covariances, attention masses (fp64, two passes over the causal
 * scores, no atomics) and weighted covariance run on the GPU; the d x d
 * eigensolves on the host.  Synchronous; allocates device scratch.
 * Errors: INVALID_ARG (dims, n_cal < 1, NULL or unaligned pointers,
 * non-finite scale), NUMERIC (non-finite statistics, no convergence), HIP. */
mla_status gqa_calibrate(const gqa_dims *dims, const uint16_t *q_cal,
                         const uint16_t *k_cal, const uint16_t *v_cal,
                         int64_t n_cal, float softmax_scale, float *R_k,
                         float *R_v, double *eig_k, double *eig_v,
                         void *stream);

/* gqa_prepare_rotation — R_apply_t[h] = bf16(R[h])^T for every KV head
 * (mla_prepare_rotation per head).  R device [H_kv][d][d] fp32, R_apply_t
 * device [H_kv][d][d] bf16.  Asynchronous. */
mla_status gqa_prepare_rotation(const gqa_dims *dims, const float *R,
                                uint16_t *R_apply_t, void *stream);

/* gqa_fit_clip — per-head, per-group clip ratios (mla_fit_clip per head).
 *   x_cal [H_kv][n_cal][d] device bf16 (the calibration keys, or values)
 *   R_apply_t [H_kv][d][d] device bf16 (of the same side)
 *   alpha_grid host [n_grid] fp32 in (0, 1], 1 <= n_grid <= 64
 *   alpha_out [H_kv][d/G] device fp32
 * Synchronous; allocates device scratch. */
mla_status gqa_fit_clip(const gqa_dims *dims, const uint16_t *x_cal,
                        int64_t n_cal, const uint16_t *R_apply_t,
                        const float *alpha_grid, int32_t n_grid,
                        float *alpha_out, void *stream);

/* gqa_append_quant — rotate, clip and quantise n new tokens' K and V rows.
 *   k, v [n][H_kv][d] device bf16 (the projection output layout)
 *   slot_mapping [n] int64 device: slot of token i (outside [0, capacity):
 *     skipped)
 *   Rk_apply_t, Rv_apply_t [H_kv][d][d] bf16; alpha_k, alpha_v [H_kv][d/G]
 * Codes and scale/zero are those mla_append_quant writes for the head's
 * rows with the head's rotation and ratios.  Asynchronous. */
mla_status gqa_append_quant(const gqa_dims *dims, const uint16_t *k,
                            const uint16_t *v, const int64_t *slot_mapping,
                            int64_t n, const uint16_t *Rk_apply_t,
                            const uint16_t *Rv_apply_t, const float *alpha_k,
                            const float *alpha_v, const gqa_cache *cache,
                            void *stream);

/* Bytes of workspace gqa_decode needs (0 for invalid arguments). */
size_t gqa_decode_workspace_size(const gqa_dims *dims, int32_t batch,
                                 int32_t tq);

/* gqa_decode — grouped-query decode over the INT2 K/V cache.
 *   q [B][tq][H_q][d] device bf16; the tq queries are the last tq positions
 *     of each sequence (causal: query t sees tokens 0 .. L - tq + t)
 *   seq_base [B] int64, seq_len [B] int32 (device): sequence b is slots
 *     seq_base[b] .. seq_base[b] + seq_len[b] - 1 of every KV head
 *   out [B][tq][H_q][d] fp32 = softmax(scale q . k_hat) v_hat with k_hat =
 *     z_k R_k,apply^T, v_hat = z_v R_v,apply^T the dequantised entries
 *     un-rotated; lse [B][tq][H_q] fp32 natural-log log-sum-exp (may be NULL)
 * An empty sequence gives out = 0, lse = -inf.  Runs as: query rotation,
 * split-K attention over each (sequence, KV head) (MFMA for head_dim 128
 * with at most 32 query rows per KV head, G * tq; vector ALU otherwise),
 * then the log-sum-exp merge and the un-rotation in one launch.  The MFMA
 * kernel takes q R_k * softmax_scale * log2(e) and the dequantised K and V
 * entries as fp16 operands: they must stay below 65504 in magnitude (no
 * range check is made).
 * Asynchronous; no host synchronisation.
 * Errors: INVALID_ARG (dims, batch < 0, tq outside 1..64, causal not 0/1,
 * NULL or unaligned pointers), WORKSPACE, HIP. */
mla_status gqa_decode(const gqa_dims *dims, const uint16_t *q,
                      const gqa_cache *cache, const uint16_t *Rk_apply_t,
                      const uint16_t *Rv_apply_t, const int64_t *seq_base,
                      const int32_t *seq_len, int32_t batch, int32_t tq,
                      int32_t causal, float softmax_scale, void *workspace,
                      size_t workspace_bytes, float *out, float *lse,
                      void *stream);

/* ------------------------------------------------------------------------
 * Diagnostics
 * ---------------------------------------------------------------------- */

/* Message for the last failed call on this host thread ("" if none). */
const char *mla_last_error(void);
const char *mla_status_string(mla_status status);
int32_t mla_abi_version(void);

/* Decode kernel selection, for tests and measurement: 0 = automatic (the
 * MFMA kernels wherever the shape has them, at any H*tq; else the vector-ALU
 * split-K kernel), 1 = always the vector-ALU kernel, 2 = always MFMA
 * (MLA_ERR_UNSUPPORTED where no MFMA kernel fits).  Process-wide. */
mla_status mla_set_decode_variant(int32_t variant);

/* Per-kernel timing with HIP events recorded on the launch stream around
 * every kernel the library enqueues while enabled.  Names: "append_quant",
 * "decode_plan", "absorb_q" (on the MFMA path this kernel also plans the
 * split-K work, and "decode_plan" is not launched), "splitk_decode",
 * "combine", "up_proj", "combine_up_proj" (the two in one launch where
 * the shape allows), "index_score", "index_select", "gqa_rotate_q",
 * "gqa_merge_unrotate", "fold_weights", "prepare_rotation", "covariance",
 * "clip_fit".
 * mla_timing_query waits for the recorded events and returns the summed
 * milliseconds and launch count since the last reset.  Process-wide; not
 * for use while another thread launches. */
mla_status mla_timing_enable(int32_t enable);
mla_status mla_timing_reset(void);
mla_status mla_timing_query(const char *kernel, double *total_ms,
                            int64_t *launches);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
