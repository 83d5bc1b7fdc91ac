// Kernel launchers shared between the translation units of libmla.
// Every launcher enqueues on `stream`, checks nothing it can assume from the
// caller (api.hip validates first) and returns the launch error.
#pragma once

#include "common.hpp"

namespace mla {

// One split-K work item: tokens [t0, t1) of sequence b.
struct WorkItem {
  int32_t b, t0, t1, pad;
};

// ---- calibration (calib.hip) ----
hipError_t launch_covariance(const void *c, mla_dtype dt, int64_t n, int r,
                             double *sigma, hipStream_t s);
hipError_t launch_prepare_rotation(const float *R, int r, uint16_t *Rt,
                                   hipStream_t s);
hipError_t launch_group_sse(const float *z, int64_t n, int r, int G,
                            const float *grid, int n_grid, double *sse,
                            float *alpha_out, hipStream_t s);
// inner > 0: store per-head blocks transposed ([head][r][inner])
hipError_t launch_fold(const uint16_t *w, int rows, int r, const uint16_t *Rt,
                       uint16_t *wf, int inner, hipStream_t s);

// ---- append (append.hip) ----
// z_out != nullptr: write the fp32 rotated latent [n][r] instead of the cache
// (same arithmetic as the cache path; used by the clip fit).
bool append_uses_mfma(const mla_dims &d, mla_dtype dt);
hipError_t launch_append(const mla_dims &d, const void *latent, mla_dtype dt,
                         const uint16_t *k_rope, const uint16_t *idx_key,
                         const int64_t *slots, int64_t n, const uint16_t *Rt,
                         const float *alpha, const mla_cache &cache,
                         float *z_out, hipStream_t s, int64_t lat_stride = 0);
// lat_stride: elements between consecutive tokens' latent rows (0: r)

// ---- decode (decode.hip, decode_mfma.hip) ----
struct DecodeArgs {
  mla_dims d;
  const uint16_t *q_nope, *q_rope, *w_uk_f, *w_uv_f;
  mla_cache cache;
  const int64_t *seq_base;
  const int32_t *seq_len;
  int32_t B, Tq, causal;
  float scale_log2;  // softmax_scale * log2(e)
  float *out, *lse;
  // workspace carve-up
  WorkItem *items;
  int32_t *item_begin;  // [B + 1]
  int32_t *meta;        // [0] = n_items, [1] = chunk tokens
  void *qbuf;           // absorbed queries
  float *oz;            // combined latent output [B*M][r]
  uint16_t *part_o;     // [max_items][M][r] fp16: the item's O / l (a convex
                        // combination of fp16 entries, so in fp16 range)
  float *part_ml;       // [max_items][M][2]  (m in log2 units, l)
  int32_t max_items;
  int32_t target_items;
  int32_t min_chunk_tiles;  // smallest split-K item, in tiles
  int32_t tile;
  // sparse decode: token t of sequence b is cache slot seq_base[b] +
  // sel[b * sel_stride + t] (seq_len then holds the selected counts); dense
  // decode: sel == nullptr and token t is slot seq_base[b] + t
  const int32_t *sel;
  int32_t sel_stride;
  // grouped-query layers (vector-ALU kernel only): values come from their own
  // INT2 cache, same slots; codes == nullptr: values are the latent itself
  mla_cache vcache;
};

hipError_t launch_plan(const DecodeArgs &a, hipStream_t s);

// ---- indexer top-k (index.hip) ----
struct IndexArgs {
  const uint16_t *q_idx;    // [B][d_idx] bf16
  const uint16_t *idx_key;  // cache index keys [capacity][d_idx] bf16
  const int64_t *seq_base;
  const int32_t *seq_len;
  int32_t B, d_idx, top_k, n_chunks;
  float *scores;            // [capacity], by cache slot
  uint32_t *hist;           // [index_passes()][B][index_hist_bins()]
  uint32_t *pfx_bits;       // [index_passes() - 1][B]: key prefix after passes 0..p
  int32_t *pfx_rank;        // [index_passes() - 1][B]: rank still to find inside it
  int32_t *chunk_above;     // [B][n_chunks]: keys above the last pass's prefix
  int32_t *chunk_suf;       // [B][n_chunks][index_last_bins()]: suffix sums of the last digit
  int32_t *sel;             // [B][top_k]
  int32_t *n_sel;           // [B]
};
int index_chunks();
int index_hist_bins();
int index_passes();
int index_last_bins();
hipError_t launch_index_topk(const IndexArgs &a, hipStream_t s);

hipError_t launch_absorb_f32(const DecodeArgs &a, hipStream_t s);
hipError_t launch_splitk_valu(const DecodeArgs &a, hipStream_t s);
hipError_t launch_combine(const DecodeArgs &a, hipStream_t s);
hipError_t launch_upproj(const DecodeArgs &a, hipStream_t s);

// ---- grouped-query (OSCAR full-attention) layers (gqa.hip) ----
// Calibration statistics: causal row statistics, the attention mass w
// [H_kv][n] of every calibration key and the score-weighted value covariance
// sigma_v [H_kv][d][d] (scratch row_m, row_inv [H_q][n]).
hipError_t launch_gqa_calib_stats(const uint16_t *q, const uint16_t *k, const uint16_t *v, int n, int d, int H_q,
                                  int H_kv, double scale, double *row_m, double *row_inv, double *w,
                                  double *sigma_v, hipStream_t s);
struct GqaDecodeArgs {
  const uint16_t *q;               // [B][Tq][H_q][d] bf16
  const uint16_t *rk_t, *rv_t;     // [H_kv][d][d] bf16, R_apply^T per KV head
  const int64_t *seq_base;
  const int32_t *seq_len;
  int64_t capacity;                // slots per KV head
  int32_t B, Tq, H_q, H_kv, d;
  float scale_log2;                // softmax_scale * log2(e)
  float *qbuf;                     // [B * H_kv][Tq * G][d] rotated queries
  int64_t *base2;                  // [B * H_kv] pseudo-sequence slot bases
  int32_t *len2;                   // [B * H_kv] pseudo-sequence lengths
  float *out, *lse;                // [B][Tq][H_q][d], [B][Tq][H_q]
};
// query rotation, plus the split-K plan of sa (one extra block)
hipError_t launch_gqa_rotate_q(const GqaDecodeArgs &a, const DecodeArgs &sa, hipStream_t s);
// the merge of the split-K partials (sa's items and partials) and the
// un-rotation in one launch
hipError_t launch_gqa_merge_unrotate(const GqaDecodeArgs &a, const DecodeArgs &sa, hipStream_t s);

// MFMA split-K path (r = 512, d_r = 64): supported() says whether it applies.
bool mfma_decode_supported(const mla_dims &d, int rows);
bool mfma_absorb_supported(const mla_dims &d);
int mfma_row_block();
// A decode step's new tokens (bf16 latent rows of kv_lora_rank values),
// appended by blocks of the query-absorb launch.
struct AppendJob {
  const void *latent;
  const uint16_t *k_rope, *idx_key;
  const int64_t *slots;
  int64_t n;
  const uint16_t *Rt;
  const float *alpha;
};
// true when launch_absorb_mfma_layout can take the append of n tokens
bool append_fusable(const mla_dims &d, mla_dtype dt, int64_t n);
hipError_t launch_absorb_mfma_layout(const DecodeArgs &a, hipStream_t s, const AppendJob *job = nullptr);
hipError_t launch_splitk_mfma(const DecodeArgs &a, hipStream_t s);
// The split-K kernel of the MFMA path for `rows` query rows per sequence
// (sparse: selected-token decode), and the work items that fill the GPU
// with it (one resident workgroup per item and row block).
enum class SplitK { kRows16, kWarpSpec };
SplitK splitk_kernel_for(int rows, bool sparse);
int splitk_target_items(int rows, bool sparse, int ncu);
// grouped-query layers: head dim 128, at most 32 query rows per KV head,
// one wave per work item (grid = max_items)
bool gqa_mfma_supported(const mla_dims &d, int rows);
// resident waves per compute unit of the grouped-query MFMA kernel for
// `rows` query rows per KV head (its work-item target per compute unit)
int gqa_waves_per_cu(int rows);
hipError_t launch_gqa_splitk_mfma(const DecodeArgs &a, hipStream_t s);

}  // namespace mla
