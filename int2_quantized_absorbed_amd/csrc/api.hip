// C ABI of libmla: argument checks, workspace carving, kernel dispatch,
// error reporting and optional per-kernel event timing.
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "eigh.hpp"
#include "kernels.hpp"

namespace mla {

// ---------------------------------------------------------------------------
// errors
// ---------------------------------------------------------------------------
static thread_local std::string g_last_error;

void set_error(const std::string &msg) { g_last_error = msg; }
void clear_error() { g_last_error.clear(); }
mla_status fail(mla_status st, const std::string &msg) {
  set_error(msg);
  return st;
}
mla_status hip_fail(hipError_t e, const char *what) {
  set_error(std::string(what) + ": " + hipGetErrorString(e));
  return MLA_ERR_HIP;
}

bool dims_valid(const mla_dims *d, std::string *why) {
  if (d == nullptr) {
    *why = "dims is NULL";
    return false;
  }
  const int r = d->kv_lora_rank, G = d->group_size;
  if (r <= 0 || r % 16 != 0) {
    *why = "kv_lora_rank must be a positive multiple of 16";
    return false;
  }
  if (G != 16 && G != 32) {
    *why = "group_size must be 16 or 32";
    return false;
  }
  if (r % G != 0) {
    *why = "kv_lora_rank must be a multiple of group_size";
    return false;
  }
  if (d->qk_rope_head_dim <= 0 || d->qk_rope_head_dim > 256 || (d->qk_rope_head_dim & 1)) {
    *why = "qk_rope_head_dim must be even and in 1..256";
    return false;
  }
  if (d->rope_bits != 0 && d->rope_bits != 4) {
    *why = "rope_bits must be 0 (bf16 rope key) or 4";
    return false;
  }
  if (d->rope_bits == 4 && d->qk_rope_head_dim % 16 != 0) {
    *why = "a 4-bit rope key needs qk_rope_head_dim a multiple of 16";
    return false;
  }
  if (d->qk_nope_head_dim <= 0 || d->qk_nope_head_dim > 1024 || d->v_head_dim <= 0 ||
      d->v_head_dim > 1024) {
    *why = "qk_nope_head_dim and v_head_dim must be in 1..1024";
    return false;
  }
  if (d->num_heads <= 0 || d->num_heads > 4096) {
    *why = "num_heads must be in 1..4096";
    return false;
  }
  if (d->index_head_dim < 0 || d->index_head_dim > 1024 || (d->index_head_dim & 1)) {
    *why = "index_head_dim must be even and in 0..1024";
    return false;
  }
  return true;
}

int device_cu_count() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  cache[dev] = n;
  return n;
}

// ---------------------------------------------------------------------------
// event timing
// ---------------------------------------------------------------------------
namespace {
struct TimingRec {
  std::string name;
  hipEvent_t start, end;
};
struct TimingState {
  bool enabled = false;
  std::vector<TimingRec> pending;
  std::vector<hipEvent_t> pool;
  std::map<std::string, std::pair<double, int64_t>> totals;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
TimingState &timing() {
  static TimingState st;
  return st;
}
}  // namespace

TimedLaunch::TimedLaunch(const char *name, hipStream_t s) : name_(name), stream_(s), start_(nullptr) {
  TimingState &t = timing();
  if (!t.enabled) return;
  hipEvent_t e = t.get();
  if (e != nullptr && hipEventRecord(e, s) == hipSuccess) start_ = e;
}

TimedLaunch::~TimedLaunch() {
  if (start_ == nullptr) return;
  TimingState &t = timing();
  hipEvent_t e = t.get();
  if (e == nullptr || hipEventRecord(e, stream_) != hipSuccess) {
    t.pool.push_back(static_cast<hipEvent_t>(start_));
    return;
  }
  t.pending.push_back({name_, static_cast<hipEvent_t>(start_), e});
}

// ---------------------------------------------------------------------------
// decode workspace layout
// ---------------------------------------------------------------------------
namespace {
int g_decode_variant = 0;

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct WsLayout {
  size_t items = 0, item_begin = 0, meta = 0, qbuf = 0, oz = 0, part_o = 0, part_ml = 0, total = 0;
  int max_items = 0;
};

// Work items that fill the GPU: one resident workgroup (or wave) per item and
// row block of the split-K kernel that runs (sparse: selected-token decode).
int target_items(int rows, bool mfma, bool sparse) {
  const int ncu = device_cu_count();
  if (mfma) return splitk_target_items(rows, sparse, ncu);
  const int t = 2 * ncu / ((rows + 15) / 16);  // two 16-row blocks per compute unit
  return t < 1 ? 1 : t;
}

// Shortest split-K chunk, in tokens: below it the fixed cost of an item
// (query rows in, partial rows out, the combine reading them back) outweighs
// spreading a short context over more compute units.
#ifndef MLA_SPLIT_MIN_TOKENS
#define MLA_SPLIT_MIN_TOKENS 64
#endif
int min_chunk_tiles(int tile) { return (MLA_SPLIT_MIN_TOKENS + tile - 1) / tile; }

WsLayout layout(const mla_dims &d, int B, int Tq, int min_items = 0) {
  WsLayout w;
  const int r = d.kv_lora_rank, K = r + d.qk_rope_head_dim;
  const int M = d.num_heads * Tq;
  // the planner emits at most max(target, number of sequences) items
  int tgt = target_items(M, false, false);
  if (mfma_decode_supported(d, M))
    tgt = std::max(tgt, std::max(target_items(M, true, false), target_items(M, true, true)));
  w.max_items = std::max(std::max(tgt, B), min_items);
  size_t off = 0;
  w.items = off;
  off = align256(off + sizeof(WorkItem) * w.max_items);
  w.item_begin = off;
  off = align256(off + sizeof(int32_t) * (B + 1));
  w.meta = off;
  off = align256(off + sizeof(int32_t) * 4);
  w.qbuf = off;
  const size_t q32 = static_cast<size_t>(B) * M * K * sizeof(float);
  const int rbm = (M + mfma_row_block() - 1) / mfma_row_block();
  const size_t q16 = static_cast<size_t>(B) * rbm * mfma_row_block() * K * sizeof(uint16_t);
  off = align256(off + std::max(q32, q16));
  w.oz = off;
  off = align256(off + static_cast<size_t>(B) * M * r * sizeof(float));
  w.part_o = off;
  off = align256(off + static_cast<size_t>(w.max_items) * M * r * sizeof(uint16_t));
  w.part_ml = off;
  off = align256(off + static_cast<size_t>(w.max_items) * M * 2 * sizeof(float));
  w.total = off;
  return w;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// sw = (M + ridge I)^(-1/2) Sigma (M + ridge I)^(-1/2), symmetrised, with M
// the metric scaled to trace r (mean eigenvalue 1): Sigma seen in the metric
// in which errors count.  The ridge keeps directions the metric ignores
// finite (they get the largest weighted variance and the coarsest groups).
// False if the metric is zero or not finite, or its eigensolve fails.
constexpr double kMetricRidge = 1e-8;

bool metric_whitened(int r, std::vector<double> metric, const std::vector<double> &sigma,
                     std::vector<double> &sw) {
  const size_t rr = static_cast<size_t>(r) * r;
  double tr = 0.0;
  for (int i = 0; i < r; ++i) tr += metric[static_cast<size_t>(i) * r + i];
  if (!(tr > 0.0) || !std::isfinite(tr)) return false;
  for (size_t i = 0; i < rr; ++i) metric[i] *= static_cast<double>(r) / tr;
  std::vector<double> gv(r), gvec(rr), gh(rr, 0.0), tmp(rr, 0.0);
  if (!eigh_ascending(r, metric.data(), gv.data(), gvec.data())) return false;
  // (M + ridge I)^(-1/2) = V diag(1 / sqrt(max(lambda, 0) + ridge)) V^T
  for (int k = 0; k < r; ++k) {
    const double sq = 1.0 / std::sqrt(std::max(gv[k], 0.0) + kMetricRidge);
    for (int i = 0; i < r; ++i) {
      const double vik = gvec[static_cast<size_t>(i) * r + k] * sq;
      if (vik == 0.0) continue;
      double *row = gh.data() + static_cast<size_t>(i) * r;
      for (int j = 0; j < r; ++j) row[j] += vik * gvec[static_cast<size_t>(j) * r + k];
    }
  }
  auto matmul = [r](const std::vector<double> &a, const std::vector<double> &b, std::vector<double> &c) {
    std::fill(c.begin(), c.end(), 0.0);
    for (int i = 0; i < r; ++i)
      for (int k = 0; k < r; ++k) {
        const double aik = a[static_cast<size_t>(i) * r + k];
        if (aik == 0.0) continue;
        const double *brow = b.data() + static_cast<size_t>(k) * r;
        double *crow = c.data() + static_cast<size_t>(i) * r;
        for (int j = 0; j < r; ++j) crow[j] += aik * brow[j];
      }
  };
  sw.assign(rr, 0.0);
  matmul(gh, sigma, tmp);
  matmul(tmp, gh, sw);
  for (int i = 0; i < r; ++i)
    for (int j = i + 1; j < r; ++j) {
      const double m = 0.5 * (sw[static_cast<size_t>(i) * r + j] + sw[static_cast<size_t>(j) * r + i]);
      sw[static_cast<size_t>(i) * r + j] = m;
      sw[static_cast<size_t>(j) * r + i] = m;
    }
  return true;
}

// ---- grouped-query layers ----
bool gqa_dims_valid(const gqa_dims *g, std::string *why) {
  if (g == nullptr) {
    *why = "dims is NULL";
    return false;
  }
  if (g->group_size != 16 && g->group_size != 32) {
    *why = "group_size must be 16 or 32";
    return false;
  }
  if (g->head_dim < 16 || g->head_dim > 256 || g->head_dim % g->group_size != 0 || g->head_dim % 8 != 0) {
    *why = "head_dim must be in 16..256 and a multiple of group_size and of 8";
    return false;
  }
  if (g->num_kv_heads < 1 || g->num_q_heads < g->num_kv_heads || g->num_q_heads > 4096 ||
      g->num_q_heads % g->num_kv_heads != 0) {
    *why = "num_q_heads must be a multiple of num_kv_heads >= 1 and at most 4096";
    return false;
  }
  if (g->k_rotation != GQA_K_QUERY_COVARIANCE && g->k_rotation != GQA_K_QUERY_METRIC) {
    *why = "k_rotation must be GQA_K_QUERY_COVARIANCE or GQA_K_QUERY_METRIC";
    return false;
  }
  return true;
}

// A KV head's K or V rows as a latent of width d with no side keys, and the
// G query heads of one KV head as the decode's heads.
mla_dims gqa_latent_dims(const gqa_dims &g) {
  mla_dims d{};
  d.kv_lora_rank = g.head_dim;
  d.qk_rope_head_dim = 0;
  d.rope_bits = 0;
  d.qk_nope_head_dim = g.head_dim;
  d.v_head_dim = g.head_dim;
  d.num_heads = g.num_q_heads / g.num_kv_heads;
  d.group_size = g.group_size;
  d.index_head_dim = 0;
  return d;
}

struct GqaWs {
  WsLayout split;  // the shared decode workspace of B * H_kv pseudo-sequences
  size_t base2 = 0, len2 = 0, total = 0;
};

// Work items of the grouped-query split-K: one wave per item on the MFMA
// kernels, as many as are resident per CU (gqa_waves_per_cu); otherwise the
// vector-ALU kernel's own target.

bool gqa_use_mfma(const gqa_dims &g, int Tq) {
  const int rows = g.num_q_heads / g.num_kv_heads * Tq;
  return g_decode_variant != 1 && gqa_mfma_supported(gqa_latent_dims(g), rows);
}

int gqa_target_items(const gqa_dims &g, int Tq) {
  const int rows = g.num_q_heads / g.num_kv_heads * Tq;
  return gqa_use_mfma(g, Tq) ? gqa_waves_per_cu(rows) * device_cu_count() : target_items(rows, false, false);
}

GqaWs gqa_layout(const gqa_dims &g, int B, int Tq) {
  GqaWs w;
  const int Bp = B * g.num_kv_heads;
  w.split = layout(gqa_latent_dims(g), Bp, Tq, gqa_target_items(g, Tq));
  size_t off = w.split.total;
  w.base2 = off;
  off = align256(off + sizeof(int64_t) * Bp);
  w.len2 = off;
  off = align256(off + sizeof(int32_t) * Bp);
  w.total = off;
  return w;
}

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" {

const char *mla_last_error(void) { return g_last_error.c_str(); }

const char *mla_status_string(mla_status st) {
  switch (st) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported shape";
    case MLA_ERR_WORKSPACE: return "workspace too small";
    case MLA_ERR_NUMERIC: return "numerical failure";
    case MLA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

mla_status mla_set_decode_variant(int32_t variant) {
  if (variant < 0 || variant > 2) return fail(MLA_ERR_INVALID_ARG, "decode variant must be 0, 1 or 2");
  g_decode_variant = variant;
  clear_error();
  return MLA_OK;
}

mla_status mla_timing_enable(int32_t enable) {
  timing().enabled = enable != 0;
  clear_error();
  return MLA_OK;
}

mla_status mla_timing_reset(void) {
  TimingState &t = timing();
  for (auto &rec : t.pending) {
    (void)hipEventSynchronize(rec.end);
    t.pool.push_back(rec.start);
    t.pool.push_back(rec.end);
  }
  t.pending.clear();
  t.totals.clear();
  clear_error();
  return MLA_OK;
}

mla_status mla_timing_query(const char *kernel, double *total_ms, int64_t *launches) {
  if (kernel == nullptr || total_ms == nullptr || launches == nullptr)
    return fail(MLA_ERR_INVALID_ARG, "mla_timing_query: NULL argument");
  TimingState &t = timing();
  for (auto &rec : t.pending) {
    hipError_t e = hipEventSynchronize(rec.end);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, rec.start, rec.end);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    auto &tot = t.totals[rec.name];
    tot.first += ms;
    tot.second += 1;
    t.pool.push_back(rec.start);
    t.pool.push_back(rec.end);
  }
  t.pending.clear();
  auto it = t.totals.find(kernel);
  *total_ms = (it == t.totals.end()) ? 0.0 : it->second.first;
  *launches = (it == t.totals.end()) ? 0 : it->second.second;
  clear_error();
  return MLA_OK;
}

// ---------------------------------------------------------------------------
mla_status mla_calibrate_rotation(const mla_dims *dims, const void *c_cal, mla_dtype dtype,
                                  int64_t n_cal, float *R_out, double *eig_out, void *stream) {
  std::string why;
  if (!dims_valid(dims, &why)) return fail(MLA_ERR_INVALID_ARG, "mla_calibrate_rotation: " + why);
  if (c_cal == nullptr || R_out == nullptr)
    return fail(MLA_ERR_INVALID_ARG, "mla_calibrate_rotation: NULL device pointer");
  if (dtype != MLA_DTYPE_BF16 && dtype != MLA_DTYPE_FP32)
    return fail(MLA_ERR_INVALID_ARG, "mla_calibrate_rotation: dtype must be bf16 or fp32");
  if (n_cal < 1) return fail(MLA_ERR_INVALID_ARG, "mla_calibrate_rotation: n_cal must be >= 1");
  const int r = dims->kv_lora_rank;
  if (r > 4096) return fail(MLA_ERR_UNSUPPORTED, "mla_calibrate_rotation: kv_lora_rank > 4096");
  hipStream_t s = static_cast<hipStream_t>(stream);
  double *sigma_d = nullptr;
  const size_t rr = static_cast<size_t>(r) * r;
  MLA_HIP_CHECK(hipMalloc(&sigma_d, rr * sizeof(double)), "hipMalloc(covariance)");
  std::vector<double> sigma(rr), vals(r), vecs(rr);
  hipError_t e = launch_covariance(c_cal, dtype, n_cal, r, sigma_d, s);
  if (e == hipSuccess) e = hipMemcpyAsync(sigma.data(), sigma_d, rr * sizeof(double), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(sigma_d);
  if (e != hipSuccess) return hip_fail(e, "mla_calibrate_rotation: covariance");
  if (!eigh_ascending(r, sigma.data(), vals.data(), vecs.data()))
    return fail(MLA_ERR_NUMERIC, "mla_calibrate_rotation: non-finite covariance or eigensolver did not converge");
  std::vector<float> R(rr);
  for (size_t i = 0; i < rr; ++i) R[i] = static_cast<float>(vecs[i]);
  MLA_HIP_CHECK(hipMemcpyAsync(R_out, R.data(), rr * sizeof(float), hipMemcpyHostToDevice, s),
                "mla_calibrate_rotation: copy R");
  MLA_HIP_CHECK(hipStreamSynchronize(s), "mla_calibrate_rotation: synchronize");
  if (eig_out != nullptr) std::memcpy(eig_out, vals.data(), sizeof(double) * r);
  clear_error();
  return MLA_OK;
}

mla_status mla_calibrate_rotation_weighted(const mla_dims *dims, const void *c_cal, mla_dtype dtype,
                                           int64_t n_cal, const uint16_t *w_uk, const uint16_t *w_uv,
                                           float *R_out, double *eig_out, void *stream) {
  std::string why;
  if (!dims_valid(dims, &why)) return fail(MLA_ERR_INVALID_ARG, "mla_calibrate_rotation_weighted: " + why);
  if (c_cal == nullptr || w_uk == nullptr || w_uv == nullptr || R_out == nullptr)
    return fail(MLA_ERR_INVALID_ARG, "mla_calibrate_rotation_weighted: NULL device pointer");
  if (dtype != MLA_DTYPE_BF16 && dtype != MLA_DTYPE_FP32)
    return fail(MLA_ERR_INVALID_ARG, "mla_calibrate_rotation_weighted: dtype must be bf16 or fp32");
  if (n_cal < 1) return fail(MLA_ERR_INVALID_ARG, "mla_calibrate_rotation_weighted: n_cal must be >= 1");
  const int r = dims->kv_lora_rank;
  if (r > 4096) return fail(MLA_ERR_UNSUPPORTED, "mla_calibrate_rotation_weighted: kv_lora_rank > 4096");
  const int64_t n_uk = static_cast<int64_t>(dims->num_heads) * dims->qk_nope_head_dim;
  const int64_t n_uv = static_cast<int64_t>(dims->num_heads) * dims->v_head_dim;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t rr = static_cast<size_t>(r) * r;
  double *d_all = nullptr;
  MLA_HIP_CHECK(hipMalloc(&d_all, 3 * rr * sizeof(double)), "hipMalloc(covariances)");
  std::vector<double> sig(rr), guk(rr), guv(rr);
  // Sigma = C^T C / n over the calibration latents; W^T W / rows for the
  // stacked rows of W_UK and of W_UV (the same fp64 covariance kernel)
  hipError_t e = launch_covariance(c_cal, dtype, n_cal, r, d_all, s);
  if (e == hipSuccess) e = launch_covariance(w_uk, MLA_DTYPE_BF16, n_uk, r, d_all + rr, s);
  if (e == hipSuccess) e = launch_covariance(w_uv, MLA_DTYPE_BF16, n_uv, r, d_all + 2 * rr, s);
  if (e == hipSuccess) e = hipMemcpyAsync(sig.data(), d_all, rr * sizeof(double), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(guk.data(), d_all + rr, rr * sizeof(double), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(guv.data(), d_all + 2 * rr, rr * sizeof(double), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(d_all);
  if (e != hipSuccess) return hip_fail(e, "mla_calibrate_rotation_weighted: covariances");
  // G = sum_h W_UK[h]^T W_UK[h] + W_UV[h]^T W_UV[h] (scaled to trace r by
  // metric_whitened); Sigma_w = G^(-1/2) Sigma G^(-1/2)
  std::vector<double> g(rr), sw;
  for (size_t i = 0; i < rr; ++i) g[i] = guk[i] * static_cast<double>(n_uk) + guv[i] * static_cast<double>(n_uv);
  if (!metric_whitened(r, g, sig, sw))
    return fail(MLA_ERR_NUMERIC,
                "mla_calibrate_rotation_weighted: up-projection weights are zero or not finite, or their eigensolve failed");
  std::vector<double> vals(r), vecs(rr);
  if (!eigh_ascending(r, sw.data(), vals.data(), vecs.data()))
    return fail(MLA_ERR_NUMERIC, "mla_calibrate_rotation_weighted: non-finite covariance or eigensolver did not converge");
  std::vector<float> R(rr);
  for (size_t i = 0; i < rr; ++i) R[i] = static_cast<float>(vecs[i]);
  MLA_HIP_CHECK(hipMemcpyAsync(R_out, R.data(), rr * sizeof(float), hipMemcpyHostToDevice, s),
                "mla_calibrate_rotation_weighted: copy R");
  MLA_HIP_CHECK(hipStreamSynchronize(s), "mla_calibrate_rotation_weighted: synchronize");
  if (eig_out != nullptr) std::memcpy(eig_out, vals.data(), sizeof(double) * r);
  clear_error();
  return MLA_OK;
}

mla_status mla_prepare_rotation(const mla_dims *dims, const float *R, uint16_t *R_apply_t, void *stream) {
  std::string why;
  if (!dims_valid(dims, &why)) return fail(MLA_ERR_INVALID_ARG, "mla_prepare_rotation: " + why);
  if (R == nullptr || R_apply_t == nullptr)
    return fail(MLA_ERR_INVALID_ARG, "mla_prepare_rotation: NULL device pointer");
  hipError_t e = launch_prepare_rotation(R, dims->kv_lora_rank, R_apply_t, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mla_prepare_rotation");
  clear_error();
  return MLA_OK;
}

mla_status mla_fit_clip(const mla_dims *dims, const void *c_cal, mla_dtype dtype, int64_t n_cal,
                        const uint16_t *R_apply_t, const float *alpha_grid, int32_t n_grid,
                        float *alpha_out, double *sse_out, void *stream) {
  std::string why;
  if (!dims_valid(dims, &why)) return fail(MLA_ERR_INVALID_ARG, "mla_fit_clip: " + why);
  if (c_cal == nullptr || R_apply_t == nullptr || alpha_out == nullptr || alpha_grid == nullptr)
    return fail(MLA_ERR_INVALID_ARG, "mla_fit_clip: NULL pointer");
  if (dtype != MLA_DTYPE_BF16 && dtype != MLA_DTYPE_FP32)
    return fail(MLA_ERR_INVALID_ARG, "mla_fit_clip: dtype must be bf16 or fp32");
  if (n_cal < 1) return fail(MLA_ERR_INVALID_ARG, "mla_fit_clip: n_cal must be >= 1");
  if (n_grid < 1 || n_grid > 64) return fail(MLA_ERR_INVALID_ARG, "mla_fit_clip: n_grid must be in 1..64");
  for (int i = 0; i < n_grid; ++i)
    if (!(alpha_grid[i] > 0.0f && alpha_grid[i] <= 1.0f))
      return fail(MLA_ERR_INVALID_ARG, "mla_fit_clip: grid values must lie in (0, 1]");
  const int r = dims->kv_lora_rank, G = dims->group_size, ng = r / G;
  if (r > 1024) return fail(MLA_ERR_UNSUPPORTED, "mla_fit_clip: kv_lora_rank > 1024");
  if (!aligned16(c_cal) || !aligned16(R_apply_t))
    return fail(MLA_ERR_INVALID_ARG, "mla_fit_clip: device pointers must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  float *z = nullptr, *grid_d = nullptr;
  double *sse_d = nullptr;
  MLA_HIP_CHECK(hipMalloc(&z, static_cast<size_t>(n_cal) * r * sizeof(float)), "hipMalloc(z)");
  hipError_t e = hipMalloc(&grid_d, sizeof(float) * n_grid);
  if (e == hipSuccess) e = hipMalloc(&sse_d, sizeof(double) * ng * n_grid);
  if (e == hipSuccess) e = hipMemcpyAsync(grid_d, alpha_grid, sizeof(float) * n_grid, hipMemcpyHostToDevice, s);
  mla_cache none{};
  if (e == hipSuccess)
    e = launch_append(*dims, c_cal, dtype, nullptr, nullptr, nullptr, n_cal, R_apply_t, nullptr, none, z, s);
  if (e == hipSuccess) e = launch_group_sse(z, n_cal, r, G, grid_d, n_grid, sse_d, alpha_out, s);
  std::vector<double> sse(static_cast<size_t>(ng) * n_grid);
  if (e == hipSuccess) e = hipMemcpyAsync(sse.data(), sse_d, sizeof(double) * sse.size(), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(z);
  if (grid_d) (void)hipFree(grid_d);
  if (sse_d) (void)hipFree(sse_d);
  if (e != hipSuccess) return hip_fail(e, "mla_fit_clip");
  if (sse_out != nullptr) std::memcpy(sse_out, sse.data(), sizeof(double) * sse.size());
  clear_error();
  return MLA_OK;
}

mla_status mla_fold_absorb_weights(const mla_dims *dims, const uint16_t *w_uk, const uint16_t *w_uv,
                                   const uint16_t *R_apply_t, uint16_t *w_uk_f, uint16_t *w_uv_f,
                                   void *stream) {
  std::string why;
  if (!dims_valid(dims, &why)) return fail(MLA_ERR_INVALID_ARG, "mla_fold_absorb_weights: " + why);
  if (!w_uk || !w_uv || !R_apply_t || !w_uk_f || !w_uv_f)
    return fail(MLA_ERR_INVALID_ARG, "mla_fold_absorb_weights: NULL device pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int r = dims->kv_lora_rank, H = dims->num_heads;
  hipError_t e = launch_fold(w_uk, H * dims->qk_nope_head_dim, r, R_apply_t, w_uk_f, dims->qk_nope_head_dim, s);
  if (e == hipSuccess) e = launch_fold(w_uv, H * dims->v_head_dim, r, R_apply_t, w_uv_f, 0, s);
  if (e != hipSuccess) return hip_fail(e, "mla_fold_absorb_weights");
  clear_error();
  return MLA_OK;
}

}  // extern "C"

namespace {
// Host-side checks of a quantise-on-append call (no side effects); F names
// the entry point in the message.
mla_status append_check(const std::string &F, const mla_dims *dims, const void *latent, mla_dtype dtype,
                        const uint16_t *k_rope, const uint16_t *idx_key, const int64_t *slot_mapping, int64_t n,
                        const uint16_t *R_apply_t, const float *alpha, const mla_cache *cache) {
  std::string why;
  if (!dims_valid(dims, &why)) return fail(MLA_ERR_INVALID_ARG, F + why);
  if (dtype != MLA_DTYPE_BF16 && dtype != MLA_DTYPE_FP32)
    return fail(MLA_ERR_INVALID_ARG, F + "dtype must be bf16 or fp32");
  if (n < 0) return fail(MLA_ERR_INVALID_ARG, F + "n must be >= 0");
  if (cache == nullptr) return fail(MLA_ERR_INVALID_ARG, F + "cache is NULL");
  if (n == 0) return MLA_OK;
  if (!latent || !k_rope || !slot_mapping || !R_apply_t || !alpha || !cache->codes || !cache->scale_zero ||
      !cache->k_rope)
    return fail(MLA_ERR_INVALID_ARG, F + "NULL device pointer");
  if ((dims->index_head_dim > 0) != (idx_key != nullptr) ||
      (dims->index_head_dim > 0 && cache->idx_key == nullptr))
    return fail(MLA_ERR_INVALID_ARG, F + "idx_key and cache.idx_key must be given iff index_head_dim > 0");
  if (cache->capacity < 0) return fail(MLA_ERR_INVALID_ARG, F + "negative capacity");
  if (dims->kv_lora_rank > 1024 && !append_uses_mfma(*dims, dtype))
    return fail(MLA_ERR_UNSUPPORTED, F + "kv_lora_rank > 1024");
  if (n > (int64_t{1} << 31) - 1) return fail(MLA_ERR_UNSUPPORTED, F + "n >= 2^31");
  const void *ptrs[] = {latent, k_rope, idx_key, slot_mapping, R_apply_t, alpha, cache->codes,
                        cache->scale_zero, cache->k_rope, cache->idx_key};
  for (const void *p : ptrs)
    if (p != nullptr && !aligned16(p))
      return fail(MLA_ERR_INVALID_ARG, F + "device pointers must be 16-byte aligned");
  return MLA_OK;
}
}  // namespace

extern "C" {

mla_status mla_append_quant(const mla_dims *dims, const void *latent, mla_dtype dtype,
                            const uint16_t *k_rope, const uint16_t *idx_key, const int64_t *slot_mapping,
                            int64_t n, const uint16_t *R_apply_t, const float *alpha, const mla_cache *cache,
                            void *stream) {
  const mla_status st = append_check("mla_append_quant: ", dims, latent, dtype, k_rope, idx_key, slot_mapping, n,
                                     R_apply_t, alpha, cache);
  if (st != MLA_OK) return st;
  if (n == 0) {
    clear_error();
    return MLA_OK;
  }
  hipError_t e = launch_append(*dims, latent, dtype, k_rope, idx_key, slot_mapping, n, R_apply_t, alpha, *cache,
                               nullptr, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mla_append_quant");
  clear_error();
  return MLA_OK;
}

size_t mla_decode_workspace_size(const mla_dims *dims, int32_t batch, int32_t tq) {
  std::string why;
  if (!dims_valid(dims, &why) || batch < 0 || tq < 1 || tq > 64) return 0;
  return layout(*dims, batch, tq).total;
}

}  // extern "C"

namespace {

// Shared by the dense and the sparse entry points: with sel != nullptr the
// tokens of sequence b are the slots seq_base[b] + sel[b * sel_stride + t],
// t < seq_len[b] (the selected counts).
mla_status decode_impl(const char *fn, const mla_dims *dims, const uint16_t *q_nope, const uint16_t *q_rope,
                       const uint16_t *w_uk_f, const uint16_t *w_uv_f, const mla_cache *cache,
                       const int64_t *seq_base, const int32_t *seq_len, const int32_t *sel, int32_t sel_stride,
                       int32_t batch, int32_t tq, int32_t causal, float softmax_scale, void *workspace,
                       size_t workspace_bytes, float *out, float *lse, void *stream,
                       const AppendJob *job = nullptr, mla_dtype job_dtype = MLA_DTYPE_BF16) {
  // messages are built only on failure (no host allocation on the way)
  auto F = [fn](const std::string &m) { return std::string(fn) + ": " + m; };
  std::string why;
  if (!dims_valid(dims, &why)) return fail(MLA_ERR_INVALID_ARG, F(why));
  if (batch < 0) return fail(MLA_ERR_INVALID_ARG, F("batch must be >= 0"));
  if (tq < 1 || tq > 64) return fail(MLA_ERR_INVALID_ARG, F("tq must be in 1..64"));
  if (causal != 0 && causal != 1) return fail(MLA_ERR_INVALID_ARG, F("causal must be 0 or 1"));
  if (!std::isfinite(softmax_scale)) return fail(MLA_ERR_INVALID_ARG, F("softmax_scale not finite"));
  if (cache == nullptr) return fail(MLA_ERR_INVALID_ARG, F("cache is NULL"));
  if (batch == 0) {
    if (job != nullptr) {  // the step's append still runs
      const hipError_t e = launch_append(*dims, job->latent, job_dtype, job->k_rope, job->idx_key, job->slots, job->n,
                                         job->Rt, job->alpha, *cache, nullptr, static_cast<hipStream_t>(stream));
      if (e != hipSuccess) return hip_fail(e, fn);
    }
    clear_error();
    return MLA_OK;
  }
  if (!q_nope || !q_rope || !w_uk_f || !w_uv_f || !seq_base || !seq_len || !workspace || !out ||
      !cache->codes || !cache->scale_zero || !cache->k_rope)
    return fail(MLA_ERR_INVALID_ARG, F("NULL device pointer"));
  const void *ptrs[] = {q_nope, q_rope, w_uk_f, w_uv_f, seq_base, seq_len, workspace, out, lse,
                        cache->codes, cache->scale_zero, cache->k_rope};
  for (const void *p : ptrs)
    if (p != nullptr && !aligned16(p))
      return fail(MLA_ERR_INVALID_ARG, F("device pointers must be 16-byte aligned"));
  if (dims->kv_lora_rank > 512)
    return fail(MLA_ERR_UNSUPPORTED, F("kv_lora_rank > 512"));
  const int M = dims->num_heads * tq;
  bool use_mfma = false;
  if (g_decode_variant == 2) {
    if (!mfma_decode_supported(*dims, M))
      return fail(MLA_ERR_UNSUPPORTED, F("no MFMA kernel for this shape"));
    use_mfma = true;
  } else if (g_decode_variant == 0) {
    // the MFMA kernels wherever the shape has them (at most 16 query rows
    // take the 16-row kernel), else the vector-ALU kernel
    use_mfma = mfma_decode_supported(*dims, M) && mfma_absorb_supported(*dims);
  }
  if (use_mfma && !mfma_absorb_supported(*dims))
    return fail(MLA_ERR_UNSUPPORTED, F("qk_nope_head_dim must be a multiple of 16 for the MFMA path"));
  const WsLayout w = layout(*dims, batch, tq);
  if (workspace_bytes < w.total)
    return fail(MLA_ERR_WORKSPACE, F("workspace needs ") + std::to_string(w.total) + " bytes");
  DecodeArgs a{};
  a.d = *dims;
  a.q_nope = q_nope;
  a.q_rope = q_rope;
  a.w_uk_f = w_uk_f;
  a.w_uv_f = w_uv_f;
  a.cache = *cache;
  a.seq_base = seq_base;
  a.seq_len = seq_len;
  a.B = batch;
  a.Tq = tq;
  a.causal = causal;
  a.scale_log2 = softmax_scale * kLog2e;
  a.out = out;
  a.lse = lse;
  char *ws = static_cast<char *>(workspace);
  a.items = reinterpret_cast<WorkItem *>(ws + w.items);
  a.item_begin = reinterpret_cast<int32_t *>(ws + w.item_begin);
  a.meta = reinterpret_cast<int32_t *>(ws + w.meta);
  a.qbuf = ws + w.qbuf;
  a.oz = reinterpret_cast<float *>(ws + w.oz);
  a.part_o = reinterpret_cast<uint16_t *>(ws + w.part_o);
  a.part_ml = reinterpret_cast<float *>(ws + w.part_ml);
  a.max_items = w.max_items;
  a.target_items = target_items(M, use_mfma, sel != nullptr);
  a.tile = use_mfma ? 32 : 16;
  a.min_chunk_tiles = min_chunk_tiles(a.tile);
  a.sel = sel;
  a.sel_stride = sel_stride;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the MFMA absorb kernel also runs the planner, and takes a step's small
  // append as extra blocks; any other append runs first on its own
  const bool fuse = job != nullptr && use_mfma && append_fusable(*dims, job_dtype, job->n);
  hipError_t e = hipSuccess;
  if (job != nullptr && !fuse)
    e = launch_append(*dims, job->latent, job_dtype, job->k_rope, job->idx_key, job->slots, job->n, job->Rt,
                      job->alpha, *cache, nullptr, s);
  if (e == hipSuccess) e = use_mfma ? launch_absorb_mfma_layout(a, s, fuse ? job : nullptr) : launch_plan(a, s);
  if (e == hipSuccess && !use_mfma) e = launch_absorb_f32(a, s);
  if (e == hipSuccess) e = use_mfma ? launch_splitk_mfma(a, s) : launch_splitk_valu(a, s);
  if (e == hipSuccess) e = launch_combine(a, s);
  if (e == hipSuccess) e = launch_upproj(a, s);
  if (e != hipSuccess) return hip_fail(e, fn);
  clear_error();
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status mla_decode_absorbed(const mla_dims *dims, const uint16_t *q_nope, const uint16_t *q_rope,
                               const uint16_t *w_uk_f, const uint16_t *w_uv_f, const mla_cache *cache,
                               const int64_t *seq_base, const int32_t *seq_len, int32_t batch, int32_t tq,
                               int32_t causal, float softmax_scale, void *workspace, size_t workspace_bytes,
                               float *out, float *lse, void *stream) {
  return decode_impl("mla_decode_absorbed", dims, q_nope, q_rope, w_uk_f, w_uv_f, cache, seq_base, seq_len,
                     nullptr, 0, batch, tq, causal, softmax_scale, workspace, workspace_bytes, out, lse, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// decode with the library's own static device scratch (no allocation)
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = size_t{48} << 20;
constexpr int kMaxDevices = 64;

// The decode workspace of mla_decode_absorbed_noalloc.  Host code never
// uses this name as an address (on the host it is only a stand-in): the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on the
// device's first call and kept.
mla_status scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "mla_decode_absorbed_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MLA_ERR_UNSUPPORTED, "mla_decode_absorbed_noalloc: device index beyond the supported 64");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "mla_decode_absorbed_noalloc: hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(MLA_ERR_HIP, "mla_decode_absorbed_noalloc: scratch has no device address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}

}  // namespace

extern "C" {

size_t mla_decode_noalloc_max_workspace(void) { return kScratchBytes; }

mla_status mla_decode_absorbed_noalloc(const mla_dims *dims, const uint16_t *q_nope, const uint16_t *q_rope,
                                       const uint16_t *w_uk_f, const uint16_t *w_uv_f, const mla_cache *cache,
                                       const int64_t *seq_base, const int32_t *seq_len, int32_t batch,
                                       int32_t tq, int32_t causal, float softmax_scale, float *out, float *lse,
                                       void *stream) {
  std::string why;
  if (!dims_valid(dims, &why)) return fail(MLA_ERR_INVALID_ARG, "mla_decode_absorbed_noalloc: " + why);
  if (batch < 0 || tq < 1 || tq > 64)
    return fail(MLA_ERR_INVALID_ARG, "mla_decode_absorbed_noalloc: batch must be >= 0 and tq in 1..64");
  const size_t need = layout(*dims, batch, tq).total;
  if (need > kScratchBytes)
    return fail(MLA_ERR_WORKSPACE, "mla_decode_absorbed_noalloc: this decode needs " + std::to_string(need) +
                                       " bytes of workspace; the static scratch holds " +
                                       std::to_string(kScratchBytes) + " (use mla_decode_absorbed)");
  void *ws = nullptr;
  const mla_status st = scratch_address(&ws);
  if (st != MLA_OK) return st;
  return decode_impl("mla_decode_absorbed_noalloc", dims, q_nope, q_rope, w_uk_f, w_uv_f, cache, seq_base,
                     seq_len, nullptr, 0, batch, tq, causal, softmax_scale, ws, kScratchBytes, out, lse, stream);
}

mla_status mla_decode_step(const mla_dims *dims, const void *latent, mla_dtype dtype, const uint16_t *k_rope,
                           const uint16_t *idx_key, const int64_t *slot_mapping, int64_t n,
                           const uint16_t *R_apply_t, const float *alpha, const uint16_t *q_nope,
                           const uint16_t *q_rope, const uint16_t *w_uk_f, const uint16_t *w_uv_f,
                           const mla_cache *cache, const int64_t *seq_base, const int32_t *seq_len, int32_t batch,
                           int32_t tq, int32_t causal, float softmax_scale, void *workspace,
                           size_t workspace_bytes, float *out, float *lse, void *stream) {
  const mla_status st = append_check("mla_decode_step: ", dims, latent, dtype, k_rope, idx_key, slot_mapping, n,
                                     R_apply_t, alpha, cache);
  if (st != MLA_OK) return st;
  AppendJob job{latent, k_rope, idx_key, slot_mapping, n, R_apply_t, alpha};
  return decode_impl("mla_decode_step", dims, q_nope, q_rope, w_uk_f, w_uv_f, cache, seq_base, seq_len, nullptr,
                     0, batch, tq, causal, softmax_scale, workspace, workspace_bytes, out, lse, stream,
                     n > 0 ? &job : nullptr, dtype);
}

namespace {
// Workspace of mla_index_topk: scores, histograms, prefixes, chunk counts.
struct IndexWorkspace {
  size_t scores, hist, pfx_bits, pfx_rank, chunk_above, chunk_suf, total;
};

IndexWorkspace index_workspace(int32_t batch, int64_t capacity) {
  const size_t B = static_cast<size_t>(batch), nc = static_cast<size_t>(mla::index_chunks());
  IndexWorkspace w;
  size_t off = 0;
  w.scores = off;
  off = align256(off + static_cast<size_t>(capacity) * sizeof(float));
  w.hist = off;
  off = align256(off + sizeof(uint32_t) * mla::index_passes() * mla::index_hist_bins() * B);
  w.pfx_bits = off;
  off = align256(off + sizeof(uint32_t) * (mla::index_passes() - 1) * B);
  w.pfx_rank = off;
  off = align256(off + sizeof(int32_t) * (mla::index_passes() - 1) * B);
  w.chunk_above = off;
  off = align256(off + sizeof(int32_t) * nc * B);
  w.chunk_suf = off;
  off = align256(off + sizeof(int32_t) * nc * mla::index_last_bins() * B);
  w.total = off;
  return w;
}
}  // namespace

size_t mla_index_topk_workspace_size(const mla_dims *dims, int32_t batch, int64_t capacity) {
  std::string why;
  if (!dims_valid(dims, &why) || batch < 0 || capacity < 0) return 0;
  return index_workspace(batch, capacity).total;
}

mla_status mla_index_topk(const mla_dims *dims, const uint16_t *q_idx, const mla_cache *cache,
                          const int64_t *seq_base, const int32_t *seq_len, int32_t batch, int32_t top_k,
                          void *workspace, size_t workspace_bytes, int32_t *sel, int32_t *n_sel, void *stream) {
  std::string why;
  if (!dims_valid(dims, &why)) return fail(MLA_ERR_INVALID_ARG, "mla_index_topk: " + why);
  if (dims->index_head_dim <= 0)
    return fail(MLA_ERR_INVALID_ARG, "mla_index_topk: the layer has no indexer key (index_head_dim = 0)");
  if (dims->index_head_dim != 64 && dims->index_head_dim != 128)
    return fail(MLA_ERR_UNSUPPORTED, "mla_index_topk: index_head_dim must be 64 or 128");
  if (batch < 0) return fail(MLA_ERR_INVALID_ARG, "mla_index_topk: batch must be >= 0");
  if (top_k < 1) return fail(MLA_ERR_INVALID_ARG, "mla_index_topk: top_k must be >= 1");
  if (cache == nullptr) return fail(MLA_ERR_INVALID_ARG, "mla_index_topk: cache is NULL");
  if (batch == 0) {
    clear_error();
    return MLA_OK;
  }
  if (!q_idx || !seq_base || !seq_len || !workspace || !sel || !n_sel || !cache->idx_key)
    return fail(MLA_ERR_INVALID_ARG, "mla_index_topk: NULL device pointer");
  const void *ptrs[] = {q_idx, seq_base, seq_len, workspace, sel, n_sel, cache->idx_key};
  for (const void *p : ptrs)
    if (!aligned16(p)) return fail(MLA_ERR_INVALID_ARG, "mla_index_topk: device pointers must be 16-byte aligned");
  const size_t need = mla_index_topk_workspace_size(dims, batch, cache->capacity);
  if (workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "mla_index_topk: workspace needs " + std::to_string(need) + " bytes");
  IndexArgs a;
  a.q_idx = q_idx;
  a.idx_key = cache->idx_key;
  a.seq_base = seq_base;
  a.seq_len = seq_len;
  a.B = batch;
  a.d_idx = dims->index_head_dim;
  a.top_k = top_k;
  a.n_chunks = index_chunks();
  char *ws = static_cast<char *>(workspace);
  const IndexWorkspace w = index_workspace(batch, cache->capacity);
  a.scores = reinterpret_cast<float *>(ws + w.scores);
  a.hist = reinterpret_cast<uint32_t *>(ws + w.hist);
  a.pfx_bits = reinterpret_cast<uint32_t *>(ws + w.pfx_bits);
  a.pfx_rank = reinterpret_cast<int32_t *>(ws + w.pfx_rank);
  a.chunk_above = reinterpret_cast<int32_t *>(ws + w.chunk_above);
  a.chunk_suf = reinterpret_cast<int32_t *>(ws + w.chunk_suf);
  a.sel = sel;
  a.n_sel = n_sel;
  hipError_t e = launch_index_topk(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mla_index_topk");
  clear_error();
  return MLA_OK;
}

mla_status mla_decode_sparse(const mla_dims *dims, const uint16_t *q_nope, const uint16_t *q_rope,
                             const uint16_t *w_uk_f, const uint16_t *w_uv_f, const mla_cache *cache,
                             const int64_t *seq_base, const int32_t *sel, const int32_t *n_sel, int32_t batch,
                             int32_t top_k, float softmax_scale, void *workspace, size_t workspace_bytes,
                             float *out, float *lse, void *stream) {
  if (top_k < 1) return fail(MLA_ERR_INVALID_ARG, "mla_decode_sparse: top_k must be >= 1");
  if (batch > 0 && (sel == nullptr || n_sel == nullptr))
    return fail(MLA_ERR_INVALID_ARG, "mla_decode_sparse: NULL device pointer");
  if (batch > 0 && (!aligned16(sel) || !aligned16(n_sel)))
    return fail(MLA_ERR_INVALID_ARG, "mla_decode_sparse: device pointers must be 16-byte aligned");
  return decode_impl("mla_decode_sparse", dims, q_nope, q_rope, w_uk_f, w_uv_f, cache, seq_base, n_sel, sel, top_k,
                     batch, 1, 0, softmax_scale, workspace, workspace_bytes, out, lse, stream);
}


// ---------------------------------------------------------------------------
// OSCAR for full-attention (grouped-query) layers
mla_status gqa_calibrate(const gqa_dims *dims, const uint16_t *q_cal, const uint16_t *k_cal, const uint16_t *v_cal,
                         int64_t n_cal, float softmax_scale, float *R_k, float *R_v, double *eig_k, double *eig_v,
                         void *stream) {
  std::string why;
  if (!gqa_dims_valid(dims, &why)) return fail(MLA_ERR_INVALID_ARG, "gqa_calibrate: " + why);
  if (!q_cal || !k_cal || !v_cal || !R_k || !R_v) return fail(MLA_ERR_INVALID_ARG, "gqa_calibrate: NULL device pointer");
  const void *ptrs[] = {q_cal, k_cal, v_cal};
  for (const void *p : ptrs)
    if (!aligned16(p)) return fail(MLA_ERR_INVALID_ARG, "gqa_calibrate: device pointers must be 16-byte aligned");
  if (n_cal < 1 || n_cal > 65536) return fail(MLA_ERR_INVALID_ARG, "gqa_calibrate: n_cal must be in 1..65536");
  if (!std::isfinite(softmax_scale)) return fail(MLA_ERR_INVALID_ARG, "gqa_calibrate: softmax_scale not finite");
  const int d = dims->head_dim, Hq = dims->num_q_heads, Hkv = dims->num_kv_heads, G = Hq / Hkv;
  const int n = static_cast<int>(n_cal);
  const size_t dd = static_cast<size_t>(d) * d;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // device scratch: Sigma_q, Sigma_k, Sigma_v [H_kv][d][d], row stats [H_q][n] x 2, masses [H_kv][n]
  const size_t n_dbl = 3 * Hkv * dd + 2 * static_cast<size_t>(Hq) * n + static_cast<size_t>(Hkv) * n;
  double *buf = nullptr;
  MLA_HIP_CHECK(hipMalloc(&buf, n_dbl * sizeof(double)), "gqa_calibrate: hipMalloc");
  double *sig_q = buf, *sig_k = sig_q + Hkv * dd, *sig_v = sig_k + Hkv * dd;
  double *row_m = sig_v + Hkv * dd, *row_inv = row_m + static_cast<size_t>(Hq) * n;
  double *mass = row_inv + static_cast<size_t>(Hq) * n;
  hipError_t e = hipSuccess;
  for (int h = 0; h < Hkv && e == hipSuccess; ++h) {
    // the G query heads of KV head h are contiguous rows: [G * n][d]
    e = launch_covariance(q_cal + static_cast<size_t>(h) * G * n * d, MLA_DTYPE_BF16, static_cast<int64_t>(G) * n, d,
                          sig_q + h * dd, s);
    if (e == hipSuccess)
      e = launch_covariance(k_cal + static_cast<size_t>(h) * n * d, MLA_DTYPE_BF16, n, d, sig_k + h * dd, s);
  }
  if (e == hipSuccess)
    e = launch_gqa_calib_stats(q_cal, k_cal, v_cal, n, d, Hq, Hkv, static_cast<double>(softmax_scale), row_m,
                               row_inv, mass, sig_v, s);
  std::vector<double> hq(Hkv * dd), hk(Hkv * dd), hv(Hkv * dd);
  if (e == hipSuccess) e = hipMemcpyAsync(hq.data(), sig_q, Hkv * dd * sizeof(double), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(hk.data(), sig_k, Hkv * dd * sizeof(double), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(hv.data(), sig_v, Hkv * dd * sizeof(double), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(buf);
  if (e != hipSuccess) return hip_fail(e, "gqa_calibrate: statistics");
  std::vector<float> rk(Hkv * dd), rv(Hkv * dd);
  std::vector<double> vals(d), vecs(dd), sw;
  for (int h = 0; h < Hkv; ++h) {
    std::vector<double> sq(hq.begin() + h * dd, hq.begin() + (h + 1) * dd);
    if (dims->k_rotation == GQA_K_QUERY_METRIC) {
      std::vector<double> sk(hk.begin() + h * dd, hk.begin() + (h + 1) * dd);
      if (!metric_whitened(d, sq, sk, sw))
        return fail(MLA_ERR_NUMERIC, "gqa_calibrate: query covariance is zero or not finite, or its eigensolve failed");
    } else {
      sw = sq;
    }
    if (!eigh_ascending(d, sw.data(), vals.data(), vecs.data()))
      return fail(MLA_ERR_NUMERIC, "gqa_calibrate: key or query statistics not finite or eigensolver did not converge");
    for (size_t i = 0; i < dd; ++i) rk[h * dd + i] = static_cast<float>(vecs[i]);
    if (eig_k != nullptr) std::memcpy(eig_k + static_cast<size_t>(h) * d, vals.data(), sizeof(double) * d);
    if (!eigh_ascending(d, hv.data() + h * dd, vals.data(), vecs.data()))
      return fail(MLA_ERR_NUMERIC, "gqa_calibrate: value statistics not finite or eigensolver did not converge");
    for (size_t i = 0; i < dd; ++i) rv[h * dd + i] = static_cast<float>(vecs[i]);
    if (eig_v != nullptr) std::memcpy(eig_v + static_cast<size_t>(h) * d, vals.data(), sizeof(double) * d);
  }
  MLA_HIP_CHECK(hipMemcpyAsync(R_k, rk.data(), rk.size() * sizeof(float), hipMemcpyHostToDevice, s),
                "gqa_calibrate: copy R_k");
  MLA_HIP_CHECK(hipMemcpyAsync(R_v, rv.data(), rv.size() * sizeof(float), hipMemcpyHostToDevice, s),
                "gqa_calibrate: copy R_v");
  MLA_HIP_CHECK(hipStreamSynchronize(s), "gqa_calibrate: synchronize");
  clear_error();
  return MLA_OK;
}

mla_status gqa_prepare_rotation(const gqa_dims *dims, const float *R, uint16_t *R_apply_t, void *stream) {
  std::string why;
  if (!gqa_dims_valid(dims, &why)) return fail(MLA_ERR_INVALID_ARG, "gqa_prepare_rotation: " + why);
  if (R == nullptr || R_apply_t == nullptr) return fail(MLA_ERR_INVALID_ARG, "gqa_prepare_rotation: NULL device pointer");
  const int d = dims->head_dim;
  const size_t dd = static_cast<size_t>(d) * d;
  hipError_t e = hipSuccess;
  for (int h = 0; h < dims->num_kv_heads && e == hipSuccess; ++h)
    e = launch_prepare_rotation(R + h * dd, d, R_apply_t + h * dd, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gqa_prepare_rotation");
  clear_error();
  return MLA_OK;
}

mla_status gqa_fit_clip(const gqa_dims *dims, const uint16_t *x_cal, int64_t n_cal, const uint16_t *R_apply_t,
                        const float *alpha_grid, int32_t n_grid, float *alpha_out, void *stream) {
  std::string why;
  if (!gqa_dims_valid(dims, &why)) return fail(MLA_ERR_INVALID_ARG, "gqa_fit_clip: " + why);
  if (!x_cal || !R_apply_t || !alpha_grid || !alpha_out) return fail(MLA_ERR_INVALID_ARG, "gqa_fit_clip: NULL pointer");
  if (!aligned16(x_cal) || !aligned16(R_apply_t))
    return fail(MLA_ERR_INVALID_ARG, "gqa_fit_clip: device pointers must be 16-byte aligned");
  if (n_cal < 1) return fail(MLA_ERR_INVALID_ARG, "gqa_fit_clip: n_cal must be >= 1");
  if (n_grid < 1 || n_grid > 64) return fail(MLA_ERR_INVALID_ARG, "gqa_fit_clip: n_grid must be in 1..64");
  for (int i = 0; i < n_grid; ++i)
    if (!(alpha_grid[i] > 0.0f && alpha_grid[i] <= 1.0f))
      return fail(MLA_ERR_INVALID_ARG, "gqa_fit_clip: grid values must lie in (0, 1]");
  const mla_dims dl = gqa_latent_dims(*dims);
  const int d = dims->head_dim, G = dims->group_size, ng = d / G;
  const size_t dd = static_cast<size_t>(d) * d;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float *z = nullptr, *grid_d = nullptr;
  double *sse_d = nullptr;
  MLA_HIP_CHECK(hipMalloc(&z, static_cast<size_t>(n_cal) * d * sizeof(float)), "gqa_fit_clip: hipMalloc");
  hipError_t e = hipMalloc(&grid_d, sizeof(float) * n_grid);
  if (e == hipSuccess) e = hipMalloc(&sse_d, sizeof(double) * ng * n_grid);
  if (e == hipSuccess) e = hipMemcpyAsync(grid_d, alpha_grid, sizeof(float) * n_grid, hipMemcpyHostToDevice, s);
  mla_cache none{};
  for (int h = 0; h < dims->num_kv_heads && e == hipSuccess; ++h) {
    // rotated rows of head h (the append arithmetic), then the per-group search
    e = launch_append(dl, x_cal + static_cast<size_t>(h) * n_cal * d, MLA_DTYPE_BF16, nullptr, nullptr, nullptr,
                      n_cal, R_apply_t + h * dd, nullptr, none, z, s);
    if (e == hipSuccess) e = launch_group_sse(z, n_cal, d, G, grid_d, n_grid, sse_d, alpha_out + h * ng, s);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(z);
  if (grid_d) (void)hipFree(grid_d);
  if (sse_d) (void)hipFree(sse_d);
  if (e != hipSuccess) return hip_fail(e, "gqa_fit_clip");
  clear_error();
  return MLA_OK;
}

mla_status gqa_append_quant(const gqa_dims *dims, const uint16_t *k, const uint16_t *v, const int64_t *slot_mapping,
                            int64_t n, const uint16_t *Rk_apply_t, const uint16_t *Rv_apply_t, const float *alpha_k,
                            const float *alpha_v, const gqa_cache *cache, void *stream) {
  std::string why;
  if (!gqa_dims_valid(dims, &why)) return fail(MLA_ERR_INVALID_ARG, "gqa_append_quant: " + why);
  if (n < 0) return fail(MLA_ERR_INVALID_ARG, "gqa_append_quant: n must be >= 0");
  if (cache == nullptr) return fail(MLA_ERR_INVALID_ARG, "gqa_append_quant: cache is NULL");
  if (n == 0) {
    clear_error();
    return MLA_OK;
  }
  if (!k || !v || !slot_mapping || !Rk_apply_t || !Rv_apply_t || !alpha_k || !alpha_v || !cache->k_codes ||
      !cache->k_scale_zero || !cache->v_codes || !cache->v_scale_zero)
    return fail(MLA_ERR_INVALID_ARG, "gqa_append_quant: NULL device pointer");
  const void *ptrs[] = {k, v, Rk_apply_t, Rv_apply_t, cache->k_codes, cache->k_scale_zero, cache->v_codes,
                        cache->v_scale_zero};
  for (const void *p : ptrs)
    if (!aligned16(p)) return fail(MLA_ERR_INVALID_ARG, "gqa_append_quant: device pointers must be 16-byte aligned");
  if (cache->capacity < 0) return fail(MLA_ERR_INVALID_ARG, "gqa_append_quant: capacity must be >= 0");
  const mla_dims dl = gqa_latent_dims(*dims);
  const int d = dims->head_dim, ng = d / dims->group_size, Hkv = dims->num_kv_heads;
  const size_t dd = static_cast<size_t>(d) * d;
  const int64_t cap = cache->capacity;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  for (int h = 0; h < Hkv && e == hipSuccess; ++h) {
    for (int side = 0; side < 2 && e == hipSuccess; ++side) {
      mla_cache c{};
      c.codes = (side ? cache->v_codes : cache->k_codes) + static_cast<size_t>(h) * cap * (d / 4);
      c.scale_zero = (side ? cache->v_scale_zero : cache->k_scale_zero) + static_cast<size_t>(h) * cap * ng * 2;
      c.capacity = cap;
      e = launch_append(dl, (side ? v : k) + static_cast<size_t>(h) * d, MLA_DTYPE_BF16, nullptr, nullptr,
                        slot_mapping, n, (side ? Rv_apply_t : Rk_apply_t) + h * dd,
                        (side ? alpha_v : alpha_k) + h * ng, c, nullptr, s, static_cast<int64_t>(Hkv) * d);
    }
  }
  if (e != hipSuccess) return hip_fail(e, "gqa_append_quant");
  clear_error();
  return MLA_OK;
}

size_t gqa_decode_workspace_size(const gqa_dims *dims, int32_t batch, int32_t tq) {
  std::string why;
  if (!gqa_dims_valid(dims, &why) || batch < 0 || tq < 1 || tq > 64) return 0;
  return gqa_layout(*dims, batch, tq).total;
}

mla_status gqa_decode(const gqa_dims *dims, const uint16_t *q, const gqa_cache *cache, const uint16_t *Rk_apply_t,
                      const uint16_t *Rv_apply_t, const int64_t *seq_base, const int32_t *seq_len, int32_t batch,
                      int32_t tq, int32_t causal, float softmax_scale, void *workspace, size_t workspace_bytes,
                      float *out, float *lse, void *stream) {
  std::string why;
  if (!gqa_dims_valid(dims, &why)) return fail(MLA_ERR_INVALID_ARG, "gqa_decode: " + why);
  if (batch < 0) return fail(MLA_ERR_INVALID_ARG, "gqa_decode: batch must be >= 0");
  if (tq < 1 || tq > 64) return fail(MLA_ERR_INVALID_ARG, "gqa_decode: tq must be in 1..64");
  if (causal != 0 && causal != 1) return fail(MLA_ERR_INVALID_ARG, "gqa_decode: causal must be 0 or 1");
  if (!std::isfinite(softmax_scale)) return fail(MLA_ERR_INVALID_ARG, "gqa_decode: softmax_scale not finite");
  if (cache == nullptr) return fail(MLA_ERR_INVALID_ARG, "gqa_decode: cache is NULL");
  if (batch == 0) {
    clear_error();
    return MLA_OK;
  }
  if (!q || !Rk_apply_t || !Rv_apply_t || !seq_base || !seq_len || !workspace || !out || !cache->k_codes ||
      !cache->k_scale_zero || !cache->v_codes || !cache->v_scale_zero)
    return fail(MLA_ERR_INVALID_ARG, "gqa_decode: NULL device pointer");
  const void *ptrs[] = {q, Rk_apply_t, Rv_apply_t, seq_base, seq_len, workspace, out, lse,
                        cache->k_codes, cache->k_scale_zero, cache->v_codes, cache->v_scale_zero};
  for (const void *p : ptrs)
    if (p != nullptr && !aligned16(p))
      return fail(MLA_ERR_INVALID_ARG, "gqa_decode: device pointers must be 16-byte aligned");
  const GqaWs w = gqa_layout(*dims, batch, tq);
  if (workspace_bytes < w.total)
    return fail(MLA_ERR_WORKSPACE, "gqa_decode: workspace needs " + std::to_string(w.total) + " bytes");
  const int Hkv = dims->num_kv_heads, G = dims->num_q_heads / Hkv;
  const int Bp = batch * Hkv, M = G * tq;
  char *ws = static_cast<char *>(workspace);
  // the shared split-K stages over B * H_kv pseudo-sequences (sequence, KV
  // head) of G query heads each, K and V from their own caches
  DecodeArgs a{};
  a.d = gqa_latent_dims(*dims);
  a.cache.codes = cache->k_codes;
  a.cache.scale_zero = cache->k_scale_zero;
  a.cache.capacity = static_cast<int64_t>(Hkv) * cache->capacity;
  a.vcache.codes = cache->v_codes;
  a.vcache.scale_zero = cache->v_scale_zero;
  a.vcache.capacity = a.cache.capacity;
  a.seq_base = reinterpret_cast<int64_t *>(ws + w.base2);
  a.seq_len = reinterpret_cast<int32_t *>(ws + w.len2);
  a.B = Bp;
  a.Tq = tq;
  a.causal = causal;
  a.scale_log2 = softmax_scale * kLog2e;
  a.items = reinterpret_cast<WorkItem *>(ws + w.split.items);
  a.item_begin = reinterpret_cast<int32_t *>(ws + w.split.item_begin);
  a.meta = reinterpret_cast<int32_t *>(ws + w.split.meta);
  a.qbuf = ws + w.split.qbuf;
  a.oz = reinterpret_cast<float *>(ws + w.split.oz);
  a.part_o = reinterpret_cast<uint16_t *>(ws + w.split.part_o);
  a.part_ml = reinterpret_cast<float *>(ws + w.split.part_ml);
  a.max_items = w.split.max_items;
  const bool use_mfma = gqa_use_mfma(*dims, tq);
  a.target_items = gqa_target_items(*dims, tq);
  a.tile = use_mfma ? 32 : 16;
  a.min_chunk_tiles = min_chunk_tiles(a.tile);
  GqaDecodeArgs g{};
  g.q = q;
  g.rk_t = Rk_apply_t;
  g.rv_t = Rv_apply_t;
  g.seq_base = seq_base;
  g.seq_len = seq_len;
  g.capacity = cache->capacity;
  g.B = batch;
  g.Tq = tq;
  g.H_q = dims->num_q_heads;
  g.H_kv = Hkv;
  g.d = dims->head_dim;
  g.scale_log2 = a.scale_log2;
  g.qbuf = static_cast<float *>(a.qbuf);
  g.base2 = const_cast<int64_t *>(a.seq_base);
  g.len2 = const_cast<int32_t *>(a.seq_len);
  g.out = out;
  g.lse = lse;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_gqa_rotate_q(g, a, s);  // also plans the split-K items
  if (e == hipSuccess) e = use_mfma ? launch_gqa_splitk_mfma(a, s) : launch_splitk_valu(a, s);
  if (e == hipSuccess) e = launch_gqa_merge_unrotate(g, a, s);
  if (e != hipSuccess) return hip_fail(e, "gqa_decode");
  clear_error();
  return MLA_OK;
}

}  // extern "C"
