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

// Work items that fill the GPU: one resident block per (item, row block).
int target_items(int rows, bool mfma) {
  const int ncu = device_cu_count();
  const int rb = mfma ? (rows + mfma_row_block() - 1) / mfma_row_block() : (rows + 15) / 16;
  const int slots = mfma ? ncu : 2 * ncu;  // resident blocks per launch
  const int t = slots / rb;
  return t < 1 ? 1 : t;
}

// Shortest split-K chunk, in tokens: below it the fixed cost of an item
// (query rows in, partial rows out, the combine reading them back) outweighs
// spreading a short context over more compute units.
#ifndef MLA_SPLIT_MIN_TOKENS
#define MLA_SPLIT_MIN_TOKENS 64
#endif
int min_chunk_tiles(int tile) { return (MLA_SPLIT_MIN_TOKENS + tile - 1) / tile; }

WsLayout layout(const mla_dims &d, int B, int Tq) {
  WsLayout w;
  const int r = d.kv_lora_rank, K = r + d.qk_rope_head_dim;
  const int M = d.num_heads * Tq;
  // the planner emits at most max(target, number of sequences) items
  const int tgt = std::max(target_items(M, true), target_items(M, false));
  w.max_items = std::max(tgt, B);
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
  // G = sum_h W_UK[h]^T W_UK[h] + W_UV[h]^T W_UV[h], scaled to trace r
  std::vector<double> g(rr);
  double tr = 0.0;
  for (size_t i = 0; i < rr; ++i) g[i] = guk[i] * static_cast<double>(n_uk) + guv[i] * static_cast<double>(n_uv);
  for (int i = 0; i < r; ++i) tr += g[static_cast<size_t>(i) * r + i];
  if (!(tr > 0.0) || !std::isfinite(tr))
    return fail(MLA_ERR_NUMERIC, "mla_calibrate_rotation_weighted: up-projection weights are zero or not finite");
  for (size_t i = 0; i < rr; ++i) g[i] *= static_cast<double>(r) / tr;
  // (G + ridge I)^(-1/2) = V diag(1 / sqrt(max(lambda, 0) + ridge)) V^T; the
  // ridge keeps latent directions the up-projection ignores finite (they get
  // the largest weighted variance and the coarsest groups)
  constexpr double kMetricRidge = 1e-8;  // G has mean eigenvalue 1
  std::vector<double> gv(r), gvec(rr), gh(rr, 0.0), tmp(rr, 0.0), sw(rr, 0.0);
  if (!eigh_ascending(r, g.data(), gv.data(), gvec.data()))
    return fail(MLA_ERR_NUMERIC, "mla_calibrate_rotation_weighted: eigensolver did not converge on the metric");
  for (int k = 0; k < r; ++k) {
    const double sq = 1.0 / std::sqrt(std::max(gv[k], 0.0) + kMetricRidge);
    for (int i = 0; i < r; ++i) {
      const double vik = gvec[static_cast<size_t>(i) * r + k] * sq;
      if (vik == 0.0) continue;
      double *row = gh.data() + static_cast<size_t>(i) * r;
      for (int j = 0; j < r; ++j) row[j] += vik * gvec[static_cast<size_t>(j) * r + k];
    }
  }
  // Sigma_w = G^(-1/2) Sigma G^(-1/2), symmetrised
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
  matmul(gh, sig, tmp);
  matmul(tmp, gh, sw);
  for (int i = 0; i < r; ++i)
    for (int j = i + 1; j < r; ++j) {
      const double m = 0.5 * (sw[static_cast<size_t>(i) * r + j] + sw[static_cast<size_t>(j) * r + i]);
      sw[static_cast<size_t>(i) * r + j] = m;
      sw[static_cast<size_t>(j) * r + i] = m;
    }
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

mla_status mla_append_quant(const mla_dims *dims, const void *latent, mla_dtype dtype,
                            const uint16_t *k_rope, const uint16_t *idx_key, const int64_t *slot_mapping,
                            int64_t n, const uint16_t *R_apply_t, const float *alpha, const mla_cache *cache,
                            void *stream) {
  std::string why;
  if (!dims_valid(dims, &why)) return fail(MLA_ERR_INVALID_ARG, "mla_append_quant: " + why);
  if (dtype != MLA_DTYPE_BF16 && dtype != MLA_DTYPE_FP32)
    return fail(MLA_ERR_INVALID_ARG, "mla_append_quant: dtype must be bf16 or fp32");
  if (n < 0) return fail(MLA_ERR_INVALID_ARG, "mla_append_quant: n must be >= 0");
  if (cache == nullptr) return fail(MLA_ERR_INVALID_ARG, "mla_append_quant: cache is NULL");
  if (n == 0) {
    clear_error();
    return MLA_OK;
  }
  if (!latent || !k_rope || !slot_mapping || !R_apply_t || !alpha || !cache->codes || !cache->scale_zero ||
      !cache->k_rope)
    return fail(MLA_ERR_INVALID_ARG, "mla_append_quant: NULL device pointer");
  if ((dims->index_head_dim > 0) != (idx_key != nullptr) ||
      (dims->index_head_dim > 0 && cache->idx_key == nullptr))
    return fail(MLA_ERR_INVALID_ARG, "mla_append_quant: idx_key and cache.idx_key must be given iff index_head_dim > 0");
  if (cache->capacity < 0) return fail(MLA_ERR_INVALID_ARG, "mla_append_quant: negative capacity");
  if (dims->kv_lora_rank > 1024 && !append_uses_mfma(*dims, dtype))
    return fail(MLA_ERR_UNSUPPORTED, "mla_append_quant: kv_lora_rank > 1024");
  if (n > (int64_t{1} << 31) - 1) return fail(MLA_ERR_UNSUPPORTED, "mla_append_quant: n >= 2^31");
  const void *ptrs[] = {latent, k_rope, idx_key, slot_mapping, R_apply_t, alpha, cache->codes,
                        cache->scale_zero, cache->k_rope, cache->idx_key};
  for (const void *p : ptrs)
    if (p != nullptr && !aligned16(p))
      return fail(MLA_ERR_INVALID_ARG, "mla_append_quant: device pointers must be 16-byte aligned");
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
                       size_t workspace_bytes, float *out, float *lse, void *stream) {
  const std::string F = std::string(fn) + ": ";
  std::string why;
  if (!dims_valid(dims, &why)) return fail(MLA_ERR_INVALID_ARG, F + "" + why);
  if (batch < 0) return fail(MLA_ERR_INVALID_ARG, F + "batch must be >= 0");
  if (tq < 1 || tq > 64) return fail(MLA_ERR_INVALID_ARG, F + "tq must be in 1..64");
  if (causal != 0 && causal != 1) return fail(MLA_ERR_INVALID_ARG, F + "causal must be 0 or 1");
  if (!std::isfinite(softmax_scale)) return fail(MLA_ERR_INVALID_ARG, F + "softmax_scale not finite");
  if (cache == nullptr) return fail(MLA_ERR_INVALID_ARG, F + "cache is NULL");
  if (batch == 0) {
    clear_error();
    return MLA_OK;
  }
  if (!q_nope || !q_rope || !w_uk_f || !w_uv_f || !seq_base || !seq_len || !workspace || !out ||
      !cache->codes || !cache->scale_zero || !cache->k_rope)
    return fail(MLA_ERR_INVALID_ARG, F + "NULL device pointer");
  const void *ptrs[] = {q_nope, q_rope, w_uk_f, w_uv_f, seq_base, seq_len, workspace, out, lse,
                        cache->codes, cache->scale_zero, cache->k_rope};
  for (const void *p : ptrs)
    if (p != nullptr && !aligned16(p))
      return fail(MLA_ERR_INVALID_ARG, F + "device pointers must be 16-byte aligned");
  if (dims->kv_lora_rank > 512)
    return fail(MLA_ERR_UNSUPPORTED, F + "kv_lora_rank > 512");
  const int M = dims->num_heads * tq;
  bool use_mfma = false;
  if (g_decode_variant == 2) {
    if (!mfma_decode_supported(*dims, M))
      return fail(MLA_ERR_UNSUPPORTED, F + "no MFMA kernel for this shape");
    use_mfma = true;
  } else if (g_decode_variant == 0) {
    use_mfma = M >= 16 && mfma_decode_supported(*dims, M);
  }
  if (use_mfma && !mfma_absorb_supported(*dims))
    return fail(MLA_ERR_UNSUPPORTED, F + "qk_nope_head_dim must be a multiple of 16 for the MFMA path");
  const WsLayout w = layout(*dims, batch, tq);
  if (workspace_bytes < w.total)
    return fail(MLA_ERR_WORKSPACE, F + "workspace needs " + std::to_string(w.total) + " bytes");
  DecodeArgs a;
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
  a.target_items = target_items(M, use_mfma);
  a.tile = use_mfma ? 32 : 16;
  a.min_chunk_tiles = min_chunk_tiles(a.tile);
  a.sel = sel;
  a.sel_stride = sel_stride;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the MFMA absorb kernel also runs the planner
  hipError_t e = use_mfma ? launch_absorb_mfma_layout(a, s) : launch_plan(a, s);
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

}  // extern "C"
