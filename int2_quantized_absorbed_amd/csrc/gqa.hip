// OSCAR on full-attention (grouped-query) layers: the calibration statistics
// of the two per-KV-head rotations, and the query rotation / output
// un-rotation around the shared split-K decode.
//
// [OSCAR issue #10, "MLA model support", maintainer reply, part "How the
// rotation adapts to the latent", first point]: on full-attention models the
// method fits, per layer and per KV head, a rotation for K from the query
// covariance and a rotation for V from a score-weighted value covariance.
// The statistics here follow the readings the library documents with
// gqa_calibrate: causal self-attention over one calibration sequence, the
// attention mass each key receives as its weight.
//
// Layout: H_q query heads, H_kv KV heads, G = H_q / H_kv; query head g reads
// KV head g / G.  Calibration inputs are head-major bf16: q [H_q][n][d],
// k and v [H_kv][n][d].
#include "kernels.hpp"

namespace mla {
namespace {

constexpr int kThreads = 256;

// fp64 dot product of a bf16 row (16-byte aligned, d % 8 == 0) with an fp64
// vector in LDS; every bf16 value is exact in fp64.
__device__ __forceinline__ double dot_row(const uint16_t *x, const double *y, int d) {
  double acc = 0.0;
  for (int k = 0; k < d; k += 8) {
    const uint4 w = *reinterpret_cast<const uint4 *>(x + k);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc = fma(static_cast<double>(__uint_as_float(ww[j] << 16)), y[k + 2 * j], acc);
      acc = fma(static_cast<double>(__uint_as_float(ww[j] & 0xffff0000u)), y[k + 2 * j + 1], acc);
    }
  }
  return acc;
}

// Block-wide fp64 reduction (sum or max) in a fixed order; every thread gets
// the result.
template <bool kMax>
__device__ double block_reduce(double v, double *red) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int off = 32; off > 0; off >>= 1) {
    const double o = __shfl_xor(v, off);
    v = kMax ? fmax(v, o) : v + o;
  }
  if (lane == 0) red[wv] = v;
  __syncthreads();
  const double r = kMax ? fmax(fmax(red[0], red[1]), fmax(red[2], red[3])) : (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();  // red is rewritten by the next call
  return r;
}

// Row statistics of the causal calibration attention: for query head g and
// position i, m = max_{t <= i} s_t and 1 / sum_{t <= i} exp(s_t - m), with
// s_t = scale * q_{g,i} . k_{h,t} in fp64.  Grid (n, H_q).
__global__ __launch_bounds__(kThreads) void gqa_row_stats_kernel(const uint16_t *q, const uint16_t *k, int n,
                                                                 int d, int G, double scale, double *row_m,
                                                                 double *row_inv) {
  __shared__ double qv[256];
  __shared__ double red[kThreads / 64];
  const int i = blockIdx.x, g = blockIdx.y, h = g / G, tid = threadIdx.x;
  const uint16_t *qr = q + (static_cast<int64_t>(g) * n + i) * d;
  for (int e = tid; e < d; e += kThreads) qv[e] = static_cast<double>(bf16_to_f32(qr[e]));
  __syncthreads();
  const uint16_t *kh = k + static_cast<int64_t>(h) * n * d;
  double m = -INFINITY;
  for (int t = tid; t <= i; t += kThreads) m = fmax(m, scale * dot_row(kh + static_cast<int64_t>(t) * d, qv, d));
  m = block_reduce<true>(m, red);
  double s = 0.0;
  for (int t = tid; t <= i; t += kThreads) s += exp(scale * dot_row(kh + static_cast<int64_t>(t) * d, qv, d) - m);
  s = block_reduce<false>(s, red);
  if (tid == 0) {
    row_m[static_cast<int64_t>(g) * n + i] = m;
    row_inv[static_cast<int64_t>(g) * n + i] = 1.0 / s;
  }
}

// Attention mass of calibration key t of KV head h: the sum over the G query
// heads of h and the positions i >= t of softmax_t(scale q_{g,i} . k_{h,.}).
// Grid (n, H_kv).
__global__ __launch_bounds__(kThreads) void gqa_col_mass_kernel(const uint16_t *q, const uint16_t *k, int n, int d,
                                                                int G, double scale, const double *row_m,
                                                                const double *row_inv, double *w) {
  __shared__ double kv[256];
  __shared__ double red[kThreads / 64];
  const int t = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const uint16_t *kr = k + (static_cast<int64_t>(h) * n + t) * d;
  for (int e = tid; e < d; e += kThreads) kv[e] = static_cast<double>(bf16_to_f32(kr[e]));
  __syncthreads();
  const int span = n - t;
  double acc = 0.0;
  for (int e = tid; e < G * span; e += kThreads) {
    const int g = h * G + e / span, i = t + e % span;
    const int64_t gi = static_cast<int64_t>(g) * n + i;
    const double s = scale * dot_row(q + gi * d, kv, d);
    acc += exp(s - row_m[gi]) * row_inv[gi];
  }
  acc = block_reduce<false>(acc, red);
  if (tid == 0) w[static_cast<int64_t>(h) * n + t] = acc;
}

// Score-weighted value covariance: sigma[h][a][b] = sum_t w_t v_ta v_tb /
// sum_t w_t, fp64.  Grid (d, H_kv); thread b < d.
__global__ __launch_bounds__(kThreads) void gqa_weighted_cov_kernel(const uint16_t *v, const double *w, int n, int d,
                                                                    double *sigma) {
  const int a = blockIdx.x, h = blockIdx.y;
  const uint16_t *vh = v + static_cast<int64_t>(h) * n * d;
  const double *wh = w + static_cast<int64_t>(h) * n;
  for (int b = threadIdx.x; b < d; b += kThreads) {
    double acc = 0.0, wsum = 0.0;
    for (int t = 0; t < n; ++t) {
      const double wt = wh[t];
      acc += wt * static_cast<double>(bf16_to_f32(vh[static_cast<int64_t>(t) * d + a])) *
             static_cast<double>(bf16_to_f32(vh[static_cast<int64_t>(t) * d + b]));
      wsum += wt;
    }
    sigma[(static_cast<int64_t>(h) * d + a) * d + b] = acc / wsum;
  }
}

// Rotated, scaled queries in the split-K kernel's layout (one pseudo-sequence
// b' = b * H_kv + h per sequence and KV head, rows m = t * G + g):
//   qbuf[b'][m][c] = scale * log2(e) * sum_n q[b][t][h G + g][n] R_k,apply[h][n][c]
// and the pseudo-sequences' slots: KV head h's entries are cache slots
// h * capacity + seq_base[b] ...  Grid (Tq, B * H_kv).
__global__ __launch_bounds__(kThreads) void gqa_rotate_q_kernel(GqaDecodeArgs a) {
  const int t = blockIdx.x, bp = blockIdx.y, b = bp / a.H_kv, h = bp % a.H_kv, tid = threadIdx.x;
  const int G = a.H_q / a.H_kv, d = a.d;
  if (t == 0 && tid == 0) {
    a.base2[bp] = static_cast<int64_t>(h) * a.capacity + a.seq_base[b];
    a.len2[bp] = a.seq_len[b];
  }
  for (int e = tid; e < G * d; e += kThreads) {
    const int g = e / d, c = e % d;
    const uint16_t *qr = a.q + ((static_cast<int64_t>(b) * a.Tq + t) * a.H_q + h * G + g) * d;
    const uint16_t *rr = a.rk_t + (static_cast<int64_t>(h) * d + c) * d;  // row c of R_apply^T
    float acc = 0.0f;
    for (int k = 0; k < d; ++k) acc = fmaf(bf16_to_f32(rr[k]), bf16_to_f32(qr[k]), acc);
    a.qbuf[((static_cast<int64_t>(bp) * a.Tq + t) * G + g) * d + c] = acc * a.scale_log2;
  }
}

// out[b][t][h G + g][v] = sum_c R_v,apply[h][v][c] o_z[b'][t G + g][c] (the
// merged attention output, still in KV head h's rotated basis), fp32; lse
// copied into the output layout.  Grid (B * Tq * H_q).
__global__ __launch_bounds__(kThreads) void gqa_unrotate_kernel(GqaDecodeArgs a) {
  __shared__ float oz[256];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int G = a.H_q / a.H_kv, d = a.d;
  const int qh = row % a.H_q, t = (row / a.H_q) % a.Tq, b = row / (a.H_q * a.Tq);
  const int h = qh / G, g = qh % G;
  const int64_t row2 = (static_cast<int64_t>(b * a.H_kv + h) * a.Tq + t) * G + g;
  for (int e = tid; e < d; e += kThreads) oz[e] = a.oz[row2 * d + e];
  __syncthreads();
  const uint16_t *rv = a.rv_t + static_cast<int64_t>(h) * d * d;  // rv[c][v] = R_v,apply[v][c]
  for (int v = tid; v < d; v += kThreads) {
    float acc = 0.0f;
    for (int c = 0; c < d; ++c) acc = fmaf(bf16_to_f32(rv[static_cast<int64_t>(c) * d + v]), oz[c], acc);
    a.out[static_cast<int64_t>(row) * d + v] = acc;
  }
  if (tid == 0 && a.lse != nullptr) a.lse[row] = a.lse2[row2];
}

}  // namespace

hipError_t launch_gqa_calib_stats(const uint16_t *q, const uint16_t *k, const uint16_t *v, int n, int d, int H_q,
                                  int H_kv, double scale, double *row_m, double *row_inv, double *w,
                                  double *sigma_v, hipStream_t s) {
  if (d > 256 || d % 8 != 0) return hipErrorInvalidValue;
  const int G = H_q / H_kv;
  gqa_row_stats_kernel<<<dim3(n, H_q), kThreads, 0, s>>>(q, k, n, d, G, scale, row_m, row_inv);
  gqa_col_mass_kernel<<<dim3(n, H_kv), kThreads, 0, s>>>(q, k, n, d, G, scale, row_m, row_inv, w);
  gqa_weighted_cov_kernel<<<dim3(d, H_kv), kThreads, 0, s>>>(v, w, n, d, sigma_v);
  return hipGetLastError();
}

hipError_t launch_gqa_rotate_q(const GqaDecodeArgs &a, hipStream_t s) {
  if (a.d > 256) return hipErrorInvalidValue;
  TimedLaunch tl("gqa_rotate_q", s);
  gqa_rotate_q_kernel<<<dim3(a.Tq, a.B * a.H_kv), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gqa_unrotate(const GqaDecodeArgs &a, hipStream_t s) {
  if (a.d > 256) return hipErrorInvalidValue;
  TimedLaunch tl("gqa_unrotate", s);
  gqa_unrotate_kernel<<<a.B * a.Tq * a.H_q, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
