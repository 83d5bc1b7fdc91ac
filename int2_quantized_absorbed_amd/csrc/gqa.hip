// OSCAR on full-attention (grouped-query) layers: the calibration statistics
// of the two per-KV-head rotations, and the query rotation / partial merge
// and output un-rotation around the split-K decode.
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
#include "plan.hpp"

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

// Query heads of one KV head handled together by the rotation kernels: the
// lane's row (or column) of the rotation is loaded once and applied to all
// of them from LDS.
constexpr int kHeadChunk = 8;

// Rotated, scaled queries in the split-K kernel's layout (one pseudo-sequence
// b' = b * H_kv + h per sequence and KV head, rows m = t * G + g):
//   qbuf[b'][m][c] = scale * log2(e) * sum_n q[b][t][h G + g][n] R_k,apply[h][n][c]
// and the pseudo-sequences' slots: KV head h's entries are cache slots
// h * capacity + seq_base[b] ...  Grid (B * H_kv + 1, Tq); thread c < d
// holds row c of R_apply^T (the rotation's column c) and forms channel c of
// every query head of the group.  One extra block plans the split-K items
// from seq_len alongside (each sequence counted once per KV head), which
// saves a launch.
template <int DMAX>  // head dim bound: the lane's rotation row is loaded whole, all loads in flight together
__global__ __launch_bounds__(kThreads) void gqa_rotate_q_kernel(GqaDecodeArgs a, DecodeArgs sa) {
  __shared__ float qs[kHeadChunk][256];
  if (blockIdx.x == a.B * a.H_kv) {  // the extra block column: block (B * H_kv, 0) plans the split-K work
    if (blockIdx.y == 0)
      plan_block(a.seq_len, sa.B, sa.target_items, sa.tile, sa.min_chunk_tiles, sa.max_items, sa.items,
                 sa.item_begin, sa.meta, a.H_kv);
    return;
  }
  const int bp = blockIdx.x, t = blockIdx.y, b = bp / a.H_kv, h = bp % a.H_kv, c = threadIdx.x;
  const int G = a.H_q / a.H_kv, d = a.d;
  if (t == 0 && c == 0) {
    a.base2[bp] = static_cast<int64_t>(h) * a.capacity + a.seq_base[b];
    a.len2[bp] = a.seq_len[b];
  }
  const uint16_t *qbase = a.q + ((static_cast<int64_t>(b) * a.Tq + t) * a.H_q + h * G) * d;
  uint4 rw[DMAX / 8];  // row min(c, d-1) of R_apply^T, i.e. column c of the rotation
  {
    const uint4 *rrow = reinterpret_cast<const uint4 *>(a.rk_t + (static_cast<int64_t>(h) * d + min(c, d - 1)) * d);
#pragma unroll
    for (int i = 0; i < DMAX / 8; ++i) rw[i] = 8 * i < d ? rrow[i] : make_uint4(0u, 0u, 0u, 0u);
  }
  for (int g0 = 0; g0 < G; g0 += kHeadChunk) {
    const int ng = min(kHeadChunk, G - g0);
    __syncthreads();  // qs is rewritten
    for (int e = c; e < ng * d; e += blockDim.x) qs[e / d][e % d] = bf16_to_f32(qbase[static_cast<int64_t>(g0) * d + e]);
    __syncthreads();
    if (c >= d) continue;
    float acc[kHeadChunk];
#pragma unroll
    for (int g = 0; g < kHeadChunk; ++g) acc[g] = 0.0f;
#pragma unroll
    for (int n = 0; n < DMAX; n += 8) {
      if (n < d) {  // uniform; rw stays statically indexed
        const uint4 w = rw[n / 8];
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float r0 = __uint_as_float(ww[j] << 16), r1 = __uint_as_float(ww[j] & 0xffff0000u);
#pragma unroll
          for (int g = 0; g < kHeadChunk; ++g) {
            acc[g] = fmaf(r0, qs[g][n + 2 * j], acc[g]);
            acc[g] = fmaf(r1, qs[g][n + 2 * j + 1], acc[g]);
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < kHeadChunk; ++g)
      if (g < ng) a.qbuf[((static_cast<int64_t>(bp) * a.Tq + t) * G + g0 + g) * d + c] = acc[g] * a.scale_log2;
  }
}

// Merge of the split-K partials and un-rotation in one launch.  Grid
// (B * H_kv, Tq): the block takes the G query heads of one (sequence, KV
// head, query position), kHeadChunk at a time.  R_apply^T of the head is
// staged in LDS first (its loads in flight during the merge).  Thread (row,
// 4-channel chunk) folds the items of the pseudo-sequence into a running
// (max, sum, O), kMergeU at a time (O_k = l_k times the stored fp16 O_k / l_k):
//   o_z = sum_k 2^(m_k - m) O_k / sum_k 2^(m_k - m) l_k,
//   lse = ln 2 (m + log2 sum_k 2^(m_k - m) l_k);
// then thread v forms out[v] = sum_c R_v,apply[v][c] o_z[c] for every row.
constexpr int kMergeU = 16;

template <int GC>  // query heads per pass: min(G, kHeadChunk) rounded up to a power of two
__global__ __launch_bounds__(kThreads) void gqa_merge_unrotate_kernel(GqaDecodeArgs a, DecodeArgs sa) {
  extern __shared__ uint16_t rs[];  // [d][d] R_apply^T of head h, then zs [kHeadChunk][256]
  const int bp = blockIdx.x, t = blockIdx.y, b = bp / a.H_kv, h = bp % a.H_kv, tid = threadIdx.x;
  const int G = a.H_q / a.H_kv, d = a.d, M = G * a.Tq, nch = d / 4;
  float(*zs)[256] = reinterpret_cast<float(*)[256]>(rs + d * d);
  {
    const uint4 *src = reinterpret_cast<const uint4 *>(a.rv_t + static_cast<int64_t>(h) * d * d);
    uint4 *dst = reinterpret_cast<uint4 *>(rs);
    for (int e0 = 0; e0 < d * d / 8; e0 += 8 * kThreads) {  // eight loads in flight per thread
      uint4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = src[min(e0 + j * kThreads + tid, d * d / 8 - 1)];  // clamped: always defined
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = e0 + j * kThreads + tid;
        if (e < d * d / 8) dst[e] = v[j];
      }
    }
  }
  const int ib = sa.item_begin[bp], ie = sa.item_begin[bp + 1];
  const f16 *po = reinterpret_cast<const f16 *>(sa.part_o);
  const int64_t row = (static_cast<int64_t>(b) * a.Tq + t) * a.H_q + h * G;  // first output row
  for (int g0 = 0; g0 < G; g0 += GC) {
    const int ng = min(GC, G - g0);
    __syncthreads();  // zs is rewritten
    for (int pr = tid; pr < ng * nch; pr += blockDim.x) {
      const int g = pr / nch, c = pr % nch, m = t * G + g0 + g;
      const float *ml = sa.part_ml + static_cast<int64_t>(m) * 2;
      const f16 *pp = po + static_cast<int64_t>(m) * d + 4 * c;
      const int64_t ml_stride = static_cast<int64_t>(M) * 2, po_stride = static_cast<int64_t>(M) * d;
      float mrun = -INFINITY, lrun = 0.0f;
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int k0 = ib; k0 < ie; k0 += kMergeU) {
        f16x4 v[kMergeU];
        float2 st[kMergeU];
#pragma unroll
        for (int e = 0; e < kMergeU; ++e) {
          const int k = min(k0 + e, ie - 1);
          v[e] = *reinterpret_cast<const f16x4 *>(pp + k * po_stride);
          st[e] = *reinterpret_cast<const float2 *>(ml + k * ml_stride);
          if (k0 + e >= ie) st[e].x = -INFINITY;
        }
        float rm = mrun;
#pragma unroll
        for (int e = 0; e < kMergeU; ++e) rm = fmaxf(rm, st[e].x);
        if (rm != -INFINITY) {
          const float sc = exp2f(mrun - rm);  // 0 while nothing was folded in
          acc *= sc;
          lrun *= sc;
#pragma unroll
          for (int e = 0; e < kMergeU; ++e) {
            const float wgt = st[e].x == -INFINITY ? 0.0f : exp2f(st[e].x - rm);
            acc += (wgt * st[e].y) * __builtin_convertvector(v[e], f32x4);
            lrun += wgt * st[e].y;
          }
          mrun = rm;
        }
      }
      const float inv = lrun > 0.0f ? 1.0f / lrun : 0.0f;
      *reinterpret_cast<f32x4 *>(&zs[g][4 * c]) = acc * inv;
      if (c == 0 && a.lse != nullptr) a.lse[row + g0 + g] = lrun > 0.0f ? (mrun + log2f(lrun)) * kLn2 : -INFINITY;
    }
    __syncthreads();
    const int v = tid;
    if (v >= d) continue;
    float acc[GC];
#pragma unroll
    for (int g = 0; g < GC; ++g) acc[g] = 0.0f;
    for (int c = 0; c < d; c += 4) {  // four channels per step: 16-byte reads of the merged rows
      float r[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] = bf16_to_f32(rs[(c + j) * d + v]);  // R_v,apply[v][c + j]
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        const f32x4 z = *reinterpret_cast<const f32x4 *>(&zs[g][c]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[g] = fmaf(r[j], z[j], acc[g]);
      }
    }
#pragma unroll
    for (int g = 0; g < GC; ++g)
      if (g < ng) a.out[(row + g0 + g) * d + v] = acc[g];
  }
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

hipError_t launch_gqa_rotate_q(const GqaDecodeArgs &a, const DecodeArgs &sa, hipStream_t s) {
  if (a.d > 256) return hipErrorInvalidValue;
  TimedLaunch tl("gqa_rotate_q", s);
  // 256 threads: the planner block needs all of them
  const dim3 grid(a.B * a.H_kv + 1, a.Tq);
  if (a.d <= 64)
    gqa_rotate_q_kernel<64><<<grid, kThreads, 0, s>>>(a, sa);
  else if (a.d <= 128)
    gqa_rotate_q_kernel<128><<<grid, kThreads, 0, s>>>(a, sa);
  else
    gqa_rotate_q_kernel<256><<<grid, kThreads, 0, s>>>(a, sa);
  return hipGetLastError();
}

hipError_t launch_gqa_merge_unrotate(const GqaDecodeArgs &a, const DecodeArgs &sa, hipStream_t s) {
  if (a.d > 256 || a.d % 4 != 0) return hipErrorInvalidValue;
  TimedLaunch tl("gqa_merge_unrotate", s);
  const size_t lds = static_cast<size_t>(a.d) * a.d * sizeof(uint16_t) + kHeadChunk * 256 * sizeof(float);
  const dim3 grid(a.B * a.H_kv, a.Tq);
  const int G = a.H_q / a.H_kv;
  if (G >= 8)
    gqa_merge_unrotate_kernel<8><<<grid, kThreads, lds, s>>>(a, sa);
  else if (G >= 4)
    gqa_merge_unrotate_kernel<4><<<grid, kThreads, lds, s>>>(a, sa);
  else if (G >= 2)
    gqa_merge_unrotate_kernel<2><<<grid, kThreads, lds, s>>>(a, sa);
  else
    gqa_merge_unrotate_kernel<1><<<grid, kThreads, lds, s>>>(a, sa);
  return hipGetLastError();
}

}  // namespace mla
