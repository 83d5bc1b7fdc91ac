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

// The rotation kernels work on column slices of CW output channels (32, or
// 16 when the head dim is not a multiple of 32): a block stages its slice
// of the rotation into LDS with coalesced loads (rows padded by 16 bytes, so
// the 16-byte reads of 16 consecutive rows hit distinct banks), and thread
// (g, c) forms output channel c of query head g as a dot product over the
// head dim, 256 / CW query heads per pass.
__host__ __device__ __forceinline__ int rot_cw(int d) { return d % 32 == 0 ? 32 : 16; }

// dot product of a staged bf16 row (d values) with a staged fp32 row
__device__ __forceinline__ float dot_row(const uint16_t *mrow, const float *x, int d) {
  float acc = 0.0f;
  for (int n = 0; n < d; n += 8) {
    const u32x4 w = *reinterpret_cast<const u32x4 *>(mrow + n);
    const f32x4 x0 = *reinterpret_cast<const f32x4 *>(x + n);
    const f32x4 x1 = *reinterpret_cast<const f32x4 *>(x + n + 4);
    acc = fmaf(__uint_as_float(w[0] << 16), x0[0], acc);
    acc = fmaf(__uint_as_float(w[0] & 0xffff0000u), x0[1], acc);
    acc = fmaf(__uint_as_float(w[1] << 16), x0[2], acc);
    acc = fmaf(__uint_as_float(w[1] & 0xffff0000u), x0[3], acc);
    acc = fmaf(__uint_as_float(w[2] << 16), x1[0], acc);
    acc = fmaf(__uint_as_float(w[2] & 0xffff0000u), x1[1], acc);
    acc = fmaf(__uint_as_float(w[3] << 16), x1[2], acc);
    acc = fmaf(__uint_as_float(w[3] & 0xffff0000u), x1[3], acc);
  }
  return acc;
}

// Rotated, scaled queries in the split-K kernel's layout (one pseudo-sequence
// b' = b * H_kv + h per sequence and KV head, rows m = t * G + g):
//   qbuf[b'][m][c] = scale * log2(e) * sum_n q[b][t][h G + g][n] R_k,apply[h][n][c]
// and the pseudo-sequences' slots: KV head h's entries are cache slots
// h * capacity + seq_base[b] ...  Grid (B * H_kv * (d / CW) + 1, Tq): block
// (b', slice) stages rows [CW slice, +CW) of R_apply^T (rotation columns).
// The last block plans the split-K items from seq_len alongside (each
// sequence counted once per KV head), which saves a launch.
template <int CW>
__global__ __launch_bounds__(kThreads) void gqa_rotate_q_kernel(GqaDecodeArgs a, DecodeArgs sa) {
  __shared__ __align__(16) uint16_t rsm[CW * (256 + 8)];
  __shared__ __align__(16) float qs[kThreads / CW][256];
  const int d = a.d, G = a.H_q / a.H_kv, ncs = d / CW, rst = d + 8;
  if (static_cast<int>(blockIdx.x) == a.B * a.H_kv * ncs) {  // the planner block
    if (blockIdx.y == 0)
      plan_block(a.seq_len, sa.B, sa.target_items, sa.tile, sa.min_chunk_tiles, sa.max_items, sa.items,
                 sa.item_begin, sa.meta, a.H_kv);
    return;
  }
  const int bp = blockIdx.x / ncs, cs = blockIdx.x % ncs, t = blockIdx.y, b = bp / a.H_kv, h = bp % a.H_kv;
  const int tid = threadIdx.x;
  if (t == 0 && cs == 0 && tid == 0) {
    a.base2[bp] = static_cast<int64_t>(h) * a.capacity + a.seq_base[b];
    a.len2[bp] = a.seq_len[b];
  }
  // rows [CW cs, +CW) of R_apply^T[h] are CW * d contiguous values (at most
  // kRotLoads 16-byte pieces per thread), requested together with the first
  // pass's query values (at most kQLoads per thread): one memory round trip
  const uint16_t *qbase = a.q + ((static_cast<int64_t>(b) * a.Tq + t) * a.H_q + h * G) * d;
  const int c = tid % CW, gl = tid / CW;
  constexpr int GP = kThreads / CW;  // query heads per pass
  constexpr int kRotLoads = CW * 256 / 8 / kThreads, kQLoads = GP * 256 / kThreads;
  const int np = d / 8, total = CW * np, nq0 = min(GP, G) * d;
  {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(a.rk_t + (static_cast<int64_t>(h) * d + CW * cs) * d);
    u32x4 rw[kRotLoads];
    uint16_t qv[kQLoads];
#pragma unroll
    for (int k = 0; k < kRotLoads; ++k) rw[k] = src[min(tid + k * kThreads, total - 1)];  // clamped: always defined
#pragma unroll
    for (int k = 0; k < kQLoads; ++k) qv[k] = qbase[min(tid + k * kThreads, nq0 - 1)];
#pragma unroll
    for (int k = 0; k < kRotLoads; ++k) {
      const int e = tid + k * kThreads;
      if (e < total) *reinterpret_cast<u32x4 *>(rsm + (e / np) * rst + 8 * (e % np)) = rw[k];
    }
#pragma unroll
    for (int k = 0; k < kQLoads; ++k) {
      const int e = tid + k * kThreads;
      if (e < nq0) qs[e / d][e % d] = bf16_to_f32(qv[k]);
    }
  }
  for (int g0 = 0; g0 < G; g0 += GP) {
    const int ng = min(GP, G - g0);
    if (g0 > 0) {
      __syncthreads();  // qs is rewritten
      for (int e = tid; e < ng * d; e += kThreads) qs[e / d][e % d] = bf16_to_f32(qbase[static_cast<int64_t>(g0) * d + e]);
    }
    __syncthreads();
    if (gl < ng) {
      const float acc = dot_row(rsm + c * rst, qs[gl], d);
      a.qbuf[((static_cast<int64_t>(bp) * a.Tq + t) * G + g0 + gl) * d + CW * cs + c] = acc * a.scale_log2;
    }
  }
}

// Merge of the split-K partials and un-rotation in one launch.  Grid
// (B * H_kv * (d / CW), Tq): block (b', slice) merges every query head of one
// (sequence, KV head, query position) over all d channels and forms output
// channels [CW slice, +CW).  Thread (row, 4-channel chunk) folds the items of
// the pseudo-sequence into a running (max, sum, O), kMergeU at a time (O_k =
// l_k times the stored fp16 O_k / l_k):
//   o_z = sum_k 2^(m_k - m) O_k / sum_k 2^(m_k - m) l_k,
//   lse = ln 2 (m + log2 sum_k 2^(m_k - m) l_k);
// the columns [CW slice, +CW) of R_v,apply^T are staged transposed (row v of
// the rotation, all c) and thread (g, v) forms out[g][v] = sum_c R_v,apply[v][c] o_z[g][c].
constexpr int kMergeU = 16;
constexpr int kRotPieces = 4;  // 16-byte pieces of the rotation slice per thread: 256 * 32 / 8 / 256

template <int CW>
__global__ __launch_bounds__(kThreads) void gqa_merge_unrotate_kernel(GqaDecodeArgs a, DecodeArgs sa) {
  __shared__ __align__(16) uint16_t rsm[CW * (256 + 8)];
  __shared__ __align__(16) float zs[kThreads / CW][256];
  const int d = a.d, G = a.H_q / a.H_kv, M = G * a.Tq, nch = d / 4, ncs = d / CW, rst = d + 8;
  const int bp = blockIdx.x / ncs, cs = blockIdx.x % ncs, t = blockIdx.y, b = bp / a.H_kv, h = bp % a.H_kv;
  const int tid = threadIdx.x;
  const int ib = sa.item_begin[bp], ie = sa.item_begin[bp + 1];
  const f16 *po = reinterpret_cast<const f16 *>(sa.part_o);
  const int64_t row = (static_cast<int64_t>(b) * a.Tq + t) * a.H_q + h * G;  // first output row
  const int v = tid % CW, gl = tid / CW;
  // the rotation slice is requested first, so its loads are in flight with
  // the merge's: rows c of R_v,apply^T, columns [CW cs, +CW), 16 bytes at a
  // time (d * CW / 8 pieces, at most kRotPieces per thread)
  u32x4 rw[kRotPieces];
#pragma unroll
  for (int k = 0; k < kRotPieces; ++k) {
    const int e = min(tid + k * kThreads, d * (CW / 8) - 1);  // clamped: always defined
    const int cc = e / (CW / 8), p8 = e % (CW / 8);
    rw[k] = *reinterpret_cast<const u32x4 *>(a.rv_t + static_cast<int64_t>(h) * d * d + static_cast<int64_t>(cc) * d +
                                             CW * cs + 8 * p8);
  }
  constexpr int GP = kThreads / CW;  // query heads per pass
  for (int g0 = 0; g0 < G; g0 += GP) {
    const int ng = min(GP, G - g0);
    __syncthreads();  // zs is rewritten
    for (int pr = tid; pr < ng * nch; pr += kThreads) {
      const int g = pr / nch, c = pr % nch, m = t * G + g0 + g;
      const float *ml = sa.part_ml + static_cast<int64_t>(m) * 2;
      const f16 *pp = po + static_cast<int64_t>(m) * d + 4 * c;
      const int64_t ml_stride = static_cast<int64_t>(M) * 2, po_stride = static_cast<int64_t>(M) * d;
      float mrun = -INFINITY, lrun = 0.0f;
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int k0 = ib; k0 < ie; k0 += kMergeU) {
        f16x4 vv[kMergeU];
        float2 st[kMergeU];
#pragma unroll
        for (int e = 0; e < kMergeU; ++e) {
          const int k = min(k0 + e, ie - 1);
          vv[e] = *reinterpret_cast<const f16x4 *>(pp + k * po_stride);
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
            acc += (wgt * st[e].y) * __builtin_convertvector(vv[e], f32x4);
            lrun += wgt * st[e].y;
          }
          mrun = rm;
        }
      }
      const float inv = lrun > 0.0f ? 1.0f / lrun : 0.0f;
      *reinterpret_cast<f32x4 *>(&zs[g][4 * c]) = acc * inv;
      if (c == 0 && cs == 0 && a.lse != nullptr)
        a.lse[row + g0 + g] = lrun > 0.0f ? (mrun + log2f(lrun)) * kLn2 : -INFINITY;
    }
    if (g0 == 0) {
      // the rotation slice, stored transposed (row v, column c)
#pragma unroll
      for (int k = 0; k < kRotPieces; ++k) {
        const int e = tid + k * kThreads;
        if (e < d * (CW / 8)) {
          const int cc = e / (CW / 8), p8 = e % (CW / 8);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            rsm[(8 * p8 + 2 * j) * rst + cc] = static_cast<uint16_t>(rw[k][j] & 0xffffu);
            rsm[(8 * p8 + 2 * j + 1) * rst + cc] = static_cast<uint16_t>(rw[k][j] >> 16);
          }
        }
      }
    }
    __syncthreads();
    if (gl < ng) a.out[(row + g0 + gl) * d + CW * cs + v] = dot_row(rsm + v * rst, zs[gl], d);
  }
}

// The same merge and un-rotation for d = 128 with one block per query row
// (pseudo-sequence b', position t, head g of the KV group), so no block
// repeats another's merge.  Grid (B * H_kv * G, Tq), 256 threads.
//  * Thread (slice s, 4-channel chunk c) folds items ib + s, ib + s + 8, ...
//    of the row, kRowU per round with their loads issued together; the
//    eight slices are merged in slice order into o_z (LDS) and lse.
//  * Un-rotation out[v] = sum_c R_v,apply^T[c][v] o_z[c]: wave q sums
//    channels c in [32 q, 32 q + 32), lane l the output pair (2 l, 2 l + 1);
//    its 32 rotation words are requested at kernel start, so they are in
//    flight during the merge; the four quarters are added in order.
constexpr int kRowD = 128, kRowU = 8;

__global__ __launch_bounds__(kThreads) void gqa_merge_row128_kernel(GqaDecodeArgs a, DecodeArgs sa) {
  constexpr int NCH = kRowD / 4, S = kThreads / NCH;
  static_assert(S * NCH == kThreads, "one (slice, chunk) per thread");
  __shared__ f32x4 s_o[S][NCH];
  __shared__ float s_m[S], s_l[S];
  __shared__ __align__(16) float s_z[kRowD];
  __shared__ float s_part[4][kRowD];
  const int G = a.H_q / a.H_kv, M = G * a.Tq;
  const int bp = blockIdx.x / G, g = blockIdx.x % G, t = blockIdx.y, b = bp / a.H_kv, h = bp % a.H_kv;
  const int tid = threadIdx.x, lane = tid & 63, q4 = tid >> 6;
  const int m = t * G + g;
  const int64_t row = (static_cast<int64_t>(b) * a.Tq + t) * a.H_q + h * G + g;
  uint32_t rv[32];
  {
    const uint32_t *src = reinterpret_cast<const uint32_t *>(a.rv_t + (static_cast<int64_t>(h) * kRowD + 32 * q4) * kRowD) + lane;
#pragma unroll
    for (int i = 0; i < 32; ++i) rv[i] = src[i * (kRowD / 2)];
  }
  {
    const int c = tid % NCH, sl = tid / NCH;
    const int ib = sa.item_begin[bp], ie = sa.item_begin[bp + 1];
    const float *ml = sa.part_ml + static_cast<int64_t>(m) * 2;
    const f16 *po = reinterpret_cast<const f16 *>(sa.part_o) + static_cast<int64_t>(m) * kRowD + 4 * c;
    const int64_t ml_stride = static_cast<int64_t>(M) * 2, po_stride = static_cast<int64_t>(M) * kRowD;
    float mrun = -INFINITY, lrun = 0.0f;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k0 = ib + sl; k0 < ie; k0 += kRowU * S) {
      f16x4 vv[kRowU];
      float2 st[kRowU];
#pragma unroll
      for (int e = 0; e < kRowU; ++e) {
        const int k = min(k0 + e * S, ie - 1);
        vv[e] = *reinterpret_cast<const f16x4 *>(po + k * po_stride);
        st[e] = *reinterpret_cast<const float2 *>(ml + k * ml_stride);
        if (k0 + e * S >= ie) st[e].x = -INFINITY;
      }
      float rm = mrun;
#pragma unroll
      for (int e = 0; e < kRowU; ++e) rm = fmaxf(rm, st[e].x);
      if (rm != -INFINITY) {
        const float sc = exp2f(mrun - rm);  // 0 while nothing was folded in
        acc *= sc;
        lrun *= sc;
#pragma unroll
        for (int e = 0; e < kRowU; ++e) {
          const float wgt = st[e].x == -INFINITY ? 0.0f : exp2f(st[e].x - rm);
          acc += (wgt * st[e].y) * __builtin_convertvector(vv[e], f32x4);
          lrun += wgt * st[e].y;
        }
        mrun = rm;
      }
    }
    s_o[sl][c] = acc;
    if (c == 0) {  // every chunk thread of a slice holds the same (max, sum)
      s_m[sl] = mrun;
      s_l[sl] = lrun;
    }
  }
  __syncthreads();
  if (tid < NCH) {
    float mx = -INFINITY;
#pragma unroll
    for (int sl = 0; sl < S; ++sl) mx = fmaxf(mx, s_m[sl]);
    float den = 0.0f;
    f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f};
    if (mx != -INFINITY) {
#pragma unroll
      for (int sl = 0; sl < S; ++sl) {
        if (s_m[sl] == -INFINITY) continue;
        const float wgt = exp2f(s_m[sl] - mx);
        den += wgt * s_l[sl];
        o += wgt * s_o[sl][tid];
      }
    }
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    *reinterpret_cast<f32x4 *>(&s_z[4 * tid]) = o * inv;
    if (tid == 0 && a.lse != nullptr) a.lse[row] = den > 0.0f ? (mx + log2f(den)) * kLn2 : -INFINITY;
  }
  __syncthreads();
  float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float z = s_z[32 * q4 + i];
    p0 = fmaf(__uint_as_float(rv[i] << 16), z, p0);
    p1 = fmaf(__uint_as_float(rv[i] & 0xffff0000u), z, p1);
  }
  s_part[q4][2 * lane] = p0;
  s_part[q4][2 * lane + 1] = p1;
  __syncthreads();
  if (tid < kRowD)
    a.out[row * kRowD + tid] = (s_part[0][tid] + s_part[1][tid]) + (s_part[2][tid] + s_part[3][tid]);
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
  if (a.d > 256 || a.d % 16 != 0) return hipErrorInvalidValue;
  TimedLaunch tl("gqa_rotate_q", s);
  // 256 threads: the planner block needs all of them
  const int cw = rot_cw(a.d);
  const dim3 grid(a.B * a.H_kv * (a.d / cw) + 1, a.Tq);
  if (cw == 32)
    gqa_rotate_q_kernel<32><<<grid, kThreads, 0, s>>>(a, sa);
  else
    gqa_rotate_q_kernel<16><<<grid, kThreads, 0, s>>>(a, sa);
  return hipGetLastError();
}

hipError_t launch_gqa_merge_unrotate(const GqaDecodeArgs &a, const DecodeArgs &sa, hipStream_t s) {
  if (a.d > 256 || a.d % 16 != 0) return hipErrorInvalidValue;
  TimedLaunch tl("gqa_merge_unrotate", s);
  if (a.d == kRowD) {
    gqa_merge_row128_kernel<<<dim3(a.B * a.H_q, a.Tq), kThreads, 0, s>>>(a, sa);
    return hipGetLastError();
  }
  const int cw = rot_cw(a.d);
  const dim3 grid(a.B * a.H_kv * (a.d / cw), a.Tq);
  if (cw == 32)
    gqa_merge_unrotate_kernel<32><<<grid, kThreads, 0, s>>>(a, sa);
  else
    gqa_merge_unrotate_kernel<16><<<grid, kThreads, 0, s>>>(a, sa);
  return hipGetLastError();
}

}  // namespace mla
