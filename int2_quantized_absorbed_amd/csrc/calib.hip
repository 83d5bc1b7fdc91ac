// Calibration-side kernels: latent covariance, the applied bf16 rotation,
// the clip-ratio search and the absorb-weight fold.
//
// [OSCAR issue #10, maintainer reply, "How the rotation adapts to the
// latent"]: the rotation comes from the covariance of the latent c_kv over
// calibration tokens, and the clip thresholds are fitted on the rotated
// latent; the up-projection works on the dequantised latent, which is what
// folding R into the kv_b_proj halves achieves.
#include "kernels.hpp"

namespace mla {
namespace {

template <typename T>
__device__ __forceinline__ double load_as_f64(const T *p, int64_t i);
template <>
__device__ __forceinline__ double load_as_f64<float>(const float *p, int64_t i) {
  return static_cast<double>(p[i]);
}
template <>
__device__ __forceinline__ double load_as_f64<uint16_t>(const uint16_t *p, int64_t i) {
  return static_cast<double>(bf16_to_f32(p[i]));
}

// Sigma[i][j] = sum_t c[t][i] c[t][j] / n in fp64, one 32x32 tile per block,
// fixed summation order (deterministic).
template <typename T>
__global__ __launch_bounds__(256) void covariance_kernel(const T *__restrict__ c,
                                                         int64_t n, int r,
                                                         double *__restrict__ sigma) {
  constexpr int TK = 32;
  __shared__ double si[TK][33];
  __shared__ double sj[TK][33];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int i0 = blockIdx.y * 32, j0 = blockIdx.x * 32;
  double acc[2][2] = {{0.0, 0.0}, {0.0, 0.0}};
  for (int64_t t0 = 0; t0 < n; t0 += TK) {
    for (int e = threadIdx.x; e < TK * 32; e += 256) {
      const int tk = e >> 5, col = e & 31;
      const int64_t t = t0 + tk;
      const bool ok_t = t < n;
      si[tk][col] = (ok_t && i0 + col < r) ? load_as_f64(c, t * r + i0 + col) : 0.0;
      sj[tk][col] = (ok_t && j0 + col < r) ? load_as_f64(c, t * r + j0 + col) : 0.0;
    }
    __syncthreads();
#pragma unroll 4
    for (int k = 0; k < TK; ++k) {
      const double a0 = si[k][ty], a1 = si[k][ty + 16];
      const double b0 = sj[k][tx], b1 = sj[k][tx + 16];
      acc[0][0] = fma(a0, b0, acc[0][0]);
      acc[0][1] = fma(a0, b1, acc[0][1]);
      acc[1][0] = fma(a1, b0, acc[1][0]);
      acc[1][1] = fma(a1, b1, acc[1][1]);
    }
    __syncthreads();
  }
  const double inv_n = 1.0 / static_cast<double>(n);
  for (int a = 0; a < 2; ++a)
    for (int b = 0; b < 2; ++b) {
      const int i = i0 + ty + 16 * a, j = j0 + tx + 16 * b;
      if (i < r && j < r) sigma[static_cast<int64_t>(i) * r + j] = acc[a][b] * inv_n;
    }
}

// Rt[j][i] = bf16(R[i][j])
__global__ __launch_bounds__(256) void prepare_rotation_kernel(const float *__restrict__ R,
                                                               int r,
                                                               uint16_t *__restrict__ Rt) {
  __shared__ float tile[32][33];
  const int i0 = blockIdx.y * 32, j0 = blockIdx.x * 32;
  for (int e = threadIdx.x; e < 1024; e += 256) {
    const int a = e >> 5, b = e & 31;  // a: row offset in R, b: column offset
    tile[a][b] = (i0 + a < r && j0 + b < r) ? R[static_cast<int64_t>(i0 + a) * r + j0 + b] : 0.0f;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 1024; e += 256) {
    const int a = e >> 5, b = e & 31;  // write Rt[j0 + a][i0 + b] = R[i0 + b][j0 + a]
    if (j0 + a < r && i0 + b < r)
      Rt[static_cast<int64_t>(j0 + a) * r + i0 + b] = f32_to_bf16(tile[b][a]);
  }
}

// sse[g][a] = sum over tokens and channels of group g of (z - z_hat)^2 at
// clip ratio grid[a] (fp64), fixed-order block reduction.
__global__ __launch_bounds__(256) void group_sse_kernel(const float *__restrict__ z,
                                                        int64_t n, int r, int G,
                                                        const float *__restrict__ grid,
                                                        int n_grid,
                                                        double *__restrict__ sse) {
  const int g = blockIdx.x, a = blockIdx.y;
  const float alpha = grid[a];
  double local = 0.0;
  float v[32];
  for (int64_t t = threadIdx.x; t < n; t += blockDim.x) {
    const float *row = z + t * r + static_cast<int64_t>(g) * G;
    float mx = -INFINITY, mn = INFINITY;
    for (int k = 0; k < G; ++k) {
      v[k] = row[k];
      mx = fmaxf(mx, v[k]);
      mn = fminf(mn, v[k]);
    }
    const QuantParams q = quant_params(mx, mn, alpha);
    const double s64 = static_cast<double>(q.scale_f), z64 = static_cast<double>(q.zero_f);
    for (int k = 0; k < G; ++k) {
      const uint32_t code = quant_code(v[k], q);
      const double zh = z64 + s64 * static_cast<double>(code);
      const double e = static_cast<double>(v[k]) - zh;
      local += e * e;
    }
  }
  __shared__ double red[256];
  red[threadIdx.x] = local;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) sse[static_cast<int64_t>(g) * n_grid + a] = red[0];
}

// alpha[g] = argmin_a sse[g][a]; exact ties go to the larger ratio.
__global__ void clip_argmin_kernel(const double *__restrict__ sse, const float *__restrict__ grid,
                                   int n_grid, int ng, float *__restrict__ alpha) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= ng) return;
  float best_a = grid[0];
  double best_e = sse[static_cast<int64_t>(g) * n_grid];
  for (int a = 1; a < n_grid; ++a) {
    const double e = sse[static_cast<int64_t>(g) * n_grid + a];
    if (e < best_e || (e == best_e && grid[a] > best_a)) {
      best_e = e;
      best_a = grid[a];
    }
  }
  alpha[g] = best_a;
}

// W~[row][j] = fp16(sum_i w[row][i] * R_apply[i][j]) = fp16(sum_i w[row][i] Rt[j][i])
// 64x64 output tile per block, fp32 accumulation.  inner > 0 stores each
// head's block transposed: row = h*inner + a goes to wf[(h*r + j)*inner + a].
__global__ __launch_bounds__(256) void fold_kernel(const uint16_t *__restrict__ w, int rows,
                                                   int r, const uint16_t *__restrict__ Rt,
                                                   uint16_t *__restrict__ wf, int inner) {
  constexpr int TK = 32;
  __shared__ float as[TK][65];
  __shared__ float bs[TK][65];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int row0 = blockIdx.y * 64, col0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < r; k0 += TK) {
    for (int e = threadIdx.x; e < 64 * TK; e += 256) {
      const int m = e / TK, kk = e % TK;
      const int k = k0 + kk;
      as[kk][m] = (row0 + m < rows && k < r) ? bf16_to_f32(w[static_cast<int64_t>(row0 + m) * r + k]) : 0.0f;
      bs[kk][m] = (col0 + m < r && k < r) ? bf16_to_f32(Rt[static_cast<int64_t>(col0 + m) * r + k]) : 0.0f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < TK; ++kk) {
      float av[4], bv[4];
      for (int i = 0; i < 4; ++i) av[i] = as[kk][ty * 4 + i];
      for (int j = 0; j < 4; ++j) bv[j] = bs[kk][tx * 4 + j];
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) {
      const int row = row0 + ty * 4 + i, col = col0 + tx * 4 + j;
      if (row < rows && col < r) {
        const int64_t dst = inner > 0 ? (static_cast<int64_t>(row / inner) * r + col) * inner + row % inner
                                      : static_cast<int64_t>(row) * r + col;
        wf[dst] = f16_bits(f32_to_f16(acc[i][j]));
      }
    }
}

}  // namespace

hipError_t launch_covariance(const void *c, mla_dtype dt, int64_t n, int r, double *sigma,
                             hipStream_t s) {
  TimedLaunch tl("covariance", s);
  dim3 grid((r + 31) / 32, (r + 31) / 32);
  if (dt == MLA_DTYPE_FP32)
    covariance_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float *>(c), n, r, sigma);
  else
    covariance_kernel<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t *>(c), n, r, sigma);
  return hipGetLastError();
}

hipError_t launch_prepare_rotation(const float *R, int r, uint16_t *Rt, hipStream_t s) {
  TimedLaunch tl("prepare_rotation", s);
  dim3 grid((r + 31) / 32, (r + 31) / 32);
  prepare_rotation_kernel<<<grid, 256, 0, s>>>(R, r, Rt);
  return hipGetLastError();
}

hipError_t launch_group_sse(const float *z, int64_t n, int r, int G, const float *grid_dev,
                            int n_grid, double *sse, float *alpha_out, hipStream_t s) {
  TimedLaunch tl("clip_fit", s);
  const int ng = r / G;
  group_sse_kernel<<<dim3(ng, n_grid), 256, 0, s>>>(z, n, r, G, grid_dev, n_grid, sse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  clip_argmin_kernel<<<(ng + 63) / 64, 64, 0, s>>>(sse, grid_dev, n_grid, ng, alpha_out);
  return hipGetLastError();
}

hipError_t launch_fold(const uint16_t *w, int rows, int r, const uint16_t *Rt, uint16_t *wf,
                       int inner, hipStream_t s) {
  TimedLaunch tl("fold_weights", s);
  dim3 grid((r + 63) / 64, (rows + 63) / 64);
  fold_kernel<<<grid, 256, 0, s>>>(w, rows, r, Rt, wf, inner);
  return hipGetLastError();
}

}  // namespace mla
