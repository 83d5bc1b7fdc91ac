// Absorbed MLA decode over the INT2 latent cache: planner, query absorb,
// vector-ALU split-K kernel, and the combine + up-projection kernel.
//
// [shard PR #5, TL;DR item 2]: the DeepSeek "absorb" form caches only the
// latent plus one shared rope key and runs attention in latent space.
// [OSCAR issue #10, maintainer reply, "How the rotation adapts to the
// latent"]: the cache holds the rotated INT2 latent and the kv_b_proj
// up-projection runs on the dequantised latent.  With W~ = W R_apply folded
// once per layer, every step here works on z_hat directly:
//   q~ = W~_UK[h]^T q_nope,   s = scale (q~ . z_hat + q_rope . k_rope),
//   out = W~_UV[h] (sum_tau softmax(s)_tau z_hat_tau).
// Scores are kept in log2 units (q~ and q_rope pre-multiplied by
// scale * log2 e) so the softmax uses exp2.
#include "kernels.hpp"

namespace mla {
namespace {

// Token-balanced split-K plan from device seq_len (no host synchronisation).
// Chunk length C = round_up(ceil(total / target), tile); sequence b gets
// ceil(L_b / C) items of equal length (rounded up to the tile).  The item
// count is then at most target + B = max_items.
__global__ __launch_bounds__(256) void plan_kernel(const int32_t *__restrict__ seq_len, int B,
                                                   int target, int tile, int max_items,
                                                   WorkItem *__restrict__ items,
                                                   int32_t *__restrict__ item_begin,
                                                   int32_t *__restrict__ meta) {
  __shared__ long long red[256];
  __shared__ int32_t scan[256];
  __shared__ int32_t carry_s;
  const int tid = threadIdx.x;
  long long tot = 0;
  for (int b = tid; b < B; b += 256) tot += max(0, seq_len[b]);
  red[tid] = tot;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  const long long total = red[0];
  long long C = (total + target - 1) / max(target, 1);
  C = ((C + tile - 1) / tile) * tile;
  if (C < tile) C = tile;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < B; base += 256) {
    const int b = base + tid;
    int nb = 0, chunk = 0, L = 0;
    if (b < B) {
      L = seq_len[b];
      if (L > 0) {
        nb = static_cast<int>((L + C - 1) / C);
        chunk = (L + nb - 1) / nb;
        chunk = ((chunk + tile - 1) / tile) * tile;
        nb = (L + chunk - 1) / chunk;
      }
    }
    scan[tid] = nb;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {  // inclusive Hillis-Steele scan
      const int v = (tid >= off) ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int carry = carry_s;
    const int excl = carry + scan[tid] - nb;
    if (b < B) {
      item_begin[b] = min(excl, max_items);
      for (int c = 0; c < nb; ++c) {
        const int idx = excl + c;
        if (idx < max_items) {
          WorkItem it;
          it.b = b;
          it.t0 = c * chunk;
          it.t1 = min(L, (c + 1) * chunk);
          it.pad = 0;
          items[idx] = it;
        }
      }
    }
    __syncthreads();
    if (tid == 255) carry_s = carry + scan[255];
    __syncthreads();
  }
  if (tid == 0) {
    const int n = min(carry_s, max_items);
    item_begin[B] = n;
    meta[0] = n;
    meta[1] = static_cast<int32_t>(C);
  }
}

// q~ in fp32, row-major [B*M][r + d_r] with M = Tq*H rows per sequence
// (row = t*H + h); columns r.. hold q_rope.  Both are pre-scaled by
// scale*log2(e).  One block per head, rows in chunks of 16.
__global__ __launch_bounds__(256) void absorb_f32_kernel(DecodeArgs a) {
  const int h = blockIdx.x;
  const int H = a.d.num_heads, dn = a.d.qk_nope_head_dim, dr = a.d.qk_rope_head_dim;
  const int r = a.d.kv_lora_rank, K = r + dr;
  const int nrows = a.B * a.Tq;
  constexpr int RC = 16;
  extern __shared__ float qs_dyn[];  // [RC][dn + 1]
  const int QP = dn + 1;
  float *qbuf = static_cast<float *>(a.qbuf);
  const uint16_t *w = a.w_uk_f + static_cast<int64_t>(h) * r * dn;  // [r][d_n] of head h
  for (int q0 = 0; q0 < nrows; q0 += RC) {
    const int nr = min(RC, nrows - q0);
    __syncthreads();
    for (int e = threadIdx.x; e < nr * dn; e += 256) {
      const int i = e / dn, k = e % dn;
      qs_dyn[i * QP + k] = bf16_to_f32(a.q_nope[(static_cast<int64_t>(q0 + i) * H + h) * dn + k]);
    }
    __syncthreads();
    for (int j = threadIdx.x; j < r; j += 256) {
      float acc[RC];
#pragma unroll
      for (int i = 0; i < RC; ++i) acc[i] = 0.0f;
      for (int k = 0; k < dn; ++k) {
        const float wv = static_cast<float>(bits_f16(w[static_cast<int64_t>(j) * dn + k]));
#pragma unroll
        for (int i = 0; i < RC; ++i) acc[i] = fmaf(wv, qs_dyn[i * QP + k], acc[i]);
      }
      for (int i = 0; i < nr; ++i)
        qbuf[(static_cast<int64_t>(q0 + i) * H + h) * K + j] = acc[i] * a.scale_log2;
    }
    for (int e = threadIdx.x; e < nr * dr; e += 256) {
      const int i = e / dr, k = e % dr;
      const int64_t row = static_cast<int64_t>(q0 + i) * H + h;
      qbuf[row * K + r + k] = bf16_to_f32(a.q_rope[row * dr + k]) * a.scale_log2;
    }
  }
}

// Vector-ALU split-K kernel: one block per (work item, 16-row block).
// For small H*Tq (below one MFMA tile) and shapes without an MFMA kernel.
template <int TT>
__global__ __launch_bounds__(256) void splitk_valu_kernel(DecodeArgs a, int row_blocks) {
  constexpr int ROWS = 16;
  constexpr int NA = 32;  // ROWS * r / 256 for r <= 512
  extern __shared__ float lds[];
  const int item = blockIdx.x / row_blocks;
  const int rb = blockIdx.x % row_blocks;
  if (item >= a.meta[0]) return;
  const WorkItem it = a.items[item];
  const int r = a.d.kv_lora_rank, dr = a.d.qk_rope_head_dim, G = a.d.group_size;
  const int H = a.d.num_heads, K = r + dr, KP = K + 1;
  const int M = H * a.Tq;
  float *q_s = lds;                    // [ROWS][KP]
  float *z_s = q_s + ROWS * KP;        // [TT][KP]
  float *p_s = z_s + TT * KP;          // [ROWS][TT]
  float *al_s = p_s + ROWS * TT;       // [ROWS]
  const int tid = threadIdx.x;
  const int row0 = rb * ROWS;
  const int L = a.seq_len[it.b];
  const int64_t base = a.seq_base[it.b];
  const float *qbuf = static_cast<const float *>(a.qbuf);
  for (int e = tid; e < ROWS * K; e += 256) {
    const int i = e / K, k = e % K;
    const int m = row0 + i;
    q_s[i * KP + k] = (m < M) ? qbuf[(static_cast<int64_t>(it.b) * M + m) * K + k] : 0.0f;
  }
  // score-thread mapping
  const int srow = tid / TT, stok = tid % TT;
  const bool scorer = tid < ROWS * TT;
  const int sm = row0 + srow;
  int vis = 0;
  if (scorer && sm < M) {
    const int t = sm / H;
    vis = a.causal ? (L - a.Tq + t + 1) : L;
  }
  float m_run = -INFINITY, l_run = 0.0f;
  float acc[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) acc[i] = 0.0f;
  const int na = ROWS * r / 256;
  const uint32_t *sz32 = reinterpret_cast<const uint32_t *>(a.cache.scale_zero);
  for (int t0 = it.t0; t0 < it.t1; t0 += TT) {
    __syncthreads();
    // dequantise the tile into LDS (fp32), rope key appended
    for (int e = tid; e < TT * r; e += 256) {
      const int tk = e / r, j = e % r;
      const int tau = t0 + tk;
      float v = 0.0f;
      if (tau < it.t1) {
        const int64_t slot = base + tau;
        const uint32_t byte = a.cache.codes[slot * (r / 4) + j / 4];
        const uint32_t code = (byte >> (2 * (j & 3))) & 3u;
        const uint32_t sz = sz32[slot * (r / G) + j / G];
        const float sc = static_cast<float>(bits_f16(static_cast<uint16_t>(sz & 0xffffu)));
        const float zr = static_cast<float>(bits_f16(static_cast<uint16_t>(sz >> 16)));
        v = fmaf(sc, static_cast<float>(code), zr);
      }
      z_s[tk * KP + j] = v;
    }
    for (int e = tid; e < TT * dr; e += 256) {
      const int tk = e / dr, k = e % dr;
      const int tau = t0 + tk;
      z_s[tk * KP + r + k] = (tau < it.t1) ? bf16_to_f32(a.cache.k_rope[(base + tau) * dr + k]) : 0.0f;
    }
    __syncthreads();
    if (scorer) {
      const int tau = t0 + stok;
      float s = -INFINITY;
      if (sm < M && tau < it.t1 && tau < vis) {
        float acc_s = 0.0f;
        const float *qr = q_s + srow * KP;
        const float *zr = z_s + stok * KP;
        for (int k = 0; k < K; ++k) acc_s = fmaf(qr[k], zr[k], acc_s);
        s = acc_s;
      }
      float mt = s;
      for (int off = TT / 2; off > 0; off >>= 1) mt = fmaxf(mt, __shfl_xor(mt, off, TT));
      const float m_new = fmaxf(m_run, mt);
      float alpha = 1.0f, p = 0.0f;
      if (m_new != -INFINITY) {
        alpha = exp2f(m_run - m_new);
        p = (s == -INFINITY) ? 0.0f : exp2f(s - m_new);
      }
      float ps = p;
      for (int off = TT / 2; off > 0; off >>= 1) ps += __shfl_xor(ps, off, TT);
      l_run = l_run * alpha + ps;
      m_run = m_new;
      p_s[srow * TT + stok] = p;
      if (stok == 0) al_s[srow] = alpha;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      if (i < na) {
        const int e = tid + 256 * i;
        const int row = e / r, j = e % r;
        float o = acc[i] * al_s[row];
        for (int tk = 0; tk < TT; ++tk) o = fmaf(p_s[row * TT + tk], z_s[tk * KP + j], o);
        acc[i] = o;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    if (i < na) {
      const int e = tid + 256 * i;
      const int row = e / r, j = e % r;
      const int m = row0 + row;
      if (m < M) a.part_o[(static_cast<int64_t>(item) * M + m) * r + j] = acc[i];
    }
  }
  if (scorer && stok == 0 && sm < M) {
    a.part_ml[(static_cast<int64_t>(item) * M + sm) * 2 + 0] = m_run;
    a.part_ml[(static_cast<int64_t>(item) * M + sm) * 2 + 1] = l_run;
  }
}

// Log-sum-exp merge of the split-K partials of one query row (b, t, h):
// m = max_i m_i, o_z = sum_i 2^(m_i - m) O_i / sum_i 2^(m_i - m) l_i,
// lse = ln 2 * (m + log2 sum_i 2^(m_i - m) l_i).  One block per row.
__global__ __launch_bounds__(128) void combine_kernel(DecodeArgs a) {
  const int H = a.d.num_heads, r = a.d.kv_lora_rank;
  const int M = H * a.Tq;
  const int row = blockIdx.x;               // (b*Tq + t)*H + h
  const int q = row / H, h = row % H;
  const int b = q / a.Tq, t = q % a.Tq, m = t * H + h;
  const int ib = a.item_begin[b], ie = a.item_begin[b + 1];
  float mx = -INFINITY;
  for (int i = ib; i < ie; ++i) mx = fmaxf(mx, a.part_ml[(static_cast<int64_t>(i) * M + m) * 2]);
  float den = 0.0f;
  if (mx != -INFINITY)
    for (int i = ib; i < ie; ++i) {
      const float mi = a.part_ml[(static_cast<int64_t>(i) * M + m) * 2];
      if (mi != -INFINITY) den += exp2f(mi - mx) * a.part_ml[(static_cast<int64_t>(i) * M + m) * 2 + 1];
    }
  if (threadIdx.x == 0 && a.lse != nullptr) a.lse[row] = (den > 0.0f) ? (mx + log2f(den)) * kLn2 : -INFINITY;
  const float inv = (den > 0.0f) ? 1.0f / den : 0.0f;
  float *dst = a.oz + static_cast<int64_t>(row) * r;
  for (int j = 4 * threadIdx.x; j < r; j += 4 * blockDim.x) {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (den > 0.0f)
      for (int i = ib; i < ie; ++i) {
        const float mi = a.part_ml[(static_cast<int64_t>(i) * M + m) * 2];
        if (mi == -INFINITY) continue;
        const float wgt = exp2f(mi - mx);
        acc += wgt * *reinterpret_cast<const f32x4 *>(a.part_o + (static_cast<int64_t>(i) * M + m) * r + j);
      }
    *reinterpret_cast<f32x4 *>(dst + j) = acc * inv;
  }
}

// out[b,t,h,:] = W~_UV[h] o_z[b,t,h,:] on MFMA (32x32x16 f16, fp32 acc).
// o_z is split as hi + lo (two fp16 parts) so the product keeps ~fp32
// precision of o_z; W~_UV is fp16.  Block = (head, 32 query rows); wave w
// produces output columns [32w, 32w + 32) of each 128-wide slice.
__global__ __launch_bounds__(256) void upproj_mfma_kernel(DecodeArgs a) {
  const int h = blockIdx.x, rt = blockIdx.y;
  const int H = a.d.num_heads, r = a.d.kv_lora_rank, dv = a.d.v_head_dim;
  const int nrows = a.B * a.Tq;
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6, hf = l >> 5, l32 = l & 31;
  const int q = rt * 32 + l32;              // A-operand row of this lane
  const bool q_ok = q < nrows;
  const float *arow = a.oz + (static_cast<int64_t>(q_ok ? q : 0) * H + h) * r;
  for (int v0 = 32 * w; v0 < dv; v0 += 128) {
    const uint16_t *brow = a.w_uv_f + (static_cast<int64_t>(h) * dv + v0 + l32) * r;
    f32x16 acc = {};
    for (int k0 = 0; k0 < r; k0 += 16) {
      f16x8 ahi, alo;
      const f32x4 x0 = q_ok ? *reinterpret_cast<const f32x4 *>(arow + k0 + 8 * hf) : f32x4{};
      const f32x4 x1 = q_ok ? *reinterpret_cast<const f32x4 *>(arow + k0 + 8 * hf + 4) : f32x4{};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f16 h0 = static_cast<f16>(x0[e]), h1 = static_cast<f16>(x1[e]);
        ahi[e] = h0;
        ahi[e + 4] = h1;
        alo[e] = static_cast<f16>(x0[e] - static_cast<float>(h0));
        alo[e + 4] = static_cast<f16>(x1[e] - static_cast<float>(h1));
      }
      const f16x8 bw = *reinterpret_cast<const f16x8 *>(brow + k0 + 8 * hf);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi, bw, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo, bw, acc, 0, 0, 0);
    }
    // C layout: lane holds column v0 + l32, rows 8(v/4) + 4hf + v%4
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int qq = rt * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
      if (qq < nrows) a.out[(static_cast<int64_t>(qq) * H + h) * dv + v0 + l32] = acc[v];
    }
  }
}

// Vector-ALU up-projection for v_head_dim not a multiple of 32: one wave per
// (head, output column), lanes split the latent channels.
__global__ __launch_bounds__(256) void upproj_valu_kernel(DecodeArgs a) {
  const int H = a.d.num_heads, r = a.d.kv_lora_rank, dv = a.d.v_head_dim;
  const int nrows = a.B * a.Tq;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (gw >= H * dv) return;
  const int h = gw / dv, v = gw % dv;
  const uint16_t *wrow = a.w_uv_f + (static_cast<int64_t>(h) * dv + v) * r;
  for (int q = 0; q < nrows; ++q) {
    const float *oz = a.oz + (static_cast<int64_t>(q) * H + h) * r;
    float s = 0.0f;
    for (int j = lane; j < r; j += 64) s = fmaf(static_cast<float>(bits_f16(wrow[j])), oz[j], s);
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) a.out[(static_cast<int64_t>(q) * H + h) * dv + v] = s;
  }
}

}  // namespace

hipError_t launch_plan(const DecodeArgs &a, hipStream_t s) {
  TimedLaunch tl("decode_plan", s);
  plan_kernel<<<1, 256, 0, s>>>(a.seq_len, a.B, a.target_items, a.tile, a.max_items, a.items,
                                a.item_begin, a.meta);
  return hipGetLastError();
}

hipError_t launch_absorb_f32(const DecodeArgs &a, hipStream_t s) {
  TimedLaunch tl("absorb_q", s);
  const size_t lds = static_cast<size_t>(16) * (a.d.qk_nope_head_dim + 1) * sizeof(float);
  absorb_f32_kernel<<<a.d.num_heads, 256, lds, s>>>(a);
  return hipGetLastError();
}

int valu_tile(const mla_dims &d) {
  const int K = d.kv_lora_rank + d.qk_rope_head_dim;
  return ((16 + 16) * (K + 1) + 16 * 16 + 16) * 4 <= 64 * 1024 ? 16 : 8;
}

hipError_t launch_splitk_valu(const DecodeArgs &a, hipStream_t s) {
  TimedLaunch tl("splitk_decode", s);
  const int M = a.d.num_heads * a.Tq;
  const int row_blocks = (M + 15) / 16;
  const int K = a.d.kv_lora_rank + a.d.qk_rope_head_dim;
  const int TT = valu_tile(a.d);
  const size_t lds = static_cast<size_t>((16 + TT) * (K + 1) + 16 * TT + 16) * sizeof(float);
  const unsigned grid = static_cast<unsigned>(a.max_items) * row_blocks;
  if (TT == 16)
    splitk_valu_kernel<16><<<grid, 256, lds, s>>>(a, row_blocks);
  else
    splitk_valu_kernel<8><<<grid, 256, lds, s>>>(a, row_blocks);
  return hipGetLastError();
}

hipError_t launch_combine(const DecodeArgs &a, hipStream_t s) {
  TimedLaunch tl("combine", s);
  const int rows = a.B * a.Tq * a.d.num_heads;
  combine_kernel<<<rows, 128, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_upproj(const DecodeArgs &a, hipStream_t s) {
  TimedLaunch tl("up_proj", s);
  if (a.d.v_head_dim % 32 == 0) {
    const int nrows = a.B * a.Tq;
    upproj_mfma_kernel<<<dim3(a.d.num_heads, (nrows + 31) / 32), 256, 0, s>>>(a);
  } else {
    const int waves = a.d.num_heads * a.d.v_head_dim;
    upproj_valu_kernel<<<(waves + 3) / 4, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace mla
