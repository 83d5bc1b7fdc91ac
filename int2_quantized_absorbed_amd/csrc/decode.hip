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
#include "plan.hpp"

namespace mla {

namespace {

__global__ __launch_bounds__(256) void plan_kernel(const int32_t *__restrict__ seq_len, int B,
                                                   int target, int tile, int min_k, int max_items,
                                                   WorkItem *__restrict__ items,
                                                   int32_t *__restrict__ item_begin,
                                                   int32_t *__restrict__ meta) {
  plan_block(seq_len, B, target, tile, min_k, max_items, items, item_begin, meta);
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
  const bool has_v = a.vcache.codes != nullptr;
  float *v_s = has_v ? al_s + ROWS : z_s;  // [TT][KP] values (their own cache, or the latent)
  const int tid = threadIdx.x;
  const int row0 = rb * ROWS;
  const int L = a.seq_len[it.b];
  const int64_t base = a.seq_base[it.b];
  const int32_t *sel = a.sel ? a.sel + static_cast<int64_t>(it.b) * a.sel_stride : nullptr;
  auto slot_of = [&](int tau) -> int64_t { return base + (sel ? sel[tau] : tau); };
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
  // dequantised entry (fp32) of channel j of cache slot `slot`
  auto dequant = [&](const mla_cache &c, int64_t slot, int j) -> float {
    const uint32_t byte = c.codes[slot * (r / 4) + j / 4];
    const uint32_t code = (byte >> (2 * (j & 3))) & 3u;
    const uint32_t sz = reinterpret_cast<const uint32_t *>(c.scale_zero)[slot * (r / G) + j / G];
    const float sc = static_cast<float>(bits_f16(static_cast<uint16_t>(sz & 0xffffu)));
    const float zr = static_cast<float>(bits_f16(static_cast<uint16_t>(sz >> 16)));
    return fmaf(sc, static_cast<float>(code), zr);
  };
  for (int t0 = it.t0; t0 < it.t1; t0 += TT) {
    __syncthreads();
    // dequantise the tile into LDS (fp32), rope key appended; values too
    // when they have their own cache
    for (int e = tid; e < TT * r; e += 256) {
      const int tk = e / r, j = e % r;
      const int tau = t0 + tk;
      float v = 0.0f, vv = 0.0f;
      if (tau < it.t1) {
        const int64_t slot = slot_of(tau);
        v = dequant(a.cache, slot, j);
        if (has_v) vv = dequant(a.vcache, slot, j);
      }
      z_s[tk * KP + j] = v;
      if (has_v) v_s[tk * KP + j] = vv;
    }
    for (int e = tid; e < TT * dr; e += 256) {
      const int tk = e / dr, k = e % dr;
      const int tau = t0 + tk;
      float v = 0.0f;
      if (tau < it.t1) {
        if (a.d.rope_bits == 4) {  // 4-bit rope key: zero + scale * code, one rounding
          const uint8_t *en = reinterpret_cast<const uint8_t *>(a.cache.k_rope) + slot_of(tau) * (dr / 2 + dr / 4);
          const uint32_t code = (en[k >> 1] >> (4 * (k & 1))) & 15u;
          const uint32_t sz = *reinterpret_cast<const uint32_t *>(en + dr / 2 + 4 * (k >> 4));
          v = fmaf(static_cast<float>(bits_f16(static_cast<uint16_t>(sz & 0xffffu))), static_cast<float>(code),
                   static_cast<float>(bits_f16(static_cast<uint16_t>(sz >> 16))));
        } else {
          v = bf16_to_f32(a.cache.k_rope[slot_of(tau) * dr + k]);
        }
      }
      z_s[tk * KP + r + k] = v;
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
        for (int tk = 0; tk < TT; ++tk) o = fmaf(p_s[row * TT + tk], v_s[tk * KP + j], o);
        acc[i] = o;
      }
    }
  }
  // partial O normalised by its row's l, in fp16
  __syncthreads();  // the last tile's alpha reads are done
  if (scorer && stok == 0) al_s[srow] = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  __syncthreads();
  f16 *po = reinterpret_cast<f16 *>(a.part_o);
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    if (i < na) {
      const int e = tid + 256 * i;
      const int row = e / r, j = e % r;
      const int m = row0 + row;
      if (m < M) po[(static_cast<int64_t>(item) * M + m) * r + j] = f32_to_f16(acc[i] * al_s[row]);
    }
  }
  if (scorer && stok == 0 && sm < M) {
    a.part_ml[(static_cast<int64_t>(item) * M + sm) * 2 + 0] = m_run;
    a.part_ml[(static_cast<int64_t>(item) * M + sm) * 2 + 1] = l_run;
  }
}

// Log-sum-exp merge of the split-K partials of one query row (b, t, h):
// m = max_i m_i, o_z = sum_i 2^(m_i - m) O_i / sum_i 2^(m_i - m) l_i,
// lse = ln 2 * (m + log2 sum_i 2^(m_i - m) l_i), with O_i = l_i * (the
// stored fp16 O_i / l_i).  One block per row; thread
// -> (item slice s, 4-channel chunk c).  Slice s folds items ib + s,
// ib + s + S, ... into a running (max, sum, O) U items per round (addresses
// clamped and weights zeroed past the end, so the U loads are issued
// together); the S slice results are then merged in slice order.
template <int U>
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
  __shared__ f32x4 part[256];
  __shared__ float part_m[256], part_l[256];
  const int H = a.d.num_heads, r = a.d.kv_lora_rank;
  const int M = H * a.Tq;
  const int row = blockIdx.x;               // (b*Tq + t)*H + h
  const int q = row / H, h = row % H;
  const int b = q / a.Tq, t = q % a.Tq, m = t * H + h;
  const int ib = a.item_begin[b], ie = a.item_begin[b + 1];
  const int chunks = r >> 2, S = 256 / chunks;
  const int tid = threadIdx.x, sl = tid / chunks, c = tid % chunks;
  const float *ml = a.part_ml + static_cast<int64_t>(m) * 2;
  const f16 *po = reinterpret_cast<const f16 *>(a.part_o) + static_cast<int64_t>(m) * r + 4 * c;
  const int64_t ml_stride = static_cast<int64_t>(M) * 2, po_stride = static_cast<int64_t>(M) * r;
  float mrun = -INFINITY, lrun = 0.0f;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  if (sl < S) {
    for (int k0 = ib + sl; k0 < ie; k0 += U * S) {
      f16x4 v[U];
      float2 st[U];
#pragma unroll
      for (int e = 0; e < U; ++e) {
        const int k = min(k0 + e * S, ie - 1);
        v[e] = *reinterpret_cast<const f16x4 *>(po + k * po_stride);
        st[e] = *reinterpret_cast<const float2 *>(ml + k * ml_stride);
        if (k0 + e * S >= ie) st[e].x = -INFINITY;
      }
      float rm = mrun;
#pragma unroll
      for (int e = 0; e < U; ++e) rm = fmaxf(rm, st[e].x);
      if (rm != -INFINITY) {
        const float sc = exp2f(mrun - rm);  // 0 while nothing was folded in
        acc *= sc;
        lrun *= sc;
#pragma unroll
        for (int e = 0; e < U; ++e) {
          // item e: weight 2^(m_e - max) on l_e and on O_e = l_e * (its O / l)
          const float wgt = st[e].x == -INFINITY ? 0.0f : exp2f(st[e].x - rm);
          acc += (wgt * st[e].y) * __builtin_convertvector(v[e], f32x4);
          lrun += wgt * st[e].y;
        }
        mrun = rm;
      }
    }
  }
  part[tid] = acc;
  part_m[tid] = mrun;
  part_l[tid] = lrun;
  __syncthreads();
  if (tid < chunks) {
    float mx = -INFINITY;
    for (int j = 0; j < S; ++j) mx = fmaxf(mx, part_m[j * chunks + c]);
    float den = 0.0f;
    f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f};
    if (mx != -INFINITY)
      for (int j = 0; j < S; ++j) {
        const float mj = part_m[j * chunks + c];
        if (mj == -INFINITY) continue;
        const float wgt = exp2f(mj - mx);
        den += wgt * part_l[j * chunks + c];
        o += wgt * part[j * chunks + c];
      }
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    *reinterpret_cast<f32x4 *>(a.oz + static_cast<int64_t>(row) * r + 4 * c) = o * inv;
    if (tid == 0 && a.lse != nullptr) a.lse[row] = den > 0.0f ? (mx + log2f(den)) * kLn2 : -INFINITY;
  }
}

// out[b,t,h,:] = W~_UV[h] o_z[b,t,h,:] on MFMA (32x32x16 f16, fp32 acc).
// o_z is split as hi + lo (two fp16 parts) so the product keeps ~fp32
// precision of o_z; W~_UV is fp16.  Block = (head, 32 output columns, 32
// query rows); wave w takes a quarter of the latent K-steps (all of its loads
// are issued before the first product), and the four partial tiles are added
// in LDS in a fixed order.
__global__ __launch_bounds__(256) void upproj_mfma_kernel(DecodeArgs a) {
  __shared__ float red[4][16][64];
  const int h = blockIdx.x, v0 = 32 * blockIdx.y, rt = blockIdx.z;
  const int H = a.d.num_heads, r = a.d.kv_lora_rank, dv = a.d.v_head_dim;
  const int nrows = a.B * a.Tq;
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6, hf = l >> 5, l32 = l & 31;
  const int q = rt * 32 + l32;              // A-operand row of this lane
  const bool q_ok = q < nrows;
  const float *arow = a.oz + (static_cast<int64_t>(q_ok ? q : 0) * H + h) * r + 8 * hf;
  const uint16_t *brow = a.w_uv_f + (static_cast<int64_t>(h) * dv + v0 + l32) * r + 8 * hf;
  const int nks = r >> 4, ks0 = (w * nks) >> 2, ks1 = ((w + 1) * nks) >> 2;
  f32x16 acc = {};
  for (int ks = ks0; ks < ks1; ks += 8) {
    f32x4 x[8][2];
    f16x8 bw[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int kk = min(ks + e, ks1 - 1) * 16;
      x[e][0] = *reinterpret_cast<const f32x4 *>(arow + kk);  // row 0 stands in for q >= nrows
      x[e][1] = *reinterpret_cast<const f32x4 *>(arow + kk + 4);
      bw[e] = *reinterpret_cast<const f16x8 *>(brow + kk);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the products
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (ks + e >= ks1) break;
      f16x8 ahi, alo;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float xv = q_ok ? x[e][j >> 2][j & 3] : 0.0f;
        const f16 hv = static_cast<f16>(xv);
        ahi[j] = hv;
        alo[j] = static_cast<f16>(xv - static_cast<float>(hv));
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi, bw[e], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo, bw[e], acc, 0, 0, 0);
    }
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) red[w][v][l] = acc[v];
  __syncthreads();
  // C layout: lane holds column v0 + l32, rows 8(v/4) + 4hf + v%4
  for (int e = tid; e < 16 * 64; e += 256) {
    const int v = e >> 6, ln = e & 63;
    const int qq = rt * 32 + 8 * (v >> 2) + 4 * (ln >> 5) + (v & 3);
    if (qq < nrows)
      a.out[(static_cast<int64_t>(qq) * H + h) * dv + v0 + (ln & 31)] =
          ((red[0][v][ln] + red[1][v][ln]) + red[2][v][ln]) + red[3][v][ln];
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

// Combine and up-projection in one launch for r = 512, d_v = 128 and at most
// kFuseMaxRows query rows per head.  Block = (head h, tile of RT query rows),
// 512 threads, blocks of one head on one XCD (they share W~_UV[h] in L2).
//  1. Merge: thread (slice s, row j, 4-channel chunk c) folds items ib + s,
//     ib + s + S, ... (S = 4 / RT slices; with RT = 8 or 16 one slice and
//     the rows j, j + 4, ... in turn) of row j into a running (max, sum,
//     O), kCombU items per round with their loads issued together; the
//     slices are merged in slice order and o_z[j] = O / l goes to LDS (and
//     lse out).
//  2. Product: wave wv owns output columns 16 wv .. 16 wv + 15; its slice of
//     W~_UV[h] (fp16) is loaded at kernel start, so it is in flight during
//     the merge.
//     RT >= 4: on MFMA (v_mfma_f32_16x16x32_f16), the RT rows padded to 16,
//     K = the 512 latent channels in 16 steps; lane l holds W~_UV rows
//     16 wv + (l & 15) at channels 32 ks + 8 (l >> 4) ..; o_z is staged in
//     LDS as two fp16 parts (hi + lo), each its own product chain, so the
//     result keeps about fp32 precision of o_z.
//     RT < 4 (the MFMA tile would be mostly padding): lane l holds latent
//     channels 8 l .. 8 l + 7 of the 16 rows and forms RT x 16 eight-term
//     fp32 partial sums; a butterfly reduce-scatter over the 64 lanes adds
//     them up (lane l ends with the output l >> (6 - log2(16 RT)) in full).
constexpr int kFuseR = 512, kFuseDv = 128, kFuseThreads = 512, kFuseMaxRows = 32, kCombU = 16;

// p[0 .. N) summed over the lanes that differ in bits log2(D) .. log2(D) - log2(N) + 1:
// at each step a lane keeps one half (the upper one if its bit D is set), adds the
// partner's copy of that half, and passes the other half on.
template <int N, int D>
__device__ __forceinline__ void lane_reduce_scatter(float *p, int lane) {
  if constexpr (N > 1) {
    const bool up = (lane & D) != 0;
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const float keep = up ? p[N / 2 + i] : p[i];
      const float give = up ? p[i] : p[N / 2 + i];
      p[i] = keep + __shfl_xor(give, D);
    }
    lane_reduce_scatter<N / 2, D / 2>(p, lane);
  }
}

template <int RT>
__global__ __launch_bounds__(kFuseThreads) void combine_upproj_kernel(DecodeArgs a, int n_rt, int n_logical) {
  // merge threads: S item slices x min(RT, 4) rows x CH chunks; with RT > 4
  // a thread merges rows j, j + 4, ... in turn
  constexpr int RJ = RT < 4 ? RT : 4, S = 4 / RJ, RPT = RT / RJ, CH = kFuseR / 4;
  constexpr int V = 16 * RT, LOGV = RT == 1 ? 4 : (RT == 2 ? 5 : 6);
  constexpr bool kMfma = RT >= 4;
  // o_z: fp32 for the vector-ALU product; fp16 hi and lo parts for the
  // MFMA one, rows padded 16 bytes so the 16-lane groups of an operand read
  // (rows 1040 bytes apart) fall on separate banks
  constexpr int ZST = kFuseR + 8;
  static_assert(S * RJ * CH == kFuseThreads, "one (slice, row, chunk) per thread and pass");
  __shared__ f32x4 s_o[S][RT][CH];
  __shared__ float s_m[S][RT], s_l[S][RT];
  __shared__ __align__(16) float s_z[kMfma ? 1 : RT][kFuseR];
  __shared__ __align__(16) f16 s_zh[kMfma ? RT : 1][ZST], s_zl[kMfma ? RT : 1][ZST];
  const int per_xcd = (n_logical + 7) / 8;
  const int logical = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (logical >= n_logical) return;
  const int h = logical / n_rt, rt = logical % n_rt;
  const int H = a.d.num_heads, M = H * a.Tq, nrows = a.B * a.Tq;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  // MFMA: wr[ks] = rows 16 wv + (lane & 15), channels 32 ks + 8 (lane >> 4) ..;
  // vector ALU: wr[i] = row 16 wv + i, channels 8 lane ..
  f16x8 wr[16];
  {
    const uint16_t *wp =
        kMfma ? a.w_uv_f + (static_cast<int64_t>(h) * kFuseDv + 16 * wv + (lane & 15)) * kFuseR + 8 * (lane >> 4)
              : a.w_uv_f + (static_cast<int64_t>(h) * kFuseDv + 16 * wv) * kFuseR + 8 * lane;
#pragma unroll
    for (int i = 0; i < 16; ++i) wr[i] = *reinterpret_cast<const f16x8 *>(wp + i * (kMfma ? 32 : kFuseR));
  }

  // ---- 1. merge the partials ----
  if constexpr (RPT > 1) {
    // rows j = jb, jb + 4, ... of the tile (S = 1): their loads of a round,
    // U items per row, are issued together, so rows with at most U items
    // take one memory round trip.  A row without items (past the batch or
    // an empty sequence) reads item 0 of a valid row, masked.
    constexpr int U = kCombU / RPT;
    const int c = tid % CH, jb = (tid / CH) % RJ;
    int ib[RPT], ie[RPT];
    const float *ml[RPT];
    const f16 *po[RPT];
    float mrun[RPT], lrun[RPT];
    f32x4 acc[RPT];
    int rounds = 0;
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
      const int q = rt * RT + jb + RJ * rr;
      const int m = q < nrows ? (q % a.Tq) * H + h : 0;
      ib[rr] = q < nrows ? a.item_begin[q / a.Tq] : 0;
      ie[rr] = q < nrows ? a.item_begin[q / a.Tq + 1] : 0;
      ml[rr] = a.part_ml + static_cast<int64_t>(m) * 2;
      po[rr] = reinterpret_cast<const f16 *>(a.part_o) + static_cast<int64_t>(m) * kFuseR + 4 * c;
      rounds = max(rounds, (ie[rr] - ib[rr] + U - 1) / U);
      mrun[rr] = -INFINITY;
      lrun[rr] = 0.0f;
      acc[rr] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const int64_t ml_stride = static_cast<int64_t>(M) * 2, po_stride = static_cast<int64_t>(M) * kFuseR;
    for (int r = 0; r < rounds; ++r) {
      f16x4 v[RPT][U];
      float2 st[RPT][U];
#pragma unroll
      for (int rr = 0; rr < RPT; ++rr)
#pragma unroll
        for (int e = 0; e < U; ++e) {
          const int kk = ib[rr] + r * U + e;
          const int k = ie[rr] > ib[rr] ? min(kk, ie[rr] - 1) : 0;
          v[rr][e] = *reinterpret_cast<const f16x4 *>(po[rr] + k * po_stride);
          st[rr][e] = *reinterpret_cast<const float2 *>(ml[rr] + k * ml_stride);
          if (kk >= ie[rr]) st[rr][e].x = -INFINITY;
        }
#pragma unroll
      for (int rr = 0; rr < RPT; ++rr) {
        float rm = mrun[rr];
#pragma unroll
        for (int e = 0; e < U; ++e) rm = fmaxf(rm, st[rr][e].x);
        if (rm != -INFINITY) {
          const float sc = exp2f(mrun[rr] - rm);  // 0 while nothing was folded in
          acc[rr] *= sc;
          lrun[rr] *= sc;
#pragma unroll
          for (int e = 0; e < U; ++e) {
            const float wgt = st[rr][e].x == -INFINITY ? 0.0f : exp2f(st[rr][e].x - rm);
            acc[rr] += (wgt * st[rr][e].y) * __builtin_convertvector(v[rr][e], f32x4);
            lrun[rr] += wgt * st[rr][e].y;
          }
          mrun[rr] = rm;
        }
      }
    }
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
      const int j = jb + RJ * rr;
      s_o[0][j][c] = acc[rr];
      if (c == 0) {  // every chunk thread of a row holds the same (max, sum)
        s_m[0][j] = mrun[rr];
        s_l[0][j] = lrun[rr];
      }
    }
  } else {
    const int c = tid % CH, j = (tid / CH) % RJ, sl = tid / (CH * RJ);
    const int q = rt * RT + j;
    float mrun = -INFINITY, lrun = 0.0f;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (q < nrows) {
      const int b = q / a.Tq, m = (q % a.Tq) * H + h;
      const int ib = a.item_begin[b], ie = a.item_begin[b + 1];
      const float *ml = a.part_ml + static_cast<int64_t>(m) * 2;
      const f16 *po = reinterpret_cast<const f16 *>(a.part_o) + static_cast<int64_t>(m) * kFuseR + 4 * c;
      const int64_t ml_stride = static_cast<int64_t>(M) * 2, po_stride = static_cast<int64_t>(M) * kFuseR;
      for (int k0 = ib + sl; k0 < ie; k0 += kCombU * S) {
        f16x4 v[kCombU];
        float2 st[kCombU];
#pragma unroll
        for (int e = 0; e < kCombU; ++e) {
          const int k = min(k0 + e * S, ie - 1);
          v[e] = *reinterpret_cast<const f16x4 *>(po + k * po_stride);
          st[e] = *reinterpret_cast<const float2 *>(ml + k * ml_stride);
          if (k0 + e * S >= ie) st[e].x = -INFINITY;
        }
        float rm = mrun;
#pragma unroll
        for (int e = 0; e < kCombU; ++e) rm = fmaxf(rm, st[e].x);
        if (rm != -INFINITY) {
          const float sc = exp2f(mrun - rm);  // 0 while nothing was folded in
          acc *= sc;
          lrun *= sc;
#pragma unroll
          for (int e = 0; e < kCombU; ++e) {
            const float wgt = st[e].x == -INFINITY ? 0.0f : exp2f(st[e].x - rm);
            acc += (wgt * st[e].y) * __builtin_convertvector(v[e], f32x4);
            lrun += wgt * st[e].y;
          }
          mrun = rm;
        }
      }
    }
    s_o[sl][j][c] = acc;
    if (c == 0) {  // every chunk thread of (slice, row) holds the same (max, sum)
      s_m[sl][j] = mrun;
      s_l[sl][j] = lrun;
    }
  }
  __syncthreads();
  for (int u = tid; u < RT * CH; u += kFuseThreads) {
    const int j = u / CH, c = u % CH;
    float mx = -INFINITY;
#pragma unroll
    for (int sl = 0; sl < S; ++sl) mx = fmaxf(mx, s_m[sl][j]);
    float den = 0.0f;
    f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f};
    if (mx != -INFINITY) {
#pragma unroll
      for (int sl = 0; sl < S; ++sl) {
        const float mj = s_m[sl][j];
        if (mj == -INFINITY) continue;
        const float wgt = exp2f(mj - mx);
        den += wgt * s_l[sl][j];
        o += wgt * s_o[sl][j][c];
      }
    }
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    const f32x4 z = o * inv;
    if constexpr (kMfma) {
      const f16x4 zh = __builtin_convertvector(z, f16x4);
      *reinterpret_cast<f16x4 *>(&s_zh[j][4 * c]) = zh;
      *reinterpret_cast<f16x4 *>(&s_zl[j][4 * c]) =
          __builtin_convertvector(z - __builtin_convertvector(zh, f32x4), f16x4);
    } else {
      *reinterpret_cast<f32x4 *>(&s_z[j][4 * c]) = z;
    }
    const int q = rt * RT + j;
    if (c == 0 && q < nrows && a.lse != nullptr)
      a.lse[static_cast<int64_t>(q) * H + h] = den > 0.0f ? (mx + log2f(den)) * kLn2 : -INFINITY;
  }
  __syncthreads();

  // ---- 2. out = W~_UV[h] o_z ----
  if constexpr (kMfma) {
    // B operand: o_z row (lane & 15) (rows past RT repeat row RT - 1; their
    // columns of the product are not stored), channels 32 ks + 8 (lane >> 4) ..
    const f16 *zh = &s_zh[min(lane & 15, RT - 1)][8 * (lane >> 4)];
    const f16 *zl = &s_zl[min(lane & 15, RT - 1)][8 * (lane >> 4)];
    f32x4 acc_h = {0.0f, 0.0f, 0.0f, 0.0f}, acc_l = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      acc_h = __builtin_amdgcn_mfma_f32_16x16x32_f16(wr[ks], *reinterpret_cast<const f16x8 *>(zh + 32 * ks), acc_h,
                                                     0, 0, 0);
      acc_l = __builtin_amdgcn_mfma_f32_16x16x32_f16(wr[ks], *reinterpret_cast<const f16x8 *>(zl + 32 * ks), acc_l,
                                                     0, 0, 0);
    }
    // lane holds out[row lane & 15][16 wv + 4 (lane >> 4) + i], i = 0..3
    const int j = lane & 15, q = rt * RT + j;
    if (j < RT && q < nrows)
      *reinterpret_cast<f32x4 *>(a.out + (static_cast<int64_t>(q) * H + h) * kFuseDv + 16 * wv + 4 * (lane >> 4)) =
          acc_h + acc_l;
  } else {
  float part[V];
#pragma unroll
  for (int j = 0; j < RT; ++j) {
    const f32x4 z0 = *reinterpret_cast<const f32x4 *>(&s_z[j][8 * lane]);
    const f32x4 z1 = *reinterpret_cast<const f32x4 *>(&s_z[j][8 * lane + 4]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float t = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) t = fmaf(static_cast<float>(wr[i][e]), z0[e], t);
#pragma unroll
      for (int e = 0; e < 4; ++e) t = fmaf(static_cast<float>(wr[i][4 + e]), z1[e], t);
      part[16 * j + i] = t;
    }
  }
  lane_reduce_scatter<V, 32>(part, lane);
#pragma unroll
  for (int d = 32 >> LOGV; d > 0; d >>= 1) part[0] += __shfl_xor(part[0], d);
  const int idx = lane >> (6 - LOGV), j = idx >> 4, q = rt * RT + j;
  if ((lane & ((1 << (6 - LOGV)) - 1)) == 0 && q < nrows)
    a.out[(static_cast<int64_t>(q) * H + h) * kFuseDv + 16 * wv + (idx & 15)] = part[0];
  }
}

}  // namespace

hipError_t launch_plan(const DecodeArgs &a, hipStream_t s) {
  TimedLaunch tl("decode_plan", s);
  plan_kernel<<<1, 256, 0, s>>>(a.seq_len, a.B, a.target_items, a.tile, a.min_chunk_tiles, a.max_items,
                                a.items, a.item_begin, a.meta);
  return hipGetLastError();
}

hipError_t launch_absorb_f32(const DecodeArgs &a, hipStream_t s) {
  TimedLaunch tl("absorb_q", s);
  const size_t lds = static_cast<size_t>(16) * (a.d.qk_nope_head_dim + 1) * sizeof(float);
  absorb_f32_kernel<<<a.d.num_heads, 256, lds, s>>>(a);
  return hipGetLastError();
}

// LDS floats of splitk_valu_kernel at tile TT: queries, latent tile, P,
// alpha, and a value tile when values have their own cache
size_t valu_lds_floats(const mla_dims &d, int TT, bool has_v) {
  const int KP = d.kv_lora_rank + d.qk_rope_head_dim + 1;
  return static_cast<size_t>(16 + TT + (has_v ? TT : 0)) * KP + 16 * TT + 16;
}

int valu_tile(const mla_dims &d, bool has_v) {
  return valu_lds_floats(d, 16, has_v) * 4 <= 64 * 1024 ? 16 : 8;
}

hipError_t launch_splitk_valu(const DecodeArgs &a, hipStream_t s) {
  TimedLaunch tl("splitk_decode", s);
  const int M = a.d.num_heads * a.Tq;
  const int row_blocks = (M + 15) / 16;
  const bool has_v = a.vcache.codes != nullptr;
  const int TT = valu_tile(a.d, has_v);
  const size_t lds = valu_lds_floats(a.d, TT, has_v) * sizeof(float);
  const unsigned grid = static_cast<unsigned>(a.max_items) * row_blocks;
  if (TT == 16)
    splitk_valu_kernel<16><<<grid, 256, lds, s>>>(a, row_blocks);
  else
    splitk_valu_kernel<8><<<grid, 256, lds, s>>>(a, row_blocks);
  return hipGetLastError();
}

static bool combine_upproj_fused(const DecodeArgs &a) {
  return a.d.kv_lora_rank == kFuseR && a.d.v_head_dim == kFuseDv && a.B * a.Tq <= kFuseMaxRows;
}

hipError_t launch_combine(const DecodeArgs &a, hipStream_t s) {
  if (combine_upproj_fused(a)) {
    TimedLaunch tl("combine_up_proj", s);
    // the widest row tile that still gives every compute unit a block
    const int nrows = a.B * a.Tq, H = a.d.num_heads, ncu = device_cu_count();
    int rt = 16;
    while (rt > 1 && H * ((nrows + rt - 1) / rt) < ncu) rt >>= 1;
    const int n_rt = (nrows + rt - 1) / rt, n_logical = H * n_rt;
    const unsigned grid = static_cast<unsigned>((n_logical + 7) / 8) * 8;
    if (rt == 16)
      combine_upproj_kernel<16><<<grid, kFuseThreads, 0, s>>>(a, n_rt, n_logical);
    else if (rt == 8)
      combine_upproj_kernel<8><<<grid, kFuseThreads, 0, s>>>(a, n_rt, n_logical);
    else if (rt == 4)
      combine_upproj_kernel<4><<<grid, kFuseThreads, 0, s>>>(a, n_rt, n_logical);
    else if (rt == 2)
      combine_upproj_kernel<2><<<grid, kFuseThreads, 0, s>>>(a, n_rt, n_logical);
    else
      combine_upproj_kernel<1><<<grid, kFuseThreads, 0, s>>>(a, n_rt, n_logical);
    return hipGetLastError();
  }
  TimedLaunch tl("combine", s);
  const int rows = a.B * a.Tq * a.d.num_heads;
  // items per sequence average (target + B) / B; rounds of 16 pay off once
  // a slice sees more than one round of 8
  const int per_seq = (a.target_items + a.B) / a.B;
  const int S = 256 / (a.d.kv_lora_rank / 4);
  if (per_seq > 8 * S)
    combine_kernel<16><<<rows, 256, 0, s>>>(a);
  else
    combine_kernel<8><<<rows, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_upproj(const DecodeArgs &a, hipStream_t s) {
  if (combine_upproj_fused(a)) return hipSuccess;  // done by launch_combine
  TimedLaunch tl("up_proj", s);
  if (a.d.v_head_dim % 32 == 0) {
    const int nrows = a.B * a.Tq;
    upproj_mfma_kernel<<<dim3(a.d.num_heads, a.d.v_head_dim / 32, (nrows + 31) / 32), 256, 0, s>>>(a);
  } else {
    const int waves = a.d.num_heads * a.d.v_head_dim;
    upproj_valu_kernel<<<(waves + 3) / 4, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace mla
