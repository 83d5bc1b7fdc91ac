// Sparse decode through the cached indexer key: per-token index scores and
// an exact top-k selection, all on the device from seq_len (no host sync).
//
// [llm-helper PR #64, PR description]: GLM-5.3-Flash's latent layers carry a
// sparse-attention indexer and cache its key next to the latent.  The page
// names no scoring rule; the one implemented is a dot product of one index
// query vector per sequence with each cached index key, accumulated in fp32
// in channel order (every bf16 x bf16 product is exact in fp32, so a fused
// multiply-add rounds exactly like a separate add), and the selection is the
// top_k tokens by score, equal scores going to the lower token index.
//
// Selection = radix select on the scores as ordered 32-bit keys (ordered()
// maps fp32 to an unsigned integer with the same order), four passes of 8
// bits from the top.  Pass p histograms digit p of the keys that match the
// prefix fixed by passes 0..p-1; every block re-derives that prefix from the
// earlier histograms (a block-wide scan per pass), so no pass needs a
// separate launch for it.  The k-th largest key T then selects every token
// with key > T and, of the tokens with key == T, the lowest-indexed ones
// still needed; a count pass and a write pass emit them in token order.
#include "kernels.hpp"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kPasses = 4;

__device__ __forceinline__ uint32_t ordered_bits(float s) {
  const uint32_t b = __float_as_uint(s);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// scores[base + t] = q_idx[b] . idx_key[base + t], t < L_b.  Block (b, 0)
// also clears pass 0's histogram of b.  D = index_head_dim (compile-time,
// so each lane's key loads are all in flight together).
template <int D>
__global__ __launch_bounds__(kThreads) void index_score_kernel(IndexArgs a) {
  __shared__ float q[D];
  const int b = blockIdx.x, tid = threadIdx.x;
  for (int e = tid; e < D; e += kThreads) q[e] = bf16_to_f32(a.q_idx[static_cast<int64_t>(b) * D + e]);
  if (blockIdx.y == 0) a.hist[(0 * a.B + b) * 256 + tid] = 0u;
  __syncthreads();
  const int L = a.seq_len[b];
  const int64_t base = a.seq_base[b];
  for (int t = blockIdx.y * kThreads + tid; t < L; t += gridDim.y * kThreads) {
    const uint4 *k = reinterpret_cast<const uint4 *>(a.idx_key + (base + t) * D);
    uint4 raw[D / 8];
#pragma unroll
    for (int i = 0; i < D / 8; ++i) raw[i] = k[i];
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
      const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc = __builtin_fmaf(__uint_as_float(w[j] << 16), q[8 * i + 2 * j], acc);
        acc = __builtin_fmaf(__uint_as_float(w[j] & 0xffff0000u), q[8 * i + 2 * j + 1], acc);
      }
    }
    a.scores[base + t] = acc;
  }
}

// Prefix (the key bits fixed by the first p passes) and the rank still to
// find inside it, from the histograms of sequence b.  Called by the whole
// block; per pass one block-wide scan over the 256 bins from the top.
struct Prefix {
  uint32_t bits;
  int k_rem;
};

__device__ Prefix derive_prefix(const uint32_t *hist, int B, int b, int p, int k) {
  __shared__ int wtot[kThreads / 64];
  __shared__ Prefix px;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  Prefix x{0u, k};
  for (int q = 0; q < p; ++q) {
    // thread i looks at bin 255 - i: inclusive count of keys in bins >= it
    const int c = static_cast<int>(hist[(static_cast<int64_t>(q) * B + b) * 256 + 255 - tid]);
    int inc = c;
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(inc, off);
      if (lane >= off) inc += y;
    }
    if (lane == 63) wtot[wv] = inc;
    __syncthreads();
    for (int j = 0; j < wv; ++j) inc += wtot[j];
    const int above = inc - c;
    if (above < x.k_rem && inc >= x.k_rem) {
      px.bits = (x.bits << 8) | static_cast<uint32_t>(255 - tid);
      px.k_rem = x.k_rem - above;
    }
    __syncthreads();
    x = px;
    __syncthreads();  // px and wtot are rewritten by the next pass
  }
  return x;
}

// Chunk c of sequence b: tokens [c * chunk, (c + 1) * chunk), chunk =
// ceil(L / n_chunks); the block reads it kUnroll groups of kThreads tokens at
// a time, loads first (clamped to the chunk, so none is predicated).
constexpr int kUnroll = 4;

__device__ __forceinline__ void chunk_range(int L, int n_chunks, int c, int *t0, int *t1) {
  const int cl = (L + n_chunks - 1) / n_chunks;
  *t0 = min(L, c * cl);
  *t1 = min(L, *t0 + cl);
}

template <typename F>
__device__ __forceinline__ void for_chunk_keys(const float *scores, int64_t base, int t0, int t1, F f) {
  const int tid = threadIdx.x;
  for (int g = t0; g < t1; g += kUnroll * kThreads) {
    uint32_t key[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) key[u] = ordered_bits(scores[base + min(g + u * kThreads + tid, t1 - 1)]);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) f(g + u * kThreads, g + u * kThreads + tid, key[u]);
  }
}

// Pass p: histogram of digit p over the keys matching the prefix.  Block
// (b, 0) clears the next pass's histogram of b.
__global__ __launch_bounds__(kThreads) void radix_pass_kernel(IndexArgs a, int p) {
  __shared__ uint32_t h[256];
  const int b = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
  const int L = a.seq_len[b];
  if (L <= a.top_k) return;  // everything is selected
  h[tid] = 0u;
  const Prefix pre = derive_prefix(a.hist, a.B, b, p, a.top_k);
  if (c == 0 && p + 1 < kPasses) a.hist[(static_cast<int64_t>(p + 1) * a.B + b) * 256 + tid] = 0u;
  __syncthreads();
  const int shift = 24 - 8 * p;
  int t0, t1;
  chunk_range(L, a.n_chunks, c, &t0, &t1);
  for_chunk_keys(a.scores, a.seq_base[b], t0, t1, [&](int, int t, uint32_t key) {
    if (t < t1 && (p == 0 || (key >> (shift + 8)) == pre.bits)) atomicAdd(&h[(key >> shift) & 255u], 1u);
  });
  __syncthreads();
  if (h[tid] != 0u) atomicAdd(&a.hist[(static_cast<int64_t>(p) * a.B + b) * 256 + tid], h[tid]);
}

// Block-wide exclusive scan of one int per thread; total in *tot.
__device__ __forceinline__ int block_excl_scan(int v, int *wtot, int *tot) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int inc = v;
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  if (lane == 63) wtot[wv] = inc;
  __syncthreads();
  int before = 0;
  for (int j = 0; j < wv; ++j) before += wtot[j];
  *tot = (wtot[0] + wtot[1]) + (wtot[2] + wtot[3]);
  __syncthreads();  // wtot may be rewritten by the next call
  return before + inc - v;
}

// Count pass: per chunk, tokens above the threshold key and tokens equal to it.
__global__ __launch_bounds__(kThreads) void select_count_kernel(IndexArgs a) {
  __shared__ int wsum[2][kThreads / 64];
  const int b = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
  const int L = a.seq_len[b];
  const bool all = L <= a.top_k;
  const uint32_t thr = all ? 0u : derive_prefix(a.hist, a.B, b, kPasses, a.top_k).bits;
  int t0, t1;
  chunk_range(L, a.n_chunks, c, &t0, &t1);
  int gt = 0, eq = 0;
  for_chunk_keys(a.scores, a.seq_base[b], t0, t1, [&](int, int t, uint32_t key) {
    gt += (t < t1 && (all || key > thr)) ? 1 : 0;
    eq += (t < t1 && !all && key == thr) ? 1 : 0;
  });
  for (int off = 32; off > 0; off >>= 1) {
    gt += __shfl_xor(gt, off);
    eq += __shfl_xor(eq, off);
  }
  if ((tid & 63) == 0) {
    wsum[0][tid >> 6] = gt;
    wsum[1][tid >> 6] = eq;
  }
  __syncthreads();
  if (tid == 0) {
    a.counts[(b * a.n_chunks + c) * 2 + 0] = (wsum[0][0] + wsum[0][1]) + (wsum[0][2] + wsum[0][3]);
    a.counts[(b * a.n_chunks + c) * 2 + 1] = (wsum[1][0] + wsum[1][1]) + (wsum[1][2] + wsum[1][3]);
  }
}

// Write pass: each chunk writes its selected tokens, in token order, after
// those of the chunks before it; of the tokens equal to the threshold key
// the first k_eq in token order are selected.  Block (b, 0) writes n_sel[b].
__global__ __launch_bounds__(kThreads) void select_write_kernel(IndexArgs a) {
  __shared__ int wtot[kThreads / 64];
  const int b = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
  const int L = a.seq_len[b];
  const bool all = L <= a.top_k;
  const Prefix pre = all ? Prefix{0u, 0} : derive_prefix(a.hist, a.B, b, kPasses, a.top_k);
  const uint32_t thr = pre.bits;
  const int k_eq = pre.k_rem;  // tokens needed from those equal to the threshold
  // counts of the chunks before this one (one per thread, n_chunks <= kThreads)
  int gt_before, eq_before;
  {
    const int j = tid;
    const int g = j < c ? a.counts[(b * a.n_chunks + j) * 2 + 0] : 0;
    const int e = j < c ? a.counts[(b * a.n_chunks + j) * 2 + 1] : 0;
    block_excl_scan(g, wtot, &gt_before);
    block_excl_scan(e, wtot, &eq_before);
  }
  if (c == 0 && tid == 0) a.n_sel[b] = min(L, a.top_k);
  int t0, t1;
  chunk_range(L, a.n_chunks, c, &t0, &t1);
  int eq_run = eq_before;                          // equal-key tokens before this group
  int pos = gt_before + min(eq_before, k_eq);      // selected tokens before this group
  for_chunk_keys(a.scores, a.seq_base[b], t0, t1, [&](int, int t, uint32_t key) {
    const int is_gt = (t < t1 && (all || key > thr)) ? 1 : 0;
    const int is_eq = (t < t1 && !all && key == thr) ? 1 : 0;
    int n_eq, n_sel;
    const int eq_rank = eq_run + block_excl_scan(is_eq, wtot, &n_eq);
    const int sel = is_gt | ((is_eq && eq_rank < k_eq) ? 1 : 0);
    const int idx = pos + block_excl_scan(sel, wtot, &n_sel);
    if (sel && idx < a.top_k) a.sel[static_cast<int64_t>(b) * a.top_k + idx] = t;
    pos += n_sel;
    eq_run += n_eq;
  });
}

}  // namespace

int index_chunks() { return kThreads; }

hipError_t launch_index_topk(const IndexArgs &a, hipStream_t s) {
  const dim3 chunks(a.B, a.n_chunks);
  {
    TimedLaunch tl("index_score", s);
    switch (a.d_idx) {
      case 64: index_score_kernel<64><<<chunks, kThreads, 0, s>>>(a); break;
      case 128: index_score_kernel<128><<<chunks, kThreads, 0, s>>>(a); break;
      default: return hipErrorInvalidValue;
    }
  }
  TimedLaunch tl("index_select", s);
  for (int p = 0; p < kPasses; ++p) radix_pass_kernel<<<chunks, kThreads, 0, s>>>(a, p);
  select_count_kernel<<<chunks, kThreads, 0, s>>>(a);
  select_write_kernel<<<chunks, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
