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
// Selection = radix select on unique 64-bit keys
//     key(t) = ordered(score_t) << 32 | (0xffffffff - t)
// (ordered() maps fp32 to an unsigned integer with the same order), eight
// passes of 8 bits from the top.  Pass p histograms digit p of the keys that
// match the prefix fixed by passes 0..p-1; every block re-derives that prefix
// from the earlier histograms, so no pass needs a separate scan launch.  The
// k-th largest key T then selects exactly top_k tokens (key >= T); a count
// pass and a write pass emit them in token order.
#include "kernels.hpp"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kPasses = 8;

__device__ __forceinline__ uint32_t ordered_bits(float s) {
  const uint32_t b = __float_as_uint(s);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint64_t token_key(float s, int t) {
  return (static_cast<uint64_t>(ordered_bits(s)) << 32) | static_cast<uint64_t>(0xffffffffu - static_cast<uint32_t>(t));
}

// scores[base + t] = q_idx[b] . idx_key[base + t], t < L_b.  Block (b, 0)
// also clears pass 0's histogram of b.
__global__ __launch_bounds__(kThreads) void index_score_kernel(IndexArgs a) {
  __shared__ float q[256];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int d = a.d_idx;
  for (int e = tid; e < d; e += kThreads) q[e] = bf16_to_f32(a.q_idx[static_cast<int64_t>(b) * d + e]);
  if (blockIdx.y == 0)
    for (int j = tid; j < 256; j += kThreads) a.hist[(0 * a.B + b) * 256 + j] = 0u;
  __syncthreads();
  const int L = a.seq_len[b];
  const int64_t base = a.seq_base[b];
  for (int t = blockIdx.y * kThreads + tid; t < L; t += gridDim.y * kThreads) {
    const uint16_t *k = a.idx_key + (base + t) * d;
    float acc = 0.0f;
    for (int e0 = 0; e0 < d; e0 += 8) {
      const uint4 raw = *reinterpret_cast<const uint4 *>(k + e0);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc = __builtin_fmaf(__uint_as_float(w[j] << 16), q[e0 + 2 * j], acc);
        acc = __builtin_fmaf(__uint_as_float(w[j] & 0xffff0000u), q[e0 + 2 * j + 1], acc);
      }
    }
    a.scores[base + t] = acc;
  }
}

// Prefix (the key bits fixed so far) and the rank still to find inside it,
// from the histograms of passes 0 .. p-1 of sequence b.
struct Prefix {
  uint64_t bits;
  int k_rem;
};

__device__ __forceinline__ Prefix derive_prefix(const uint32_t *hist, int B, int b, int p, int k) {
  Prefix x{0, k};
  for (int q = 0; q < p; ++q) {
    const uint32_t *h = hist + (static_cast<int64_t>(q) * B + b) * 256;
    int above = 0, j = 255;
    for (; j > 0; --j) {
      const int c = static_cast<int>(h[j]);
      if (above + c >= x.k_rem) break;
      above += c;
    }
    x.bits = (x.bits << 8) | static_cast<uint64_t>(j);
    x.k_rem -= above;
  }
  return x;
}

// Pass p: histogram of digit p over the keys matching the prefix.  Block
// (b, 0) clears the next pass's histogram of b.
__global__ __launch_bounds__(kThreads) void radix_pass_kernel(IndexArgs a, int p) {
  __shared__ uint32_t h[256];
  __shared__ Prefix pre;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int L = a.seq_len[b];
  if (L <= a.top_k) return;  // everything is selected
  h[tid] = 0u;
  if (tid == 0) pre = derive_prefix(a.hist, a.B, b, p, a.top_k);
  if (blockIdx.y == 0 && p + 1 < kPasses) a.hist[(static_cast<int64_t>(p + 1) * a.B + b) * 256 + tid] = 0u;
  __syncthreads();
  const uint64_t bits = pre.bits;
  const int shift = 56 - 8 * p;
  const int64_t base = a.seq_base[b];
  for (int t = blockIdx.y * kThreads + tid; t < L; t += gridDim.y * kThreads) {
    const uint64_t key = token_key(a.scores[base + t], t);
    if (p == 0 || (key >> (shift + 8)) == bits) atomicAdd(&h[(key >> shift) & 255u], 1u);
  }
  __syncthreads();
  if (h[tid] != 0u) atomicAdd(&a.hist[(static_cast<int64_t>(p) * a.B + b) * 256 + tid], h[tid]);
}

// The k-th largest key of sequence b (all eight digits fixed).
__device__ __forceinline__ uint64_t threshold_key(const IndexArgs &a, int b) {
  return derive_prefix(a.hist, a.B, b, kPasses, a.top_k).bits;
}

// Chunk c of sequence b for the count and write passes: tokens
// [c * chunk, (c + 1) * chunk), chunk = ceil(L / n_chunks).
__device__ __forceinline__ int chunk_len(int L, int n_chunks) { return (L + n_chunks - 1) / n_chunks; }

// Count pass: selected tokens per chunk.
__global__ __launch_bounds__(kThreads) void select_count_kernel(IndexArgs a) {
  __shared__ uint64_t thr;
  __shared__ int wsum[kThreads / 64];
  const int b = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
  const int L = a.seq_len[b];
  const bool all = L <= a.top_k;
  if (tid == 0) thr = all ? 0 : threshold_key(a, b);
  __syncthreads();
  const int64_t base = a.seq_base[b];
  const int cl = chunk_len(L, a.n_chunks);
  const int t0 = min(L, c * cl), t1 = min(L, t0 + cl);
  int n = 0;
  for (int t = t0 + tid; t < t1; t += kThreads) n += (all || token_key(a.scores[base + t], t) >= thr) ? 1 : 0;
  for (int off = 32; off > 0; off >>= 1) n += __shfl_xor(n, off);
  if ((tid & 63) == 0) wsum[tid >> 6] = n;
  __syncthreads();
  if (tid == 0) a.counts[b * a.n_chunks + c] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
}

// Write pass: each chunk writes its selected tokens, in token order, after
// those of the chunks before it.  Block (b, 0) writes n_sel[b].
__global__ __launch_bounds__(kThreads) void select_write_kernel(IndexArgs a) {
  __shared__ uint64_t thr;
  __shared__ int start;
  __shared__ int wtot[kThreads / 64];
  const int b = blockIdx.x, c = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int L = a.seq_len[b];
  const bool all = L <= a.top_k;
  if (tid == 0) {
    thr = all ? 0 : threshold_key(a, b);
    int s = 0;
    for (int j = 0; j < c; ++j) s += a.counts[b * a.n_chunks + j];
    start = s;
    if (c == 0) a.n_sel[b] = min(L, a.top_k);
  }
  __syncthreads();
  const int64_t base = a.seq_base[b];
  const int cl = chunk_len(L, a.n_chunks);
  const int t0 = min(L, c * cl), t1 = min(L, t0 + cl);
  int pos = start;
  for (int g = t0; g < t1; g += kThreads) {
    const int t = g + tid;
    const int sel = (t < t1 && (all || token_key(a.scores[base + t], t) >= thr)) ? 1 : 0;
    int inc = sel;  // inclusive scan over the block
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(inc, off);
      if (lane >= off) inc += y;
    }
    if (lane == 63) wtot[wv] = inc;
    __syncthreads();
    int before = 0;
    for (int j = 0; j < wv; ++j) before += wtot[j];
    const int idx = pos + before + inc - sel;
    if (sel && idx < a.top_k) a.sel[static_cast<int64_t>(b) * a.top_k + idx] = t;
    pos += wtot[0] + wtot[1] + wtot[2] + wtot[3];
    __syncthreads();  // wtot is rewritten by the next group
  }
}

}  // namespace

int index_chunks() { return 64; }

hipError_t launch_index_topk(const IndexArgs &a, hipStream_t s) {
  // scores and histograms stride over the tokens with 4x the chunk blocks
  const dim3 wide(a.B, 4 * a.n_chunks), chunks(a.B, a.n_chunks);
  {
    TimedLaunch tl("index_score", s);
    index_score_kernel<<<wide, kThreads, 0, s>>>(a);
  }
  TimedLaunch tl("index_select", s);
  for (int p = 0; p < kPasses; ++p) radix_pass_kernel<<<wide, kThreads, 0, s>>>(a, p);
  select_count_kernel<<<chunks, kThreads, 0, s>>>(a);
  select_write_kernel<<<chunks, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
