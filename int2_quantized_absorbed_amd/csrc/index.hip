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
// Selection = radix select on the scores as ordered 32-bit keys (ordered_bits
// maps fp32 to an unsigned integer with the same order), three digits from
// the top: 12, 12 and 8 bits.  Pass p histograms digit p of the keys that
// match the prefix fixed by the passes before it; the score kernel does pass
// 0 as it writes the scores.  Each later launch reads the prefix the launch
// before it derived and extends it by one digit from that launch's histogram
// (one block-wide scan), so every launch scans one histogram.  The k-th
// largest key T selects every token with key > T and, of the tokens with
// key == T, the lowest-indexed ones still needed.  The last radix pass also
// keeps, per chunk of the sequence, the count of keys above its prefix and
// the suffix sums of its own last-digit histogram, from which the write pass
// knows how many tokens every earlier chunk selects without a count pass.
#include <algorithm>

#include "kernels.hpp"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kPasses = 3;
constexpr int kHistBins = 4096;  // per (pass, sequence) slot: the widest digit
constexpr int kLastBins = 256;

__host__ __device__ constexpr int digit_bits(int p) { return p == kPasses - 1 ? 8 : 12; }
__host__ __device__ constexpr int digit_shift(int p) { return p == 0 ? 20 : (p == 1 ? 8 : 0); }

static_assert(digit_bits(0) + digit_bits(1) + digit_bits(2) == 32, "three digits cover the key");
static_assert(digit_shift(1) + digit_bits(1) == digit_shift(0), "digits are contiguous");
static_assert(digit_shift(2) + digit_bits(2) == digit_shift(1), "digits are contiguous");
static_assert((1 << digit_bits(kPasses - 1)) == kLastBins, "last digit");

__device__ __forceinline__ uint32_t ordered_bits(float s) {
  const uint32_t b = __float_as_uint(s);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint32_t *hist_of(const IndexArgs &a, int p, int b) {
  return a.hist + (static_cast<int64_t>(p) * a.B + b) * kHistBins;
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

// Clears the three histograms of every sequence (grid (B, kPasses)).
__global__ __launch_bounds__(kThreads) void index_clear_kernel(IndexArgs a) {
  uint4 *h = reinterpret_cast<uint4 *>(hist_of(a, blockIdx.y, blockIdx.x));
#pragma unroll
  for (int i = 0; i < kHistBins / 4 / kThreads; ++i) h[i * kThreads + threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
}

// Flushes a block's LDS histogram into the global one (nonzero bins only).
template <int NB>
__device__ __forceinline__ void flush_hist(const uint32_t *h, uint32_t *g) {
#pragma unroll
  for (int i = 0; i < NB / kThreads; ++i) {
    const int bin = i * kThreads + threadIdx.x;
    if (h[bin] != 0u) atomicAdd(&g[bin], h[bin]);
  }
}

// scores[base + t] = q_idx[b] . idx_key[base + t], t < L_b, and radix pass
// 0 (digit 0 of every key) when the sequence has more than top_k tokens.
// D = index_head_dim (compile-time, so each lane's key loads are all in
// flight together).  A wave's 64 consecutive keys are read with contiguous
// 16-byte pieces per instruction (lane l takes piece l of each 1 KB) and
// passed to the lane of their token through the wave's 4 KB LDS buffer, in
// D / 32 rounds of 2048 / D tokens (piece p of a round's token r stored at
// slot p ^ (r & 7) of its row, so both sides spread over the banks); a lane
// then adds its token's products in channel order.
template <int D>
__global__ __launch_bounds__(kThreads) void index_score_kernel(IndexArgs a) {
  constexpr int PT = D / 8;             // 16-byte pieces per key
  constexpr int NR = D / 32;            // rounds through the buffer
  constexpr int TPR = 64 / NR;          // tokens per round
  constexpr int IPR = PT / NR;          // load instructions per round (4)
  static_assert(NR * TPR == 64 && IPR * 64 == TPR * PT, "a round is 4 KB of whole keys");
  __shared__ float q[D];
  __shared__ uint32_t h[1 << digit_bits(0)];
  __shared__ uint4 kbuf[kThreads / 64][TPR * PT];
  const int b = blockIdx.x, tid = threadIdx.x;
  for (int e = tid; e < D; e += kThreads) q[e] = bf16_to_f32(a.q_idx[static_cast<int64_t>(b) * D + e]);
  const int L = a.seq_len[b];
  const bool radix = L > a.top_k;
  if (radix) {
#pragma unroll
    for (int i = 0; i < (1 << digit_bits(0)) / kThreads; ++i) h[i * kThreads + tid] = 0u;
  }
  __syncthreads();
  const int64_t base = a.seq_base[b];
  const int lane = tid & 63;
  uint4 *kb = kbuf[tid >> 6];
  // uniform over the wave: its first token t - lane is below L
  for (int t = blockIdx.y * kThreads + tid; t - lane < L; t += gridDim.y * kThreads) {
    const int tw = t - lane;  // the wave's first token
    uint4 piece[PT];  // piece e = 64 i + lane of the wave's keys: token e / PT, piece e % PT
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int e = i * 64 + lane;
      piece[i] = reinterpret_cast<const uint4 *>(a.idx_key + (base + min(tw + e / PT, L - 1)) * D)[e % PT];
    }
    // Round rd: the round's keys into the buffer, then every lane reads the
    // round's token lane % TPR and the lanes whose token is in this round keep
    // it.  A wave's LDS operations run in order, and a lane's stores and
    // reads of the buffer may alias, so the compiler keeps their order too.
    uint32_t kw[PT][4];
#pragma unroll
    for (int rd = 0; rd < NR; ++rd) {
#pragma unroll
      for (int ii = 0; ii < IPR; ++ii) {
        const int e = (rd * IPR + ii) * 64 + lane, r = e / PT - rd * TPR, p = e % PT;
        kb[r * PT + (p ^ (r & 7))] = piece[rd * IPR + ii];
      }
      const int r = lane % TPR;
      const bool keep = rd == 0 || lane / TPR == rd;
#pragma unroll
      for (int i = 0; i < PT; ++i) {
        const uint4 v = kb[r * PT + (i ^ (r & 7))];
        kw[i][0] = keep ? v.x : kw[i][0];
        kw[i][1] = keep ? v.y : kw[i][1];
        kw[i][2] = keep ? v.z : kw[i][2];
        kw[i][3] = keep ? v.w : kw[i][3];
      }
    }
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < PT; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc = __builtin_fmaf(__uint_as_float(kw[i][j] << 16), q[8 * i + 2 * j], acc);
        acc = __builtin_fmaf(__uint_as_float(kw[i][j] & 0xffff0000u), q[8 * i + 2 * j + 1], acc);
      }
    if (t >= L) continue;
    a.scores[base + t] = acc;
    if (radix) atomicAdd(&h[ordered_bits(acc) >> digit_shift(0)], 1u);
  }
  if (!radix) return;  // uniform over the block
  __syncthreads();
  flush_hist<1 << digit_bits(0)>(h, hist_of(a, 0, b));
}

// The key bits fixed so far and the rank still to find among the keys that
// carry them.
struct Prefix {
  uint32_t bits;
  int k_rem;
};

// Extends `x` (the prefix after passes 0..p-1) by digit p, from pass p's
// histogram of sequence b: the bin, counted from the top, in which the
// k_rem-th largest matching key falls.  Called by the whole block; thread i
// reads the i-th run of NB / kThreads bins from the top.
template <int P>
__device__ Prefix extend_prefix(const IndexArgs &a, int b, Prefix x) {
  constexpr int NB = 1 << digit_bits(P), M = NB / kThreads;
  __shared__ int wtot[kThreads / 64];
  __shared__ Prefix px;
  const int tid = threadIdx.x;
  const uint32_t *hist = hist_of(a, P, b) + NB - (tid + 1) * M;  // bins [NB - (tid+1)M, NB - tid M)
  uint32_t c[M];
  if constexpr (M % 4 == 0) {
#pragma unroll
    for (int i = 0; i < M / 4; ++i) {
      const uint4 v = reinterpret_cast<const uint4 *>(hist)[i];
      c[4 * i] = v.x;
      c[4 * i + 1] = v.y;
      c[4 * i + 2] = v.z;
      c[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < M; ++i) c[i] = hist[i];
  }
  int sum = 0;
#pragma unroll
  for (int i = 0; i < M; ++i) sum += static_cast<int>(c[i]);
  if (tid == 0) px = Prefix{x.bits << digit_bits(P), x.k_rem};  // kept only if no bin matches
  int tot;
  const int above = block_excl_scan(sum, wtot, &tot);
  if (above < x.k_rem && above + sum >= x.k_rem) {
    int run = above;
#pragma unroll
    for (int i = M - 1; i >= 0; --i) {  // descending bins
      const int ci = static_cast<int>(c[i]);
      if (run < x.k_rem && run + ci >= x.k_rem) {
        px.bits = (x.bits << digit_bits(P)) | static_cast<uint32_t>(NB - (tid + 1) * M + i);
        px.k_rem = x.k_rem - run;
      }
      run += ci;
    }
  }
  __syncthreads();
  const Prefix r = px;
  __syncthreads();  // px is rewritten by a later call
  return r;
}

// Prefix after passes 0..P-1: pass 0 needs nothing; later ones read what the
// previous launch stored for sequence b.
template <int P>
__device__ __forceinline__ Prefix stored_prefix(const IndexArgs &a, int b) {
  if constexpr (P == 0) {
    return Prefix{0u, a.top_k};
  } else {
    return Prefix{a.pfx_bits[(P - 1) * a.B + b], a.pfx_rank[(P - 1) * a.B + b]};
  }
}

// Chunk c of sequence b: tokens [c * cl, (c + 1) * cl), cl = ceil(L /
// n_chunks).  A group is kUnroll * kThreads consecutive tokens; thread i
// holds tokens g + kUnroll i + u, u < kUnroll (contiguous per thread, so a
// block-wide scan of per-thread counts follows token order).  Loads are
// clamped to the chunk, so none is predicated; the caller never loads from
// an empty chunk.
constexpr int kUnroll = 4;
constexpr int kGroup = kUnroll * kThreads;

__device__ __forceinline__ void chunk_range(int L, int n_chunks, int c, int *t0, int *t1) {
  const int cl = (L + n_chunks - 1) / n_chunks;
  *t0 = min(L, c * cl);
  *t1 = min(L, *t0 + cl);
}

__device__ __forceinline__ void load_group(const float *scores, int64_t base, int g, int t1, uint32_t key[kUnroll]) {
  const int t = g + kUnroll * static_cast<int>(threadIdx.x);
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) key[u] = ordered_bits(scores[base + min(t + u, t1 - 1)]);
}

// Radix pass P (1 .. kPasses-1) over chunk blockIdx.y of sequence blockIdx.x:
// histogram of digit P over the keys that match the prefix.  The last pass
// also stores the chunk's count of keys above the prefix and the suffix sums
// of its own histogram.
template <int P>
__global__ __launch_bounds__(kThreads) void radix_pass_kernel(IndexArgs a) {
  constexpr int NB = 1 << digit_bits(P);
  constexpr bool kLast = P == kPasses - 1;
  __shared__ uint32_t h[NB];
  __shared__ int wtot[kThreads / 64];
  const int b = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
  const int L = a.seq_len[b];
  if (L <= a.top_k) return;  // everything is selected
  const int64_t base = a.seq_base[b];
  int t0, t1;
  chunk_range(L, a.n_chunks, c, &t0, &t1);
  uint32_t key[kUnroll];
  if (t0 < t1) load_group(a.scores, base, t0, t1, key);  // in flight while the prefix is derived
#pragma unroll
  for (int i = 0; i < NB / kThreads; ++i) h[i * kThreads + tid] = 0u;
  const Prefix pre = extend_prefix<P - 1>(a, b, stored_prefix<P - 1>(a, b));
  if (c == 0 && tid == 0) {
    a.pfx_bits[(P - 1) * a.B + b] = pre.bits;
    a.pfx_rank[(P - 1) * a.B + b] = pre.k_rem;
  }
  constexpr int kShift = digit_shift(P);
  int above = 0;
  for (int g = t0; g < t1; g += kGroup) {
    if (g != t0) load_group(a.scores, base, g, t1, key);
    const int t = g + kUnroll * tid;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t hi = key[u] >> (kShift + digit_bits(P));
      if (t + u < t1 && hi == pre.bits) atomicAdd(&h[(key[u] >> kShift) & (NB - 1)], 1u);
      if (kLast) above += (t + u < t1 && hi > pre.bits) ? 1 : 0;
    }
  }
  __syncthreads();
  flush_hist<NB>(h, hist_of(a, P, b));
  if constexpr (kLast) {
    // thread i: bin NB-1-i; inclusive count of the chunk's matching keys in bins >= it
    const int own = static_cast<int>(h[NB - 1 - tid]);
    int tot;
    const int excl = block_excl_scan(own, wtot, &tot);
    const int64_t row = static_cast<int64_t>(b) * a.n_chunks + c;
    a.chunk_suf[row * NB + NB - 1 - tid] = excl + own;
    block_excl_scan(above, wtot, &tot);
    if (tid == 0) a.chunk_above[row] = tot;
  }
}

// Write pass: each chunk writes its selected tokens, in token order, after
// those of the chunks before it.  A token is selected if its key is above
// the threshold key T, or equal to T with fewer than k_eq tokens equal to T
// before it; the selected tokens before a token number (keys above T before
// it) + min(keys equal to T before it, k_eq).  Block (b, 0) writes n_sel[b].
__global__ __launch_bounds__(kThreads) void select_write_kernel(IndexArgs a) {
  constexpr int P = kPasses - 1;
  __shared__ int wtot[kThreads / 64];
  const int b = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
  const int L = a.seq_len[b];
  const bool all = L <= a.top_k;
  const int64_t base = a.seq_base[b];
  int t0, t1;
  chunk_range(L, a.n_chunks, c, &t0, &t1);
  uint32_t key[kUnroll];
  if (t0 < t1) load_group(a.scores, base, t0, t1, key);
  if (c == 0 && tid == 0) a.n_sel[b] = min(L, a.top_k);
  uint32_t thr = 0u;
  int k_eq = 0, gt_run = t0, eq_run = 0;  // every token before the chunk is selected when all
  if (!all) {  // uniform over the block
    const Prefix pre = extend_prefix<P>(a, b, stored_prefix<P>(a, b));
    thr = pre.bits;
    k_eq = pre.k_rem;
    // tokens of the chunks before this one above and equal to T (n_chunks <= kThreads)
    const int d = static_cast<int>(thr & (kLastBins - 1));
    int gt_j = 0, eq_j = 0;
    if (tid < c) {
      const int64_t row = static_cast<int64_t>(b) * a.n_chunks + tid;
      const int s_d = a.chunk_suf[row * kLastBins + d];
      const int s_up = d + 1 < kLastBins ? a.chunk_suf[row * kLastBins + d + 1] : 0;
      gt_j = a.chunk_above[row] + s_up;
      eq_j = s_d - s_up;
    }
    block_excl_scan(gt_j, wtot, &gt_run);
    block_excl_scan(eq_j, wtot, &eq_run);
  }
  int32_t *out = a.sel + static_cast<int64_t>(b) * a.top_k;
  for (int g = t0; g < t1; g += kGroup) {
    if (g != t0) load_group(a.scores, base, g, t1, key);
    const int t = g + kUnroll * tid;
    int n_gt = 0, n_eq = 0;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      n_gt += (t + u < t1 && (all || key[u] > thr)) ? 1 : 0;
      n_eq += (t + u < t1 && !all && key[u] == thr) ? 1 : 0;
    }
    int tot;  // per group both counts are at most kGroup < 2^16: one packed scan
    const int before = block_excl_scan(n_gt | (n_eq << 16), wtot, &tot);
    int gb = gt_run + (before & 0xffff), eb = eq_run + (before >> 16);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (t + u >= t1) break;
      if (all || key[u] > thr) {
        const int idx = gb + min(eb, k_eq);  // eb = k_eq = 0 when all
        if (idx < a.top_k) out[idx] = t + u;
        ++gb;
      } else if (key[u] == thr) {
        if (eb < k_eq && gb + eb < a.top_k) out[gb + eb] = t + u;
        ++eb;
      }
    }
    gt_run += tot & 0xffff;
    eq_run += tot >> 16;
  }
}

}  // namespace

int index_chunks() { return kThreads; }
int index_hist_bins() { return kHistBins; }
int index_passes() { return kPasses; }
int index_last_bins() { return kLastBins; }

hipError_t launch_index_topk(const IndexArgs &a, hipStream_t s) {
  const dim3 chunks(a.B, a.n_chunks);
  {
    TimedLaunch tl("index_score", s);
    index_clear_kernel<<<dim3(a.B, kPasses), kThreads, 0, s>>>(a);
    // the score kernel's blocks stride over their sequence: two per compute
    // unit over the batch measured fastest (more, at its register use, run
    // in a second round; fewer hold fewer loads in flight)
    const dim3 score_grid(a.B, std::min(a.n_chunks, std::max(1, 2 * device_cu_count() / std::max(1, a.B))));
    switch (a.d_idx) {
      case 64: index_score_kernel<64><<<score_grid, kThreads, 0, s>>>(a); break;
      case 128: index_score_kernel<128><<<score_grid, kThreads, 0, s>>>(a); break;
      default: return hipErrorInvalidValue;
    }
  }
  TimedLaunch tl("index_select", s);
  radix_pass_kernel<1><<<chunks, kThreads, 0, s>>>(a);
  radix_pass_kernel<2><<<chunks, kThreads, 0, s>>>(a);
  select_write_kernel<<<chunks, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
