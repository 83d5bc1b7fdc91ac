// Split-K work planner shared by the decode translation units.
#pragma once

#include "kernels.hpp"

namespace mla {

__device__ inline int plan_wave_incl_scan(int x, int lane) {
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// Token-balanced split-K plan from device seq_len (no host synchronisation),
// run by one whole block of 256 threads.  A chunk length C (a multiple of
// the tile) gives sequence b nb(L_b, C) items of equal length: nb =
// ceil(L_b / C), the chunk rounded up to the tile, nb recomputed from it.
// The item count is non-increasing in C; the planner takes the smallest C
// whose count fits `target` (the work-item slots that fill the GPU), so the
// grid is as full as the lengths allow, or one item per sequence when even
// that exceeds target.  C is at least min_k tiles (or the longest
// sequence), so an item holds more than half of that, a sequence's last item
// aside: an item has a fixed cost (its query rows in, its partial rows out)
// that one or two tiles of tokens do not repay.  max_items bounds the count
// and the item array.
__device__ inline int plan_items_of(int L, int C, int tile, int *chunk_out) {
  if (L <= 0) {
    *chunk_out = 0;
    return 0;
  }
  int nb = (L + C - 1) / C;
  int chunk = (L + nb - 1) / nb;
  chunk = ((chunk + tile - 1) / tile) * tile;
  *chunk_out = chunk;
  return (L + chunk - 1) / chunk;
}

// rep > 1: B pseudo-sequences, pseudo-sequence b having the length of
// sequence b / rep (a sequence's KV heads in grouped-query decode).
__device__ inline void plan_block(const int32_t *__restrict__ seq_len, int B, int target, int tile,
                                  int min_k, int max_items, WorkItem *__restrict__ items,
                                  int32_t *__restrict__ item_begin, int32_t *__restrict__ meta, int rep = 1) {
  // called by one whole block of 256 threads
  __shared__ long long wsum[4];
  __shared__ int32_t wne[4], wmax[4], wred[4];
  __shared__ int32_t wtot[4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int L0 = tid < B ? seq_len[tid / rep] : 0;
  auto len_of = [&](int b) -> int { return b < 256 ? L0 : seq_len[b / rep]; };
  // totals: tokens, non-empty sequences, longest sequence (one barrier pair)
  long long tot = 0;
  int ne = 0, lmax = 0;
  for (int b = tid; b < B; b += 256) {
    const int L = max(0, len_of(b));
    tot += L;
    ne += L > 0;
    lmax = max(lmax, L);
  }
  for (int off = 32; off > 0; off >>= 1) {
    tot += __shfl_xor(tot, off);
    ne += __shfl_xor(ne, off);
    lmax = max(lmax, __shfl_xor(lmax, off));
  }
  if (lane == 0) {
    wsum[wv] = tot;
    wne[wv] = ne;
    wmax[wv] = lmax;
  }
  __syncthreads();
  const long long total = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  const int nonempty = (wne[0] + wne[1]) + (wne[2] + wne[3]);
  lmax = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  // item count at C = k * tile (block-wide sum, two barriers)
  auto count = [&](int k) -> int {
    int chunk, n = 0;
    for (int b = tid; b < B; b += 256) n += plan_items_of(len_of(b), k * tile, tile, &chunk);
    for (int off = 32; off > 0; off >>= 1) n += __shfl_xor(n, off);
    __syncthreads();  // wred may still be read from the previous call
    if (lane == 0) wred[wv] = n;
    __syncthreads();
    return (wred[0] + wred[1]) + (wred[2] + wred[3]);
  };
  // count(C) >= total / C, so C >= total / target; and every chunk is at
  // most C, so count(C) <= total / C + nonempty, which fits target once
  // C >= total / (target - nonempty).  Search the smallest fitting k between.
  const long long T = target;
  const int khi = max(1, (lmax + tile - 1) / tile);  // one item per sequence
  int lo, hi;
  if (T <= nonempty) {
    lo = hi = khi;
  } else {
    const long long per_lo = T * tile, per_hi = (T - nonempty) * tile;
    lo = static_cast<int>(min<long long>(khi, max<long long>(1, (total + per_lo - 1) / per_lo)));
    hi = static_cast<int>(min<long long>(khi, max<long long>(lo, (total + per_hi - 1) / per_hi)));
    lo = max(lo, min(khi, min_k));
    hi = max(hi, lo);
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (count(mid) <= target)
        hi = mid;
      else
        lo = mid + 1;
    }
  }
  const int C = lo * tile;
  // Items, 256 sequences at a time: thread b finds its sequence's item count
  // and first item (a block-wide scan) and leaves them in LDS; then wave wv
  // writes the items of sequences wv, wv + 4, ... of the group, its 64 lanes
  // the consecutive items of one sequence (one thread writing a sequence's
  // items in a loop took most of the planner's time).  Lane l fetches the
  // values of the wave's sequence l of the group up front; the loop takes
  // them from the lanes (readlane), not from LDS.
  __shared__ int32_t s_first[256], s_count[256], s_chunk[256], s_len[256];
  int carry = 0;
  for (int base = 0; base < B; base += 256) {
    const int b = base + tid;
    const int L = b < B ? len_of(b) : 0;
    int chunk;
    const int nb = plan_items_of(L, C, tile, &chunk);
    const int inc = plan_wave_incl_scan(nb, lane);
    if (lane == 63) wtot[wv] = inc;
    __syncthreads();
    int before = 0;
    for (int j = 0; j < wv; ++j) before += wtot[j];
    const int excl = carry + before + inc - nb;
    s_first[tid] = excl;
    s_count[tid] = nb;
    s_chunk[tid] = chunk;
    s_len[tid] = L;
    if (b < B) item_begin[b] = min(excl, max_items);
    __syncthreads();
    const int cnt = min(256, B - base), nw = (cnt - wv + 3) / 4;  // the wave's sequences: wv + 4k, k < nw
    const int jl = min(wv + 4 * lane, 255);
    const int f_l = s_first[jl], n_l = s_count[jl], ch_l = s_chunk[jl], len_l = s_len[jl];
    for (int k = 0; k < nw; ++k) {
      const int first = __builtin_amdgcn_readlane(f_l, k), n = __builtin_amdgcn_readlane(n_l, k);
      const int ch = __builtin_amdgcn_readlane(ch_l, k), Lj = __builtin_amdgcn_readlane(len_l, k);
      for (int c = lane; c < n; c += 64) {
        const int idx = first + c;
        if (idx < max_items) {
          WorkItem it;
          it.b = base + wv + 4 * k;
          it.t0 = c * ch;
          it.t1 = min(Lj, (c + 1) * ch);
          it.pad = 0;
          items[idx] = it;
        }
      }
    }
    carry += (wtot[0] + wtot[1]) + (wtot[2] + wtot[3]);
    __syncthreads();  // wtot and the per-sequence arrays are rewritten by the next group
  }
  if (tid == 0) {
    const int n = min(carry, max_items);
    item_begin[B] = n;
    meta[0] = n;
    meta[1] = C;
  }
}

}  // namespace mla
