// Split-K work planner shared by the decode translation units.
#pragma once

#include "kernels.hpp"

namespace mla {

__device__ inline long long plan_wave_sum(long long x) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ inline int plan_wave_incl_scan(int x, int lane) {
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// Token-balanced split-K plan from device seq_len (no host synchronisation),
// run by one whole block of 256 threads.
// Chunk length C = round_up(ceil(total / target), tile); sequence b gets
// ceil(L_b / C) items of equal length (rounded up to the tile).  The item
// count is then at most target + B = max_items.
__device__ inline void plan_block(const int32_t *__restrict__ seq_len, int B, int target, int tile,
                                  int max_items, WorkItem *__restrict__ items,
                                  int32_t *__restrict__ item_begin, int32_t *__restrict__ meta) {
  // called by one whole block of 256 threads
  __shared__ long long wsum[4];
  __shared__ int32_t wtot[4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int L0 = tid < B ? seq_len[tid] : 0;
  long long tot = max(0, L0);
  for (int b = tid + 256; b < B; b += 256) tot += max(0, seq_len[b]);
  tot = plan_wave_sum(tot);
  if (lane == 0) wsum[wv] = tot;
  __syncthreads();
  const long long total = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  long long C = (total + target - 1) / max(target, 1);
  C = ((C + tile - 1) / tile) * tile;
  if (C < tile) C = tile;
  int carry = 0;
  for (int base = 0; base < B; base += 256) {
    const int b = base + tid;
    int nb = 0, chunk = 0;
    const int L = base == 0 ? L0 : (b < B ? seq_len[b] : 0);
    if (L > 0) {
      nb = static_cast<int>((L + C - 1) / C);
      chunk = (L + nb - 1) / nb;
      chunk = ((chunk + tile - 1) / tile) * tile;
      nb = (L + chunk - 1) / chunk;
    }
    const int inc = plan_wave_incl_scan(nb, lane);
    if (lane == 63) wtot[wv] = inc;
    __syncthreads();
    int before = 0;
    for (int j = 0; j < wv; ++j) before += wtot[j];
    const int excl = carry + before + inc - nb;
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
    carry += (wtot[0] + wtot[1]) + (wtot[2] + wtot[3]);
    __syncthreads();  // wtot is rewritten by the next group
  }
  if (tid == 0) {
    const int n = min(carry, max_items);
    item_begin[B] = n;
    meta[0] = n;
    meta[1] = static_cast<int32_t>(C);
  }
}

}  // namespace mla
