// MFMA kernels of the absorbed decode around the split-K kernel, for r = 512,
// d_r = 64 (DeepSeek-V3 / GLM-5.3-style MLA layers), and the grouped-query
// split-K kernel, on gfx950.
//
// [shard PR #5, TL;DR item 2]: attention runs in latent space over the cached
// latent plus one shared rope key: each query's nope part is absorbed into
// latent space through the folded W_UK (q~ = W~_UK^T q_nope) before the
// split-K pass (splitk.hip), which consumes q~ in the operand order this
// file writes.
#include "append_tile.hpp"
#include "plan.hpp"
#include "splitk_tile.hpp"

namespace mla {
namespace {

// q~ = W~_UK[h]^T q_nope on MFMA (32x32x16 f16, fp32 acc), and q_rope; both
// times scale*log2(e), written in fp16 straight into the per-lane operand
// order of the split-K kernel's producers: [b][row block][wave][mt][kb][lane][8], zero
// for padding rows.  Block = (head, latent quarter = split-K wave slot,
// 32 query rows (b, t)); wave w computes 32 channels.  The results are staged
// in LDS so every operand unit (8 halves) is written with one 16-byte store.
// One extra block runs the split-K planner.  w_uk_f is stored [H][r][d_n].
__device__ __forceinline__ int64_t qpos(int rb_count, int b, int m, int w, int hf, int kb) {
  const int rb = m / ROWS, mt = (m % ROWS) / 32, lane = (m % 32) + 32 * hf;
  return ((((static_cast<int64_t>(b) * rb_count + rb) * 4 + w) * 2 + mt) * KB + kb) * 512 + lane * 8;
}

constexpr int QTSTRIDE = 136;  // halves per staged row (128 channels + pad)

// Query absorb (q~ = W~_UK^T q_nope per head, in split-K operand order), the
// split-K planner (block (0, 0)), and optionally a decode step's small append
// (columns 1 .. x0 - 1, dispatched right after the planner so its memory
// round trip overlaps the absorb): per 32-token tile one block per 32-channel
// tile (staged_skinny_tile: the latent rows staged in LDS, wave 0 computes;
// the same MFMA sequence as the stand-alone append kernels, so the cache
// bytes are identical), then one block for the tile's side keys (rope keys
// copied or quantised to 4 bits, indexer keys).  The absorb blocks are the
// columns from x0 on.
template <int G>  // INT2 group size of the fused append (0: no append)
__global__ __launch_bounds__(256) void absorb_mfma_kernel(DecodeArgs a, int rb_count, AppendParams ap, int x0) {
  __shared__ __align__(16) f16 qt[32 * QTSTRIDE];
  // the quarter's 128 W~_UK rows, 128 values of the contraction at a time;
  // 16-byte piece p of row j sits at piece p ^ (j & 15) (conflict-free
  // operand reads by 16 consecutive lanes)
  __shared__ __align__(16) u32x4 wk[128 * 16];
  const int H = a.d.num_heads, dn = a.d.qk_nope_head_dim;
  // the extra first block column: block (0, 0) plans the split-K work in
  // parallel with the absorb blocks (and is dispatched first), the rest of
  // that column has nothing to do
  if (blockIdx.x == 0) {
    if (blockIdx.y == 0)
      plan_block(a.seq_len, a.B, a.target_items, a.tile, a.min_chunk_tiles, a.max_items, a.items, a.item_begin,
                 a.meta);
    return;
  }
  if constexpr (G != 0) {
    if (static_cast<int>(blockIdx.x) < x0) {
      // append blocks: tiles (ct = blk % (R / 32), ty = blk / (R / 32)), then
      // the side-key blocks (token tile blk - n_tiles R / 32)
      const int blk = (blockIdx.x - 1) * gridDim.y + blockIdx.y;
      const int n_tiles = static_cast<int>((ap.n + 31) / 32);
      if (blk < n_tiles * (R / 32)) {
        staged_skinny_tile<R, G, 2>(ap, blk % (R / 32), blk / (R / 32), threadIdx.x, wk);
      } else if (blk < n_tiles * (R / 32 + 1)) {
        side_key_block(ap, blk - n_tiles * (R / 32), threadIdx.x);
      }
      return;
    }
  }
  const int h = (blockIdx.x - x0) >> 2, cq = (blockIdx.x - x0) & 3, rt = blockIdx.y;
  const int M = H * a.Tq;
  const int nrows = a.B * a.Tq;
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6, hf = l >> 5, l32 = l & 31;
  f16 *qb = static_cast<f16 *>(a.qbuf);
  const int q = rt * 32 + l32;
  const bool q_ok = q < nrows;
  const uint16_t *arow = a.q_nope + (static_cast<int64_t>(q_ok ? q : 0) * H + h) * dn;
  // coalesced weight rows: thread tid moves piece tid & 15 of rows (tid >> 4) + 16i
  const uint16_t *wbase = a.w_uk_f + (static_cast<int64_t>(h) * R + 128 * cq) * dn;
  const int wp = tid & 15, wr0 = tid >> 4;
  const int brow = 32 * w + l32;  // this lane's B column = latent channel 128cq + brow
  f32x16 acc = {};
  for (int k0 = 0; k0 < dn; k0 += 128) {
    const int kc = min(128, dn - k0);  // a multiple of 16
    u32x4 wv[8];
    u32x4 raw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      wv[i] = *reinterpret_cast<const u32x4 *>(wbase + static_cast<int64_t>(wr0 + 16 * i) * dn + k0 + 8 * min(wp, kc / 8 - 1));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int kk = k0 + min(16 * e, kc - 16) + 8 * hf;
      raw[e] = *reinterpret_cast<const u32x4 *>(arow + kk);  // row 0 stands in for q >= nrows
    }
    if (k0 > 0) __syncthreads();  // the previous chunk's operand reads are done
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = wr0 + 16 * i;
      wk[j * 16 + (wp ^ (j & 15))] = wv[i];
    }
    __syncthreads();
    // K-steps past the chunk (kc < 128) repeat its last step with a zero
    // query operand, so every step reads written, finite weights
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int ee = min(e, kc / 16 - 1);
      const bool use = q_ok && e == ee;
      const u32x4 bw = wk[brow * 16 + ((2 * ee + hf) ^ (brow & 15))];
      const f16x8 bv = __builtin_bit_cast(f16x8, bw);
      const u32x4 rr = raw[e];
      f16x8 av;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        av[2 * j] = use ? static_cast<f16>(__uint_as_float(rr[j] << 16)) : f16(0.0f);
        av[2 * j + 1] = use ? static_cast<f16>(__uint_as_float(rr[j] & 0xffff0000u)) : f16(0.0f);
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, acc, 0, 0, 0);
    }
  }
  // C layout: column = channel 32w + l32 of the quarter, rows 8(v/4) + 4hf + v%4
#pragma unroll
  for (int v = 0; v < 16; ++v)
    qt[(8 * (v >> 2) + 4 * hf + (v & 3)) * QTSTRIDE + 32 * w + l32] = static_cast<f16>(acc[v] * a.scale_log2);
  __syncthreads();
  // operand units: (row i, lane half uh, K-block kb) -> 8 channels slot_channel(uh, kb, e)
  for (int u = tid; u < 32 * 16; u += 256) {
    const int i = u >> 4, uh = (u >> 3) & 1, kb = u & 7;
    const int qq = rt * 32 + i;
    if (qq >= nrows) continue;
    f16x8 v8;
#pragma unroll
    for (int e = 0; e < 8; ++e) v8[e] = qt[i * QTSTRIDE + slot_channel(uh, kb, e)];
    const int b = qq / a.Tq, t = qq % a.Tq, m = t * H + h;
    *reinterpret_cast<f16x8 *>(qb + qpos(rb_count, b, m, cq, uh, kb)) = v8;
  }
  // rope units: dims 16cq + 8uh + e
  if (tid < 64) {
    const int i = tid >> 1, uh = tid & 1, qq = rt * 32 + i;
    if (qq < nrows) {
      const uint4 raw = *reinterpret_cast<const uint4 *>(a.q_rope + (static_cast<int64_t>(qq) * H + h) * DR + 16 * cq + 8 * uh);
      const uint32_t rr[4] = {raw.x, raw.y, raw.z, raw.w};
      f16x8 v8;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v8[2 * e] = static_cast<f16>(__uint_as_float(rr[e] << 16) * a.scale_log2);
        v8[2 * e + 1] = static_cast<f16>(__uint_as_float(rr[e] & 0xffff0000u) * a.scale_log2);
      }
      const int b = qq / a.Tq, t = qq % a.Tq, m = t * H + h;
      *reinterpret_cast<f16x8 *>(qb + qpos(rb_count, b, m, cq, uh, 8)) = v8;
    }
  }
  // zero the padding rows of the last row block for this wave slot
  if (h == 0 && rt == 0 && M % ROWS != 0) {
    const int pad = rb_count * ROWS - M;
    const f16x8 z8 = {};
    for (int e = tid; e < a.B * pad * 2 * KB; e += 256) {
      const int b = e / (pad * 2 * KB), rest = e % (pad * 2 * KB);
      const int m = M + rest / (2 * KB), uh = (rest / KB) & 1, kb = rest % KB;
      *reinterpret_cast<f16x8 *>(qb + qpos(rb_count, b, m, cq, uh, kb)) = z8;
    }
  }
}

// ---- grouped-query layers (head dim 128): one wave per work item ----
// The same tile machinery for a KV head of a grouped-query layer, whose
// head dim (128) is one wave's share of the latent above: a work item is a
// token range of one (sequence, KV head) pseudo-sequence, its G * Tq query
// rows (at most 32) are the N side of the score MFMA, and the K and V tiles
// come from their own caches.  One wave per workgroup and no cross-wave
// reduction, so the loop needs no barrier: per 32-token tile the wave
// dequantises K into score operands and V into its LDS tile, takes the scores
// (8 MFMAs), runs the online softmax (a row's 32 tokens on lanes l and l ^ 32),
// stages P in LDS and accumulates O += P V_hat (8 MFMAs, V_hat through the
// transposing load).  Channels travel in the slot order of the latent kernel;
// the rotated queries are gathered into it and the partial un-permuted.
constexpr int GQ_D = 128;
constexpr int GQ_ROWS = 32;

struct __align__(16) GqaSmem {
  f16 z[TT * ZSTRIDE];         // dequantised V tile [token][slot]
  f16 p[GQ_ROWS * PRSTRIDE];   // P [row][token]
  float alpha[GQ_ROWS];
  float inv_l[GQ_ROWS];
};

// o_settle for the four output accumulators of the grouped-query kernel.
// The hardware does not interlock a register an MFMA is still writing
// against a later non-MFMA read, and the compiler does not see into inline
// asm, so the rescale's asm must first wait out the MFMA write -> read
// latency itself (24 wait states cover an 8-pass MFMA with margin), and the
// next MFMA must not read what the asm wrote before it lands.  Taking the
// accumulator tuples as operands orders this after their last MFMA and
// every asm access to them after this.
template <bool kAfterMfma>
__device__ __forceinline__ void gqa_o_settle(f32x16 (&o)[4]) {
  if (kAfterMfma)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]));
  else
    asm volatile("s_nop 4" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]));
}

template <int G>
__device__ __forceinline__ RawTile gqa_load(const mla_cache &c, int64_t slot, int hf) {
  RawTile t;
  const uint32_t *codes32 = reinterpret_cast<const uint32_t *>(c.codes);
  t.codes = *reinterpret_cast<const uint4 *>(codes32 + slot * (GQ_D / 16) + hf * 4);
  if (G == 32) {
    const uint2 s2 = *reinterpret_cast<const uint2 *>(c.scale_zero + (slot * (GQ_D / G) + 2 * hf) * 2);
    t.sz = uint4{s2.x, s2.y, 0u, 0u};
  } else {
    t.sz = *reinterpret_cast<const uint4 *>(c.scale_zero + (slot * (GQ_D / G) + 4 * hf) * 2);
  }
  t.rope = uint4{0u, 0u, 0u, 0u};
  return t;
}

template <int G>
__global__ __launch_bounds__(64) void gqa_splitk_mfma_kernel(DecodeArgs a) {
  __shared__ GqaSmem sm;
  const int item = blockIdx.x;
  if (item >= a.meta[0]) return;
  const WorkItem it = a.items[item];
  const int l = threadIdx.x, hf = l >> 5, l32 = l & 31;
  const int Gq = a.d.num_heads;  // query heads per KV head
  const int M = Gq * a.Tq;
  const int L = a.seq_len[it.b];
  const int64_t base = a.seq_base[it.b];
  const int n_tiles = (it.t1 - it.t0 + TT - 1) / TT;

  // rotated queries of row l32 as score B operands, gathered into slot order
  f16x8 aq[KB];
  {
    const float *qr = static_cast<const float *>(a.qbuf) + (static_cast<int64_t>(it.b) * M + min(l32, M - 1)) * GQ_D;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) {  // (row pointer clamped: loads without a branch)
        const float x = qr[slot_channel(hf, kb, e)];
        aq[kb][e] = static_cast<f16>(l32 < M ? x : 0.0f);
      }
  }
  // softmax ownership: row l32, tokens 8 j + 4 hf + i (j, i < 4) of each tile
  const int vis = l32 < M ? (a.causal ? (L - a.Tq + l32 / Gq + 1) : L) : -1;
  const int lim = min(it.t1, vis);  // tokens < lim are visible to this row
  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 o[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) o[nt] = f32x16{};

  const int g16 = l >> 4, s16 = l & 15;
  const int pv_krow = 8 * (g16 >> 1) + (s16 >> 2);
  const int pv_col = (16 * (g16 & 1) + 4 * (s16 & 3)) ^ (8 * ((g16 >> 1) & 1));
  // 16-byte chunk c of Z row t at chunk c ^ ((t >> 3) & 1): rows t and t + 8
  // would otherwise take the same banks in one 16-lane store group
  const int zsw = 8 * ((l32 >> 3) & 1);
  auto tile_slot = [&](int i) -> int64_t {
    const int t = min(it.t0 + min(i, n_tiles - 1) * TT + l32, it.t1 - 1);
    return base + t;
  };
  RawTile rk = gqa_load<G>(a.cache, tile_slot(0), hf);
  RawTile rv = gqa_load<G>(a.vcache, tile_slot(0), hf);
  for (int i = 0; i < n_tiles; ++i) {
    // LDS is handed between lanes of this one wave: the previous tile's
    // reads of P and the V tile stay above this tile's stores
    __builtin_amdgcn_wave_barrier();
    // K operands, the next K tile in flight, the scores; then V into the
    // same registers, the next V tile in flight, V to LDS (short live ranges
    // keep two waves per SIMD)
    f32x16 sacc = f32x16{};
    {
      f16x8 bk[KB];
      dequant<G>(rk, bk);
      rk = gqa_load<G>(a.cache, tile_slot(i + 1), hf);
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(bk[kb], aq[kb], sacc, 0, 0, 0);
    }
    {
      f16x8 bv[KB];
      dequant<G>(rv, bv);
      rv = gqa_load<G>(a.vcache, tile_slot(i + 1), hf);
      // V tile to LDS (this wave's only), chunk kb ^ 1 in rows 8..15 and 24..31
      f16 *zt = sm.z + l32 * ZSTRIDE + 64 * hf;
      f16 *ze = zt + zsw, *zo = zt - zsw;
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) *reinterpret_cast<f16x8 *>(((kb & 1) ? zo : ze) + 8 * kb) = bv[kb];
    }
    // online softmax of row l32 over this tile's tokens 8 j + 4 hf + i
    const int t_first = it.t0 + i * TT + 4 * hf;
    float s[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) s[v] = (t_first + 8 * (v >> 2) + (v & 3) < lim) ? sacc[v] : -INFINITY;
    float tmax = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, s[v]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const bool need = tmax > m_run + kRescaleThreshold;
    const float alpha = need ? __builtin_amdgcn_exp2f(m_run - tmax) : 1.0f;
    const bool scale_o = need && m_run != -INFINITY;  // O is still zero before the first visible tile
    m_run = need ? tmax : m_run;
    const float m_sub = (m_run == -INFINITY) ? 0.0f : m_run;
    float psum = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f16x4 pv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pe = __builtin_amdgcn_exp2f(s[4 * j + e] - m_sub);
        psum += pe;
        pv[e] = static_cast<f16>(pe);
      }
      *reinterpret_cast<f16x4 *>(sm.p + l32 * PRSTRIDE + 8 * j + 4 * hf) = pv;
    }
    psum += __shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    if (hf == 0) sm.alpha[l32] = alpha;
    __builtin_amdgcn_wave_barrier();  // V tile, P and alpha stored before other lanes read them
    if (__any(scale_o ? 1 : 0)) {  // in place in the accumulator registers
      gqa_o_settle<true>(o);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float al = sm.alpha[8 * (v >> 2) + 4 * hf + (v & 3)];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          float x = o[nt][v];
          agpr_scale(x, al);
          o[nt][v] = x;
        }
      }
      gqa_o_settle<false>(o);
    }
    // O += P V_hat
    const f16 *zb_base = sm.z + pv_krow * ZSTRIDE + pv_col;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const f16x8 pa = *reinterpret_cast<const f16x8 *>(sm.p + l32 * PRSTRIDE + 16 * ks + 8 * hf);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const f16 *z0 = zb_base + 16 * ks * ZSTRIDE + 32 * nt;
        const f16x4 lo = ds_read_tr16(z0);
        const f16x4 hi = ds_read_tr16(z0 + 4 * ZSTRIDE);
        const f16x8 zb = f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa, zb, o[nt], 0, 0, 0);
      }
    }
  }
  // partial: O / l in fp16 (rows 8 (v / 4) + 4 hf + v % 4, slot 32 nt + l32), (m, l)
  if (hf == 0) sm.inv_l[l32] = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  __builtin_amdgcn_wave_barrier();
  f16 *po = reinterpret_cast<f16 *>(a.part_o);
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int sl = 32 * nt + l32;
    const int ch = slot_channel(sl >> 6, (sl & 63) >> 3, sl & 7);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = 8 * (v >> 2) + 4 * hf + (v & 3);
      if (m < M) po[(static_cast<int64_t>(item) * M + m) * GQ_D + ch] = static_cast<f16>(o[nt][v] * sm.inv_l[m]);
    }
  }
  if (hf == 0 && l32 < M) {
    a.part_ml[(static_cast<int64_t>(item) * M + l32) * 2 + 0] = m_run;
    a.part_ml[(static_cast<int64_t>(item) * M + l32) * 2 + 1] = l_run;
  }
}

// ---- grouped-query layers with at most 16 query rows per KV head ----
// One wave per work item, 16-token chunks, no LDS shared between waves, so
// a wave needs about 100 registers and several share a SIMD:
//   lane (token n = l & 15, quarter g = l >> 4) holds dims 32g .. 32g + 31
//   of token n's K and V entries (8 code bytes and the groups' (scale,
//   zero) each), the next chunk's in flight;
//   scores S^T[16 tokens x 16 rows] = K_hat Q^T: 4 v_mfma_f32_16x16x32_f16,
//   K-step kb taking the eight dims 32g + slot_channel(0, kb, e) of each
//   lane's quarter (dequant_block's order), the rotated queries gathered
//   into the same order once per item;
//   the score lanes hold P^T in the layout of the next product's B operand;
//   O^T[128 x 16 rows] += V_hat^T P^T: 8 v_mfma_f32_16x16x16_f16, V_hat^T
//   read with ds_read_b64_tr_b16 from the wave's LDS copy of the chunk.
// The partial (O / l fp16, m, l) goes out through the same LDS tile.
constexpr int GQ16_ZS = GQ_D + 16;  // halves per V tile row

template <int G>
__device__ __forceinline__ RawTile gqa16_load(const mla_cache &c, int64_t slot, int g) {
  RawTile t;
  const uint2 cw = *reinterpret_cast<const uint2 *>(c.codes + slot * (GQ_D / 4) + 8 * g);
  t.codes = uint4{cw.x, cw.y, 0u, 0u};
  if (G == 32) {
    t.sz = uint4{*reinterpret_cast<const uint32_t *>(c.scale_zero + (slot * (GQ_D / G) + g) * 2), 0u, 0u, 0u};
  } else {
    const uint2 s2 = *reinterpret_cast<const uint2 *>(c.scale_zero + (slot * (GQ_D / G) + 2 * g) * 2);
    t.sz = uint4{s2.x, s2.y, 0u, 0u};
  }
  t.rope = uint4{0u, 0u, 0u, 0u};
  return t;
}

template <int G>
__global__ __launch_bounds__(64, 4) void gqa_rows16_kernel(DecodeArgs a) {  // registers for four waves per SIMD
  __shared__ __align__(16) f16 zv_s[16 * GQ16_ZS];
  const int item = blockIdx.x;
  if (item >= a.meta[0]) return;
  const WorkItem it = a.items[item];
  const int l = threadIdx.x, n = l & 15, g = l >> 4;
  const int Gq = a.d.num_heads;  // query heads per KV head
  const int M = Gq * a.Tq;
  const int L = a.seq_len[it.b];
  const int64_t base = a.seq_base[it.b];
  const int n_chunks = (it.t1 - it.t0 + 15) / 16;

  // rotated queries of row n as score B operands (rows past M: zero)
  f16x8 q[4];
  {
    const float *qr = static_cast<const float *>(a.qbuf) + (static_cast<int64_t>(it.b) * M + min(n, M - 1)) * GQ_D;
    // (the row pointer is clamped, so every load is valid and none needs a
    // branch: all 32 are in flight together)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = qr[32 * g + slot_channel(0, kb, e)];
        q[kb][e] = static_cast<f16>(n < M ? x : 0.0f);
      }
  }
  const int vis = n < M ? (a.causal ? (L - a.Tq + n / Gq + 1) : L) : -1;
  const int lim = min(it.t1, vis);  // tokens < lim are visible to row n
  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 o[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) o[ct] = f32x4{};
  // lane's token of chunk c (past the item: its last token, masked)
  auto chunk_slot = [&](int c) -> int64_t { return base + min(it.t0 + 16 * c + n, it.t1 - 1); };
  const uint32_t ztr = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>(zv_s + (4 * g + ((l & 15) >> 2)) * GQ16_ZS + 4 * (l & 3)));

  // one chunk: request chunk c + 1 into (nk, nv) (a harmless re-read past
  // the end), then process chunk c from (ck, cv)
  auto chunk = [&](int c, const RawTile &ck, const RawTile &cv, RawTile &nk, RawTile &nv) {
    const int64_t sn = chunk_slot(c + 1);
    nk = gqa16_load<G>(a.cache, sn, g);
    nv = gqa16_load<G>(a.vcache, sn, g);
    if (c >= n_chunks) return;  // a pair's second chunk past the item: its request only
    f32x4 sacc = f32x4{};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(dequant_block<G>(ck, kb), q[kb], sacc, 0, 0, 0);
    // the V chunk into LDS: row n, columns 32g + 8kb .. (slot order)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      *reinterpret_cast<f16x8 *>(zv_s + n * GQ16_ZS + 32 * g + 8 * kb) = dequant_block<G>(cv, kb);
    // online softmax of row n over tokens 4g .. 4g + 3 of the chunk
    float s[4];
    const int tok0 = it.t0 + 16 * c + 4 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = (tok0 + i < lim) ? sacc[i] : -INFINITY;
    const float lmax = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    if (__any(lmax > m_run + kRescaleThreshold ? 1 : 0)) {
      float tmax = fmaxf(lmax, __shfl_xor(lmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      if (tmax > m_run + kRescaleThreshold) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - tmax);  // 0 on the row's first visible chunk
        if (m_run != -INFINITY) {
#pragma unroll
          for (int ct = 0; ct < 8; ++ct) o[ct] *= alpha;
        }
        l_run *= alpha;
        m_run = tmax;
      }
    }
    const float m_sub = (m_run == -INFINITY) ? 0.0f : m_run;
    float pe[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pe[i] = __builtin_amdgcn_exp2f(s[i] - m_sub);  // masked: 0
    l_run += (pe[0] + pe[1]) + (pe[2] + pe[3]);
    const f16x4 pb = f16x4{static_cast<f16>(pe[0]), static_cast<f16>(pe[1]), static_cast<f16>(pe[2]),
                           static_cast<f16>(pe[3])};
    // the V tile crosses lanes: its stores above the transposing reads
    __builtin_amdgcn_wave_barrier();
    uint32_t zb = ztr;
    asm volatile("" : "+v"(zb));
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
      o[ct] = __builtin_amdgcn_mfma_f32_16x16x16f16(ds_read_tr16_lds(zb + 32 * ct), pb, o[ct], 0, 0, 0);
    // the next chunk's V stores after these reads
    __builtin_amdgcn_wave_barrier();
  };
  RawTile ka, va, kb2, vb;
  if (n_chunks > 0) {
    ka = gqa16_load<G>(a.cache, chunk_slot(0), g);
    va = gqa16_load<G>(a.vcache, chunk_slot(0), g);
  }
  // chunks in pairs, the two register sets in turn (a branch around a
  // pair's second chunk would let the compiler share the sets, and every
  // chunk would then wait for its own prefetch; past the item it issues its
  // request and stops)
  for (int c = 0; c < n_chunks; c += 2) {
    chunk(c, ka, va, kb2, vb);
    chunk(c + 1, kb2, vb, ka, va);
  }

  // ---- the partial: (m, l) of row n, O / l through the V tile ----
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  const float inv_l = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  if (g == 0 && n < M) {
    a.part_ml[(static_cast<int64_t>(item) * M + n) * 2 + 0] = m_run;
    a.part_ml[(static_cast<int64_t>(item) * M + n) * 2 + 1] = l_run;
  }
  // O tile ct holds LDS column 16 ct + 4 g + i of row n
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
    *reinterpret_cast<f16x4 *>(zv_s + n * GQ16_ZS + 16 * ct + 4 * g) = __builtin_convertvector(o[ct] * inv_l, f16x4);
  __builtin_amdgcn_wave_barrier();
  // unit (row, 16-column block ct): LDS column 16 ct + 8 (kb & 1) + e is
  // channel 16 ct + 4 (e / 2) + (kb & 1) + 2 (e & 1)
  f16 *po = reinterpret_cast<f16 *>(a.part_o);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int u = l + 64 * k, row = u >> 3, ct = u & 7;
    const f16x8 a0 = *reinterpret_cast<const f16x8 *>(zv_s + row * GQ16_ZS + 16 * ct);
    const f16x8 a1 = *reinterpret_cast<const f16x8 *>(zv_s + row * GQ16_ZS + 16 * ct + 8);
    if (row < M) {
      f16 outv[16];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        outv[4 * (e >> 1) + 2 * (e & 1)] = a0[e];
        outv[4 * (e >> 1) + 1 + 2 * (e & 1)] = a1[e];
      }
      f16 *dst = po + (static_cast<int64_t>(item) * M + row) * GQ_D + 16 * ct;
      *reinterpret_cast<f16x8 *>(dst) = f16x8{outv[0], outv[1], outv[2], outv[3], outv[4], outv[5], outv[6], outv[7]};
      *reinterpret_cast<f16x8 *>(dst + 8) =
          f16x8{outv[8], outv[9], outv[10], outv[11], outv[12], outv[13], outv[14], outv[15]};
    }
  }
}

}  // namespace

bool mfma_absorb_supported(const mla_dims &d) { return d.qk_nope_head_dim % 16 == 0; }

bool mfma_decode_supported(const mla_dims &d, int rows) {
  return d.kv_lora_rank == R && d.qk_rope_head_dim == DR && (d.group_size == 32 || d.group_size == 16) &&
         rows >= 1;
}

int mfma_row_block() { return ROWS; }

hipError_t launch_absorb_mfma_layout(const DecodeArgs &a, hipStream_t s, const AppendJob *job) {
  TimedLaunch tl(job != nullptr ? "append_absorb_q" : "absorb_q", s);
  const int M = a.d.num_heads * a.Tq;
  const int rb_count = (M + ROWS - 1) / ROWS;
  const int nrows = a.B * a.Tq;
  const int gy = (nrows + 31) / 32;
  const int absorb_cols = a.d.num_heads * 4;
  if (job == nullptr) {
    absorb_mfma_kernel<0><<<dim3(1 + absorb_cols, gy), 256, 0, s>>>(a, rb_count, AppendParams{}, 1);
    return hipGetLastError();
  }
  AppendParams ap{};
  ap.latent = job->latent;
  ap.k_rope = job->k_rope;
  ap.idx_key = job->idx_key;
  ap.slots = job->slots;
  ap.n = job->n;
  ap.Rt = job->Rt;
  ap.alpha = job->alpha;
  ap.cache = a.cache;
  ap.z_out = nullptr;
  ap.lat_stride = R;
  ap.r = R;
  ap.G = a.d.group_size;
  ap.d_r = a.d.qk_rope_head_dim;
  ap.d_idx = a.d.index_head_dim;
  ap.rope_bits = a.d.rope_bits;
  // per 32-token tile: one block per 32-channel tile, one side-key block
  const int blocks = (R / 32 + 1) * static_cast<int>((job->n + 31) / 32);
  const int cols = (blocks + gy - 1) / gy;
  const int x0 = 1 + cols;  // first absorb column
  if (a.d.group_size == 32)
    absorb_mfma_kernel<32><<<dim3(x0 + absorb_cols, gy), 256, 0, s>>>(a, rb_count, ap, x0);
  else
    absorb_mfma_kernel<16><<<dim3(x0 + absorb_cols, gy), 256, 0, s>>>(a, rb_count, ap, x0);
  return hipGetLastError();
}

bool gqa_mfma_supported(const mla_dims &d, int rows) {
  return d.kv_lora_rank == GQ_D && d.qk_rope_head_dim == 0 && rows <= GQ_ROWS &&
         (d.group_size == 16 || d.group_size == 32);
}

// Up to five 16-row waves fit a SIMD, but each more item adds partials to
// merge: three per SIMD measured fastest for the whole step.
int gqa_waves_per_cu(int rows) { return rows <= 16 ? 12 : 8; }

hipError_t launch_gqa_splitk_mfma(const DecodeArgs &a, hipStream_t s) {
  TimedLaunch tl("splitk_decode", s);
  if (a.d.num_heads * a.Tq <= 16) {
    if (a.d.group_size == 32)
      gqa_rows16_kernel<32><<<a.max_items, 64, 0, s>>>(a);
    else
      gqa_rows16_kernel<16><<<a.max_items, 64, 0, s>>>(a);
    return hipGetLastError();
  }
  if (a.d.group_size == 32)
    gqa_splitk_mfma_kernel<32><<<a.max_items, 64, 0, s>>>(a);
  else
    gqa_splitk_mfma_kernel<16><<<a.max_items, 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
