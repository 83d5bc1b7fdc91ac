// MFMA split-K absorbed decode for r = 512, d_r = 64 (DeepSeek-V3 /
// GLM-5.3-style MLA layers) on gfx950.
//
// [shard PR #5, TL;DR item 2]: attention runs in latent space over the cached
// latent plus one shared rope key.  [OSCAR issue #10, maintainer reply, "How
// the rotation adapts to the latent"]: the cached latent is the rotated INT2
// latent; the up-projection runs on its dequantised value.
//
// One workgroup = one split-K work item (tokens [t0, t1) of sequence b) x one
// block of 64 query rows (row m = t*H + h).  The four waves split the latent
// channels: wave w owns channels [128w, 128w+128) and rope dims [16w, 16w+16).
// Per 32-token tile:
//   1. each lane loads one token's 2-bit codes for 64 channels (16 B), its
//      groups' fp16 scale/zero and 8 rope values, and dequantises them in
//      registers straight into the fp16 operands of the score MFMA
//      (v_mfma_f32_32x32x16_f16): z_hat = zero + scale * code with one fp16
//      rounding (codes enter as exact small integers);
//   2. partial scores S_w^T[32 tokens x 64 rows] = Z_w Q~_w^T (K = 128 + 16),
//      token-major so each lane's accumulator quads go to LDS as 16-byte
//      stores;
//   3. the four partials are summed on reading, each wave runs the online
//      softmax for 16 rows (a row's 32 tokens on one lane quad, max and sum
//      by DPP), writes P in fp16 to LDS;
//   4. O_w[64 x 128] += P Z_w with Z read back through the gfx950
//      transposing LDS load (ds_read_b64_tr_b16).
// The tile loop is software-pipelined: the scores of tile i+1 are on the
// MFMA pipe while the softmax of tile i runs, and their partials are
// published while the PV of tile i runs (two LDS barriers per tile).
// The running max is only moved when a tile's max exceeds it by more than
// 8 (log2 units); otherwise p = 2^(s - m) <= 256 stays exact enough in fp16
// and O needs no rescaling.
#include "append_tile.hpp"
#include "plan.hpp"

namespace mla {
namespace {

constexpr int R = 512;
constexpr int DR = 64;
constexpr int ROWS = 64;        // query rows per workgroup
constexpr int TT = 32;          // tokens per tile
constexpr int KB = 9;           // K-blocks of 16 per wave: 8 latent + 1 rope
// Z tile rows: 128 halves + 16 pad, so the four rows a transposing load
// reads fall in separate banks.  16-byte chunk c of row t is stored at chunk
// c ^ ((t >> 3) & 1): without it, the 16-byte stores of tokens t and t + 8
// hit the same banks.
constexpr int ZSTRIDE = 144;
constexpr float kRescaleThreshold = 8.0f;  // log2 units

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f16x4 ds_read_tr16(const f16 *p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<s16x4 __attribute__((address_space(3))) *>(
          reinterpret_cast<uintptr_t>(p)));
  return __builtin_bit_cast(f16x4, v);
}

// Workgroup barrier that only waits for this wave's LDS operations.  HIP's
// __syncthreads() also waits for every outstanding global load, which would
// force the next tile's prefetch to land at the first barrier of each tile.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// x *= al for a value the MFMA accumulates in an AGPR.  Written as inline asm
// with an AGPR operand so the compiler keeps the accumulators in AGPRs and
// cannot hoist their copies out of the (rarely taken) rescale branch.
__device__ __forceinline__ void agpr_scale(float &x, float al) {
  float t;
  asm volatile(
      "v_accvgpr_read_b32 %1, %0\n\t"
      "v_mul_f32 %1, %1, %2\n\t"
      "v_accvgpr_write_b32 %0, %1"
      : "+a"(x), "=&v"(t)
      : "v"(al));
}

// The hardware does not interlock a register an MFMA is still writing
// against a later non-MFMA read, and the compiler does not see into inline
// asm, so asm that reads MFMA results must first wait the XDL write -> read
// latency itself: 24 wait states cover an 8-pass MFMA with margin.  Taking
// both accumulator tuples as operands orders this after their last MFMA and
// every asm read of them after this.
__device__ __forceinline__ void mfma_results_settle(f32x16 &a0, f32x16 &a1) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(a0), "+a"(a1));
}

// The same for the eight output accumulators before the rescale reads them
// (kAfterMfma) and, after the rescale's asm wrote them, before the next MFMA
// takes them as its accumulator input.
template <bool kAfterMfma>
__device__ __forceinline__ void o_settle(f32x16 (&o)[2][4]) {
  if (kAfterMfma)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[0][2]), "+a"(o[0][3]), "+a"(o[1][0]), "+a"(o[1][1]),
                   "+a"(o[1][2]), "+a"(o[1][3]));
  else
    asm volatile("s_nop 4"
                 : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[0][2]), "+a"(o[0][3]), "+a"(o[1][0]), "+a"(o[1][1]),
                   "+a"(o[1][2]), "+a"(o[1][3]));
}

// 16-byte LDS store of four values an MFMA left in AGPRs (gfx950 DS stores
// take AGPR data), without copies through VGPRs; the byte offset is an
// immediate.  Call mfma_results_settle on the accumulators first.
template <int OFF>
__device__ __forceinline__ void ds_store_agpr4(uint32_t lds_addr, f32x4 x) {
  asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"(lds_addr), "a"(x), "i"(OFF) : "memory");
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// all-reduce over the 4 lanes of a quad (DPP quad permutations)
template <bool kMax>
__device__ __forceinline__ float reduce4(float x) {
  auto op = [](float a, float b) { return kMax ? fmaxf(a, b) : a + b; };
  x = op(x, dpp_mov<0xB1>(x));  // quad_perm [1,0,3,2]
  x = op(x, dpp_mov<0x4E>(x));  // quad_perm [2,3,0,1]
  return x;
}

// Channel of latent K-slot e (0..7) in K-block kb (0..7) for lane half hf,
// relative to the wave's first channel.  Matches the dequantisation below:
// half2 j of block kb comes from byte j of code word kb/2 (channels
// 16*(kb/2) + 4j .. + 3), taking its channels kb%2 and kb%2 + 2.
__device__ __forceinline__ int slot_channel(int hf, int kb, int e) {
  return 64 * hf + 16 * (kb >> 1) + 4 * (e >> 1) + (kb & 1) + 2 * (e & 1);
}

constexpr int PRSTRIDE = 40;    // halves per row of P (32 tokens + pad)

// Double-buffered tile state (one barrier per tile):
//   z   per wave, dequantised latent tile [token][slot] (PV B operand)
//   sp  partial scores [wave][acc slot][lane (+4 for hf = 1)]
//   p   P [row][token] (PV A operand), alpha per row, per-wave rescale flags
struct __align__(16) Smem {
  f16 z[2][4][TT * ZSTRIDE];
  float sp[4][2][64][16];  // [wave][mt][lane][16 scores, 16-byte quads swizzled]
  f16 p[ROWS * PRSTRIDE];
  float alpha[ROWS];
  float inv_l[ROWS];  // 1 / l of each row, for the normalised partial
  int resc[4];
};

struct RawTile {
  uint4 codes;
  uint4 sz;     // 2 (G = 32) or 4 (G = 16) scale/zero words
  uint4 rope;
};

template <int G>
__device__ __forceinline__ RawTile load_tile(const DecodeArgs &a, int64_t slot, int w, int hf) {
  RawTile t;
  const uint32_t *codes32 = reinterpret_cast<const uint32_t *>(a.cache.codes);
  t.codes = *reinterpret_cast<const uint4 *>(codes32 + slot * (R / 16) + w * 8 + hf * 4);
  if (G == 32) {
    const uint2 s2 = *reinterpret_cast<const uint2 *>(a.cache.scale_zero + (slot * (R / G) + (4 * w + 2 * hf)) * 2);
    t.sz = uint4{s2.x, s2.y, 0u, 0u};
  } else {
    t.sz = *reinterpret_cast<const uint4 *>(a.cache.scale_zero + (slot * (R / G) + (8 * w + 4 * hf)) * 2);
  }
  t.rope = *reinterpret_cast<const uint4 *>(a.cache.k_rope + slot * DR + 16 * w + 8 * hf);
  return t;
}

// Code byte pair -> exact fp16 pair: with every 2-bit code alone in a
// nibble (bits 2-3 clear) the nibble is an OCP e2m1 number of value c/2,
// and gfx950's packed fp4 -> f16 conversion with scale 2 returns (c_lo, c_hi)
// exactly (low nibble in the low half).
template <int BYTE>
__device__ __forceinline__ f16x2 code_pair(uint32_t nibbles) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nibbles, 2.0f, BYTE);
}

// codes -> fp16 score B operands.  Per code word (16 channels): two masks
// split the codes of channels (4j, 4j+2) and (4j+1, 4j+3) into nibbles, then
// per pair one conversion and one fused fp16 multiply-add with the group's
// (scale, zero): z_hat = zero + scale * c with one rounding.
template <int G>
__device__ __forceinline__ void dequant(const RawTile &t, f16x8 (&bz)[KB]) {
  const uint32_t cws[4] = {t.codes.x, t.codes.y, t.codes.z, t.codes.w};
  const uint32_t szw[4] = {t.sz.x, t.sz.y, t.sz.z, t.sz.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t sz = szw[(G == 32) ? (q >> 1) : q];
    const f16x2 sc = __builtin_bit_cast(f16x2, (sz & 0xffffu) * 0x10001u);
    const f16x2 zr = __builtin_bit_cast(f16x2, (sz >> 16) * 0x10001u);
#pragma unroll
    for (int odd = 0; odd < 2; ++odd) {
      const uint32_t u = (cws[q] >> (2 * odd)) & 0x33333333u;
      const f16x2 c0 = __builtin_elementwise_fma(code_pair<0>(u), sc, zr);
      const f16x2 c1 = __builtin_elementwise_fma(code_pair<1>(u), sc, zr);
      const f16x2 c2 = __builtin_elementwise_fma(code_pair<2>(u), sc, zr);
      const f16x2 c3 = __builtin_elementwise_fma(code_pair<3>(u), sc, zr);
      bz[2 * q + odd] = f16x8{c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
    }
  }
  const uint32_t rws[4] = {t.rope.x, t.rope.y, t.rope.z, t.rope.w};
  f16x8 v;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = static_cast<f16>(__uint_as_float(rws[j] << 16));
    v[2 * j + 1] = static_cast<f16>(__uint_as_float(rws[j] & 0xffff0000u));
  }
  bz[8] = v;
}

template <int G>
__global__ __launch_bounds__(256, 1) void splitk_mfma_kernel(DecodeArgs a, int rb_count, int n_logical) {
  __shared__ Smem sm;
  // XCD-aware order: blocks bid, bid+8, ... run on one XCD; give them
  // consecutive logical indices so the row blocks of one item share its L2.
  const int per_xcd = (n_logical + 7) / 8;
  const int logical = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (logical >= n_logical) return;
  const int item = logical / rb_count;
  const int rb = logical % rb_count;
  if (item >= a.meta[0]) return;
  const WorkItem it = a.items[item];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, hf = l >> 5, l32 = l & 31;
  const int H = a.d.num_heads;
  const int M = H * a.Tq;
  const int L = a.seq_len[it.b];
  const int64_t base = a.seq_base[it.b];
  const int n_tiles = (it.t1 - it.t0 + TT - 1) / TT;

  // ---- Q~ operands (packed by the absorb kernel in exactly this order) ----
  f16x8 aq[2][KB];
  {
    const f16x8 *qp = reinterpret_cast<const f16x8 *>(a.qbuf) +
                      ((static_cast<int64_t>(it.b) * rb_count + rb) * 4 + w) * (2 * KB * 64);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) aq[mt][kb] = qp[(mt * KB + kb) * 64 + l];
  }

  // ---- softmax ownership: lane -> (accumulator slot, lane half, 8 tokens) ----
  // slot rho = 8w + (l >> 3) maps to row 32(rho/16) + 8((rho%16)/4) + 4*shf + rho%4
  // softmax ownership: lane -> (row, 8 consecutive tokens); a row's four
  // lanes form a quad
  const int s_row = 16 * w + (l >> 2), s_k8 = l & 3;
  const int s_m = rb * ROWS + s_row;
  int s_vis = -1;  // padding rows are never visible
  if (s_m < M) s_vis = a.causal ? (L - a.Tq + s_m / H + 1) : L;
  const int s_lim = min(it.t1, s_vis);   // tokens < s_lim are visible to this row
  float m_run = -INFINITY, l_run = 0.0f;
  // tiles [0, full_tiles) are visible to every row of this wave: no masking
  int vmin = s_lim - it.t0;
  for (int off = 32; off > 0; off >>= 1) vmin = min(vmin, __shfl_xor(vmin, off));
  const int full_tiles = __builtin_amdgcn_readfirstlane(vmin > 0 ? vmin / TT : 0);

  f32x16 o[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) o[mt][nt] = f32x16{};

  const int g16 = l >> 4, s16 = l & 15;
  const int pv_krow = 8 * (g16 >> 1) + (s16 >> 2);    // transposing-load source row
  // and column (rows pv_krow + 16 ks (+ 4) share bit 3 of pv_krow: one swizzle)
  const int pv_col = (16 * (g16 & 1) + 4 * (s16 & 3)) ^ (8 * ((g16 >> 1) & 1));
  const int32_t *sel = a.sel ? a.sel + static_cast<int64_t>(it.b) * a.sel_stride : nullptr;
  auto tile_slot = [&](int i) -> int64_t {
    const int ti = min(i, n_tiles - 1);
    const int t = min(it.t0 + ti * TT + l32, it.t1 - 1);
    return base + (sel ? sel[t] : t);
  };

  // ---- prologue: tile 0 scores summed in registers, tiles 0 and 1 in the
  // Z buffers, tile 1 dequantised, tile 2 in flight (issued with tiles 0
  // and 1, so the first iteration does not wait for it) ----
  f16x8 bz[KB];
  f32x16 sacc[2];
  const int zsw = 8 * ((l32 >> 3) & 1);  // chunk kb goes to kb ^ 1 in rows 8..15, 24..31
  auto store_z = [&](int zb, const f16x8 (&v)[KB]) {
    f16 *zt = sm.z[zb][w] + l32 * ZSTRIDE + 64 * hf;
    f16 *ze = zt + zsw, *zo = zt - zsw;  // even and odd kb
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) *reinterpret_cast<f16x8 *>(((kb & 1) ? zo : ze) + 8 * kb) = v[kb];
  };
  // Summed scores of the owned (row, 8 tokens): in the transposed score
  // layout token 8j + 4h + e of row r sits in lane (r % 32) + 32h, slot
  // 4j + e, of accumulator r / 32; each lane's four 16-byte quads are
  // stored XOR-swizzled by bits 2-3 of the lane (conflict-free stores and
  // loads in 16-lane groups).
  const int s_lane = s_row & 31, s_mt = s_row >> 5;
  const int s_q = s_k8 ^ ((s_lane >> 2) & 3);
  auto read_scores = [&](float (&s8)[8]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 acc4 = *reinterpret_cast<const f32x4 *>(&sm.sp[0][s_mt][s_lane + 32 * h][4 * s_q]);
#pragma unroll
      for (int ww = 1; ww < 4; ++ww)
        acc4 += *reinterpret_cast<const f32x4 *>(&sm.sp[ww][s_mt][s_lane + 32 * h][4 * s_q]);
      s8[4 * h] = acc4[0];
      s8[4 * h + 1] = acc4[1];
      s8[4 * h + 2] = acc4[2];
      s8[4 * h + 3] = acc4[3];
    }
  };
  // partial scores -> sm.sp[sb][w][mt][l]: four 16-byte stores per
  // accumulator; quad j of lane l at quad j ^ ((l >> 2) & 3)
  const int p_sw = (l >> 2) & 3;
  auto publish = [&](f32x16 (&acc)[2]) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4 *>(&sm.sp[w][mt][l][4 * (j ^ p_sw)]) =
            f32x4{acc[mt][4 * j], acc[mt][4 * j + 1], acc[mt][4 * j + 2], acc[mt][4 * j + 3]};
  };
  float s_next[8];
  RawTile raw;
  {
    const RawTile r0 = load_tile<G>(a, tile_slot(0), w, hf);
    const RawTile r1 = load_tile<G>(a, tile_slot(1), w, hf);
    raw = load_tile<G>(a, tile_slot(2), w, hf);
    dequant<G>(r0, bz);
    sacc[0] = f32x16{};
    sacc[1] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bz[kb], aq[mt][kb], sacc[mt], 0, 0, 0);
    store_z(0, bz);
    publish(sacc);
    dequant<G>(r1, bz);
  }
  lds_barrier();
  read_scores(s_next);

  for (int i = 0; i < n_tiles; ++i) {
    const int buf = i & 1, nb = buf ^ 1;
    // masking first, so the score MFMAs and the softmax below stay in one
    // basic block and can interleave
    float s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = s_next[e];
    if (i >= full_tiles) {
      const int ncnt = s_lim - (it.t0 + i * TT + 8 * s_k8);  // visible tokens among my 8
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] = (e < ncnt) ? s[e] : -INFINITY;
    }
    // ---- (a) scores of tile i+1 on MFMA (harmless recompute past the end) ----
    sacc[0] = f32x16{};
    sacc[1] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bz[kb], aq[mt][kb], sacc[mt], 0, 0, 0);
    // Z of tile i+1 to its buffer (last read by the PV of tile i-1), while
    // the MFMAs run
    store_z(nb, bz);

    // ---- (b) online softmax of tile i (vector ALU, overlaps the MFMAs) ----
    float tmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) tmax = fmaxf(tmax, s[e]);
    tmax = reduce4<true>(tmax);
    const bool need = tmax > m_run + kRescaleThreshold;   // true on the first visible tile
    const float alpha = need ? __builtin_amdgcn_exp2f(m_run - tmax) : 1.0f;  // exp2(-inf) = 0
    // a row's O is still zero until its first visible tile: no rescale then
    const bool scale_o = need && m_run != -INFINITY;
    m_run = need ? tmax : m_run;
    const float m_sub = (m_run == -INFINITY) ? 0.0f : m_run;
    float psum = 0.0f;
    f16x8 pv;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = __builtin_amdgcn_exp2f(s[e] - m_sub);  // masked: exp2(-inf) = 0
      psum += p;
      pv[e] = static_cast<f16>(p);
    }
    psum = reduce4<false>(psum);
    l_run = l_run * alpha + psum;
    *reinterpret_cast<f16x8 *>(sm.p + s_row * PRSTRIDE + 8 * s_k8) = pv;
    // every lane stores (the quad's lanes and the wave's lanes store equal
    // values to one address), which keeps this block branch-free
    sm.alpha[s_row] = alpha;
    sm.resc[w] = __any(scale_o ? 1 : 0);
    lds_barrier();  // A: P, alpha and the rescale flags of tile i


    // ---- (d) O = alpha * O + P Z for tile i ----
    const int rescale = sm.resc[0] | sm.resc[1] | sm.resc[2] | sm.resc[3];
    if (rescale) {
      o_settle<true>(o);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float al = sm.alpha[32 * mt + 8 * (v >> 2) + 4 * hf + (v & 3)];
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            float x = o[mt][nt][v];
            agpr_scale(x, al);
            o[mt][nt][v] = x;
          }
        }
      o_settle<false>(o);
    }
    const f16 *zb_base = sm.z[buf][w] + pv_krow * ZSTRIDE + pv_col;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      f16x8 pa[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        pa[mt] = *reinterpret_cast<const f16x8 *>(sm.p + (32 * mt + l32) * PRSTRIDE + 16 * ks + 8 * hf);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const f16 *z0 = zb_base + 16 * ks * ZSTRIDE + 32 * nt;
        const f16x4 lo = ds_read_tr16(z0);
        const f16x4 hi = ds_read_tr16(z0 + 4 * ZSTRIDE);
        const f16x8 zb = f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          o[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa[mt], zb, o[mt][nt], 0, 0, 0);
      }
    }
    // ---- (e) dequantise tile i+2 into the Z buffer tile i just used (this
    // wave's own region: its PV reads above were issued first), prefetch
    // tile i+3 and the summed partial scores of tile i+1 ----
    // ---- (c) partial scores of tile i+1 to LDS (their MFMAs finished
    // during the softmax), next tile's operands ----
    publish(sacc);
    dequant<G>(raw, bz);
    raw = load_tile<G>(a, tile_slot(i + 3), w, hf);
    lds_barrier();  // B: partial scores of tile i+1
    read_scores(s_next);
  }

  // ---- write the partial (O / l in fp16, m, l) of this work item ----
  if (s_k8 == 0) sm.inv_l[s_row] = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  lds_barrier();
  // Each 32x32 accumulator tile (rows 32 mt.., the 32 contiguous channels
  // 128 w + 32 nt..) goes through this wave's own Z buffers (no other wave
  // touches them) so that every lane then stores 4 contiguous channels of one
  // row.  Staged position of (row, col): rows in pairs of 64 floats, the half
  // chosen by bit 0 xor bit 2 of the row, so the 4-row-apart halves a store
  // writes and the adjacent rows a 16-lane read takes fall in disjoint banks.
  auto stage_pos = [](int row, int col) { return (row >> 1) * 64 + 32 * ((row ^ (row >> 2)) & 1) + col; };
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      float *st = reinterpret_cast<float *>(sm.z[nt & 1][w]);
      const int sl = 32 * nt + l32;  // slot of the wave's Z tile
      const int col = slot_channel(sl >> 6, (sl & 63) >> 3, sl & 7) - 32 * nt;
#pragma unroll
      for (int v = 0; v < 16; ++v) st[stage_pos(8 * (v >> 2) + 4 * hf + (v & 3), col)] = o[mt][nt][v];
      // the staged values cross lanes: keep the stores above the reads (and,
      // below, the reads above the stores of the tile two steps on, which
      // reuses this buffer)
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 8 * j + (l >> 3), q = l & 7;
        const f32x4 x = *reinterpret_cast<const f32x4 *>(st + stage_pos(row, 4 * q));
        const f16x4 y = __builtin_convertvector(x * sm.inv_l[32 * mt + row], f16x4);
        const int m = rb * ROWS + 32 * mt + row;
        if (m < M)  // ordinary stores: the combine kernel reads the rows next, often from the L2
          *reinterpret_cast<f16x4 *>(a.part_o + (static_cast<int64_t>(item) * M + m) * R + 128 * w + 32 * nt + 4 * q) = y;
      }
      __builtin_amdgcn_wave_barrier();
    }
  if (s_k8 == 0 && s_m < M) {
    a.part_ml[(static_cast<int64_t>(item) * M + s_m) * 2 + 0] = m_run;
    a.part_ml[(static_cast<int64_t>(item) * M + s_m) * 2 + 1] = l_run;
  }
}

// q~ = W~_UK[h]^T q_nope on MFMA (32x32x16 f16, fp32 acc), and q_rope; both
// times scale*log2(e), written in fp16 straight into the per-lane operand
// order of splitk_mfma_kernel: [b][row block][wave][mt][kb][lane][8], zero
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
// round trips overlap the absorb: each 4-wave block appends four 32-channel
// tiles of one 32-token tile, with the same tile code as the stand-alone
// small-append kernel, so the cache bytes are identical).  The absorb blocks
// are the columns from x0 on.
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
      // append block: tiles (ct = 4 (blk % (R / 128)) + wave, ty = blk / (R / 128))
      const int blk = (blockIdx.x - 1) * gridDim.y + blockIdx.y;
      const int ty = blk / (R / 128), ct = 4 * (blk % (R / 128)) + (threadIdx.x >> 6);
      if (static_cast<int64_t>(ty) * 32 < ap.n) skinny_tile<R, G, 2, false>(ap, ct, ty, threadIdx.x & 63);
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
      for (int e = 0; e < 8; ++e) aq[kb][e] = static_cast<f16>(l32 < M ? qr[slot_channel(hf, kb, e)] : 0.0f);
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
  const int blocks = (R / 128) * static_cast<int>((job->n + 31) / 32);  // four 32-channel tiles per block
  const int cols = (blocks + gy - 1) / gy;
  const int x0 = 1 + cols;  // first absorb column
  if (a.d.group_size == 32)
    absorb_mfma_kernel<32><<<dim3(x0 + absorb_cols, gy), 256, 0, s>>>(a, rb_count, ap, x0);
  else
    absorb_mfma_kernel<16><<<dim3(x0 + absorb_cols, gy), 256, 0, s>>>(a, rb_count, ap, x0);
  return hipGetLastError();
}

hipError_t launch_splitk_mfma(const DecodeArgs &a, hipStream_t s) {
  TimedLaunch tl("splitk_decode", s);
  const int M = a.d.num_heads * a.Tq;
  const int rb_count = (M + ROWS - 1) / ROWS;
  const int n_logical = a.max_items * rb_count;
  const int grid = ((n_logical + 7) / 8) * 8;
  if (a.d.group_size == 32)
    splitk_mfma_kernel<32><<<grid, 256, 0, s>>>(a, rb_count, n_logical);
  else
    splitk_mfma_kernel<16><<<grid, 256, 0, s>>>(a, rb_count, n_logical);
  return hipGetLastError();
}

bool gqa_mfma_supported(const mla_dims &d, int rows) {
  return d.kv_lora_rank == GQ_D && d.qk_rope_head_dim == 0 && rows <= GQ_ROWS &&
         (d.group_size == 16 || d.group_size == 32);
}

hipError_t launch_gqa_splitk_mfma(const DecodeArgs &a, hipStream_t s) {
  TimedLaunch tl("splitk_decode", s);
  if (a.d.group_size == 32)
    gqa_splitk_mfma_kernel<32><<<a.max_items, 64, 0, s>>>(a);
  else
    gqa_splitk_mfma_kernel<16><<<a.max_items, 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
