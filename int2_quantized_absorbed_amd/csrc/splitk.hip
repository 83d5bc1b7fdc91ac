// Split-K flash-decode over the INT2 latent cache (absorbed form) for
// r = 512, d_r = 64, on gfx950 MFMA.
//
// [shard PR #5, TL;DR item 2]: attention runs in latent space over the cached
// latent plus one shared rope key.  [OSCAR issue #10, maintainer reply, "How
// the rotation adapts to the latent"]: the cached latent is the rotated INT2
// latent; the up-projection runs on its dequantised value (after the merge).
//
// Built with the VGPR form of MFMA (build flag), so the output accumulators
// and the query operands live in ordinary VGPRs: both wave roles of the
// kernel fit in 256 registers, two waves per SIMD.
#include "splitk_tile.hpp"

namespace mla {
namespace {

// Warp-specialised split-K kernel: one workgroup = one work item x one block
// of 64 query rows, eight waves in two roles that share each SIMD.
//  * Producer w (waves 0..3) owns latent channels [128w, 128w+128) and rope
//    dims [16w, 16w+16): it loads and dequantises the tiles, stores its part
//    of each dequantised tile Z to LDS, runs the score MFMAs over its K-slice
//    and publishes the partial scores.
//  * Consumer w (waves 4..7) owns 16 rows for the softmax (it sums the four
//    partial scores, runs the online softmax, writes P and the per-row
//    rescale factor) and the output block O[64 rows x 128 channels] of slice
//    w, which it updates with the P Z MFMAs.
// Producer w and consumer w sit on one SIMD: each runs its MFMAs while the
// other runs vector-ALU and LDS work.  Per iteration i, two barriers:
//   X (before A): producer: Z of tile i+1 to LDS and the scores of tile
//                 i+1, the stores placed between the MFMAs, the partial
//                 scores published as soon as their MFMAs are done;
//                 consumer: softmax and P of tile i.
//   Y (A to B):   producer: dequantise tile i+2, request tile i+3;
//                 consumer: rescale and O += P Z for tile i, and the sum of
//                 the four partial scores of tile i+1.
// So the exchange of the partial scores overlaps the P Z MFMAs, and the
// softmax of a tile starts from scores already in registers.
// The running max moves only when a tile's max beats it by more than 8 (log2
// units).  The output accumulators live in VGPRs
// (this translation unit is built with the VGPR form of MFMA), so the
// rescale is ordinary code and the compiler inserts the MFMA read hazards.
// MT: 32-row MFMA tiles per block (2: 64 query rows; 1: 32 rows, for at most
// 32 rows in all, which would otherwise be mostly padding).  With MT = 1 the
// consumers 2 and 3 own no softmax rows.  rb_count counts blocks of 32 MT
// rows; the query operands are packed in 64-row blocks (rb_count64 of them).
template <int G, bool RQ, int MT>
__global__ __launch_bounds__(512, 1) void splitk_ws_kernel(DecodeArgs a, int rb_count, int rb_count64,
                                                           int n_logical) {
  constexpr int BROWS = 32 * MT;
  __shared__ Smem sm;
  const int per_xcd = (n_logical + 7) / 8;
  const int logical = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (logical >= n_logical) return;
  const int item = logical / rb_count;
  const int rb = logical % rb_count;
  if (item >= a.meta[0]) return;
  const WorkItem it = a.items[item];

  const int tid = threadIdx.x;
  const bool producer = tid < 256;
  const int w = (tid >> 6) & 3, l = tid & 63, hf = l >> 5, l32 = l & 31;
  const int H = a.d.num_heads;
  const int M = H * a.Tq;
  const int L = a.seq_len[it.b];
  const int64_t base = a.seq_base[it.b];
  const int n_tiles = (it.t1 - it.t0 + TT - 1) / TT;

  if (producer) {
    // ---- Q~ operands (packed by the absorb kernel in exactly this order) ----
    f16x8 aq[MT][KB];
    {
      const int rb64 = (rb * BROWS) / ROWS, mt0 = ((rb * BROWS) % ROWS) / 32;
      const f16x8 *qp = reinterpret_cast<const f16x8 *>(a.qbuf) +
                        ((static_cast<int64_t>(it.b) * rb_count64 + rb64) * 4 + w) * (2 * KB * 64);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) aq[mt][kb] = qp[((mt0 + mt) * KB + kb) * 64 + l];
    }
    const int32_t *sel = a.sel ? a.sel + static_cast<int64_t>(it.b) * a.sel_stride : nullptr;
    auto tile_slot = [&](int i) -> int64_t {
      const int ti = min(i, n_tiles - 1);
      const int t = min(it.t0 + ti * TT + l32, it.t1 - 1);
      return base + (sel ? sel[t] : t);
    };
    f16x8 bz[KB];
    f32x16 sacc[MT];
    // Z tile rows are 288 bytes apart, so rows t and t + 4 fall on the same
    // banks; 16-byte chunk kb of row t is stored at chunk kb ^ (bit 2 ^ bit 3
    // of t): the eight rows of an 8-lane store group, and the sixteen of a
    // 16-lane group, then cover distinct banks
    const int zsw = 8 * (((l32 >> 2) ^ (l32 >> 3)) & 1);
    auto store_z = [&](int zb, const f16x8 (&v)[KB]) {
      f16 *zt = sm.z[zb][w] + l32 * ZSTRIDE + 64 * hf;
      f16 *ze = zt + zsw, *zo = zt - zsw;  // even and odd kb
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) *reinterpret_cast<f16x8 *>(((kb & 1) ? zo : ze) + 8 * kb) = v[kb];
    };
    // partial scores -> sm.sp[w][mt][l]: four 16-byte stores per
    // accumulator; lanes are 64 bytes apart, so quad j of lane l goes to quad
    // j ^ ((l >> 1) & 3): any 8 consecutive lanes then store to distinct banks
    const int p_sw = (l >> 1) & 3;
    auto publish_tile = [&](int mt) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4 *>(&sm.sp[w][mt][l][4 * (j ^ p_sw)]) =
            f32x4{sacc[mt][4 * j], sacc[mt][4 * j + 1], sacc[mt][4 * j + 2], sacc[mt][4 * j + 3]};
    };
    auto mfma_steps = [&](int mt, int kb0, int kb1) {
#pragma unroll
      for (int kb = kb0; kb < kb1; ++kb)
        sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bz[kb], aq[mt][kb], sacc[mt], 0, 0, 0);
    };
    // Scores of the tile in bz, published to LDS, with the Z stores that
    // precede the call (eight per lane) spread over the first MFMAs.  With
    // two row tiles the first tile's chain runs first, and its stores issue
    // between the second chain's MFMAs.
    auto scores_publish = [&]() {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) sacc[mt] = f32x16{};
      if constexpr (MT == 2) {
        mfma_steps(0, 0, KB);
        mfma_steps(1, 0, 2);
        interleave_stores<8, false>();
        __builtin_amdgcn_sched_barrier(0);
        publish_tile(0);
        mfma_steps(1, 2, KB);
        interleave_stores<4, true>();
        __builtin_amdgcn_sched_barrier(0);
        publish_tile(1);
      } else {
        mfma_steps(0, 0, KB);
        interleave_stores<8, false>();
        __builtin_amdgcn_sched_barrier(0);
        publish_tile(0);
      }
    };
    RawTile raw;
    {
      // prologue: tile 0 scored, published and in Z buffer 0; tile 1
      // dequantised; tile 2 in flight
      const RawTile r0 = load_tile<G, RQ>(a, tile_slot(0), w, hf);
      const RawTile r1 = load_tile<G, RQ>(a, tile_slot(1), w, hf);
      raw = load_tile<G, RQ>(a, tile_slot(2), w, hf);
      dequant<G, RQ>(r0, bz);
      store_z(0, bz);
      scores_publish();
      dequant<G, RQ>(r1, bz);
    }
    lds_barrier();  // P0: partial scores and Z of tile 0
    lds_barrier();  // P1: the consumers have read the partial scores of tile 0
    for (int i = 0; i < n_tiles; ++i) {
      // X: Z of tile i+1 to the buffer the consumers read at tile i-1 (done
      // by barrier B of i-1); its scores (harmless recompute past the end),
      // published as soon as the MFMAs are done, while the consumers run the
      // softmax of tile i
      store_z((i + 1) & 1, bz);
      scores_publish();
      lds_barrier();  // A: partial scores and Z of tile i+1; P of tile i
      // Y: dequantise tile i+2, request tile i+3
      dequant<G, RQ>(raw, bz);
      raw = load_tile<G, RQ>(a, tile_slot(i + 3), w, hf);
      lds_barrier();  // B: the consumers have read the partial scores of tile i+1 and P and Z of tile i
    }
    lds_barrier();  // E: 1 / l of every row
    return;
  }

  // ---------------- consumers ----------------
  // softmax ownership: lane -> (row, 8 consecutive tokens); a row's four lanes
  // form a quad
  const int s_row = 16 * w + (l >> 2), s_k8 = l & 3;
  const bool s_own = s_row < BROWS;  // false: a consumer with no softmax rows (MT = 1)
  const int s_m = rb * BROWS + s_row;
  int s_vis = -1;  // padding rows are never visible
  if (s_own && s_m < M) s_vis = a.causal ? (L - a.Tq + s_m / H + 1) : L;
  const int s_lim = min(it.t1, s_vis);  // tokens < s_lim are visible to this row
  float m_run = -INFINITY, l_run = 0.0f;
  // tiles [0, full_tiles) are visible to every row of this wave: no masking
  int vmin = s_lim - it.t0;
  for (int off = 32; off > 0; off >>= 1) vmin = min(vmin, __shfl_xor(vmin, off));
  const int full_tiles = __builtin_amdgcn_readfirstlane(vmin > 0 ? vmin / TT : 0);
  // Summed scores of the owned (row, 8 tokens): token 8j + 4h + e of row r
  // sits in lane (r % 32) + 32h, slot 4j + e, of accumulator r / 32; each
  // lane's four 16-byte quads are stored XOR-swizzled by bits 1-2 of the lane
  const int s_lane = s_row & 31, s_mt = s_row >> 5;
  const int s_q = s_k8 ^ ((s_lane >> 1) & 3);

  f32x16 o[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) o[mt][nt] = f32x16{};
  const int g16 = l >> 4, s16 = l & 15;
  const int pv_krow = 8 * (g16 >> 1) + (s16 >> 2);    // transposing-load source row
  // and column: rows pv_krow + 16 ks share bit 3 (the chunk swizzle's bit 3
  // term); the second load's rows are 4 further on, so bit 2 flips too
  const int pv_col = (16 * (g16 & 1) + 4 * (s16 & 3)) ^ (8 * ((g16 >> 1) & 1));
  const int pv_col_hi = pv_col ^ 8;
  // the four partial scores of the owned (row, 8 tokens), summed
  float s[8];
  auto read_scores = [&]() {
    f32x4 part[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int ww = 0; ww < 4; ++ww)
        part[h][ww] = *reinterpret_cast<const f32x4 *>(&sm.sp[ww][s_mt][s_lane + 32 * h][4 * s_q]);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 acc4 = (part[h][0] + part[h][1]) + (part[h][2] + part[h][3]);
#pragma unroll
      for (int e = 0; e < 4; ++e) s[4 * h + e] = acc4[e];
    }
  };
  lds_barrier();  // P0
  read_scores();
  lds_barrier();  // P1
  for (int i = 0; i < n_tiles; ++i) {
    const int buf = i & 1;
    // X: online softmax and P of tile i (its summed scores are in s)
    if (i >= full_tiles) {
      const int ncnt = s_lim - (it.t0 + i * TT + 8 * s_k8);  // visible tokens among my 8
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] = (e < ncnt) ? s[e] : -INFINITY;
    }
    float lmax = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    // The running max of a row moves only when the tile's max beats it by
    // more than the threshold (always on its first visible tile, m = -inf).
    // Most tiles move no row of the wave: then the exponentials start from
    // the running max at once, with no row reduction on the way.
    float alpha = 1.0f;
    bool scale_o = false;
    if (__any(lmax > m_run + kRescaleThreshold ? 1 : 0)) {
      const float tmax = reduce4<true>(lmax);
      const bool need = tmax > m_run + kRescaleThreshold;
      alpha = need ? __builtin_amdgcn_exp2f(m_run - tmax) : 1.0f;  // exp2(-inf) = 0
      // a row's O is still zero until its first visible tile: no rescale then
      scale_o = need && m_run != -INFINITY;
      m_run = need ? tmax : m_run;
    }
    const float m_sub = (m_run == -INFINITY) ? 0.0f : m_run;
    float pe[8];
    f16x8 pv;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pe[e] = __builtin_amdgcn_exp2f(s[e] - m_sub);  // masked: exp2(-inf) = 0
      pv[e] = static_cast<f16>(pe[e]);
    }
    // l_run is this lane's share of the row sum (its 8 tokens); the four
    // lanes of a row are added once, after the last tile
    l_run = l_run * alpha + (((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7])));
    *reinterpret_cast<f16x8 *>(sm.p + s_row * PRSTRIDE + 8 * s_k8) = pv;
    // every lane stores (a row's lanes store equal values to one address)
    sm.alpha[s_row] = alpha;
    sm.resc[w] = __any((scale_o && s_own) ? 1 : 0);
    lds_barrier();  // A: P, alpha and the rescale flags of tile i; the partial scores of tile i+1
    // Y: O = alpha O + P Z for tile i; the summed scores of tile i+1
    read_scores();
    if (sm.resc[0] | sm.resc[1] | sm.resc[2] | sm.resc[3]) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float al = sm.alpha[32 * mt + 8 * (v >> 2) + 4 * hf + (v & 3)];
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) o[mt][nt][v] *= al;
        }
    }
    const f16 *zb_base = sm.z[buf][w] + pv_krow * ZSTRIDE + pv_col;
    const f16 *zb_hi = sm.z[buf][w] + (pv_krow + 4) * ZSTRIDE + pv_col_hi;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      f16x8 pa[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        pa[mt] = *reinterpret_cast<const f16x8 *>(sm.p + (32 * mt + l32) * PRSTRIDE + 16 * ks + 8 * hf);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const f16x4 lo = ds_read_tr16(zb_base + 16 * ks * ZSTRIDE + 32 * nt);
        const f16x4 hi = ds_read_tr16(zb_hi + 16 * ks * ZSTRIDE + 32 * nt);
        const f16x8 zb = f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          o[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa[mt], zb, o[mt][nt], 0, 0, 0);
      }
    }
    // all P Z MFMAs issue in this phase: the scheduler would sink part of
    // them past barrier B, where they hold up the softmax of the next tile
    // behind the producers' score MFMAs on the same SIMD
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();  // B
  }
  // ---- the partial (O / l in fp16, m, l) of this work item ----
  l_run = reduce4<false>(l_run);
  if (s_k8 == 0) sm.inv_l[s_row] = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  if (s_k8 == 0 && s_own && s_m < M) {
    a.part_ml[(static_cast<int64_t>(item) * M + s_m) * 2 + 0] = m_run;
    a.part_ml[(static_cast<int64_t>(item) * M + s_m) * 2 + 1] = l_run;
  }
  lds_barrier();  // E
  // Each 32x32 accumulator tile (rows 32 mt.., the 32 contiguous channels
  // 128 w + 32 nt..) goes through this slice's Z buffers (the producers are
  // done with them) so that every lane then stores 4 contiguous channels of
  // one row.  Staged position of (row, col): rows in pairs of 64 floats, the
  // half chosen by bit 0 xor bit 2 of the row, so the 4-row-apart halves a
  // store writes and the adjacent rows a 16-lane read takes fall in disjoint
  // banks.
  auto stage_pos = [](int row, int col) { return (row >> 1) * 64 + 32 * ((row ^ (row >> 2)) & 1) + col; };
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      float *st = reinterpret_cast<float *>(sm.z[nt & 1][w]);
      const int sl = 32 * nt + l32;  // slot of the wave's Z tile
      const int col = slot_channel(sl >> 6, (sl & 63) >> 3, sl & 7) - 32 * nt;
#pragma unroll
      for (int v = 0; v < 16; ++v) st[stage_pos(8 * (v >> 2) + 4 * hf + (v & 3), col)] = o[mt][nt][v];
      // the staged values cross lanes: stores above the reads (and the reads
      // above the stores of the tile two steps on, which reuses this buffer)
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 8 * j + (l >> 3), q = l & 7;
        const f32x4 x = *reinterpret_cast<const f32x4 *>(st + stage_pos(row, 4 * q));
        const f16x4 y = __builtin_convertvector(x * sm.inv_l[32 * mt + row], f16x4);
        const int m = rb * BROWS + 32 * mt + row;
        if (m < M)  // ordinary stores: the combine kernel reads the rows next, often from the L2
          *reinterpret_cast<f16x4 *>(a.part_o + (static_cast<int64_t>(item) * M + m) * R + 128 * w + 32 * nt + 4 * q) = y;
      }
      __builtin_amdgcn_wave_barrier();
    }
}


// ---------------------------------------------------------------------------
// Split-K for at most 16 query rows (one GPU's 16-head share of a layer, or
// fewer heads): every wave of the workgroup is an independent worker over
// its own 16-token chunks of the work item (chunks v, v + 8, ...), with the
// whole 576-wide contraction in its own instructions, so the tile loop has
// no workgroup barrier and no partial-score exchange:
//   scores  S^T[16 tokens x 16 rows] = Z Q^T: 18 v_mfma_f32_16x16x32_f16
//           (Z the dequantised tokens, one per lane row, as the A operand;
//           the queries, shared by the eight waves, from LDS);
//   softmax its own running max and sum per row (lazy rescale as above);
//           the score lanes already hold P^T in the layout of the next
//           product's B operand;
//   PV      O^T[512 x 16] += Z^T P^T: 32 v_mfma_f32_16x16x16_f16, Z^T read
//           with ds_read_b64_tr_b16 from a wave-private LDS copy of the tile.
// At the end each wave leaves its (m, l) and its O / l (fp16) in LDS, and
// one pass over the eight waves merges them into the usual normalised fp16
// partial of the work item.  Dense decode only (sparse decode keeps the
// kernel above).
// LDS: the query operands (18 K-steps x 64 lanes x 16 B) and per wave a Z
// tile of 16 tokens x 512 channels (rows padded by 32 B: the four rows of a
// transposing read fall in separate banks), which the wave's partial reuses
// (rows padded by 16 B: a row's 16 lanes of a merge read fall in separate
// banks).
constexpr int R16_ZS = R + 16;  // halves per Z tile row
constexpr int R16_OS = R + 8;   // halves per partial row
constexpr int R16_KS = 2 * KB;  // K-steps: per lane half 8 latent + 1 rope
static_assert(R16_OS <= R16_ZS, "a wave's partial must fit its Z region");

struct __align__(16) SmemR16 {
  f16x8 q[R16_KS * 64];
  f16 z[8][16 * R16_ZS];
  float m[8][16], l[8][16];
};

template <int G, bool RQ>
__global__ __launch_bounds__(512, 1) void splitk_rows16_kernel(DecodeArgs a, int n_logical) {
  __shared__ SmemR16 sm;
  const int per_xcd = (n_logical + 7) / 8;
  const int item = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (item >= n_logical || item >= a.meta[0]) return;
  const WorkItem it = a.items[item];
  const int tid = threadIdx.x, l = tid & 63, n = l & 15, g = l >> 4;
  const int v = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar chunk loop
  const int H = a.d.num_heads, M = H * a.Tq;
  const int L = a.seq_len[it.b];
  const int64_t base = a.seq_base[it.b];
  const int n_chunks = (it.t1 - it.t0 + 15) / 16;

  // ---- query operands of the block's rows into LDS: unit (step s = 9 hf +
  // kb, lane n + 16 q) = the producer-order unit (quarter q, half hf, kb) of
  // row n; rows past M are zero ----
  {
    const f16x8 *qb = reinterpret_cast<const f16x8 *>(a.qbuf);
    for (int u = tid; u < R16_KS * 64; u += 512) {
      const int s = u >> 6, ln = u & 63, rn = ln & 15, qq = ln >> 4, hf = s / KB, kb = s % KB;
      f16x8 val = f16x8{};
      if (rn < M) val = qb[((static_cast<int64_t>(it.b) * 4 + qq) * 2 * KB + kb) * 64 + rn + 32 * hf];
      sm.q[u] = val;
    }
  }
  // rows of this lane: visible tokens < s_lim (padding rows see none)
  int s_vis = -1;
  if (n < M) s_vis = a.causal ? (L - a.Tq + n / H + 1) : L;
  const int s_lim = min(it.t1, s_vis);
  // lane (token n of the chunk, quarter g): its cache slot (dense decode
  // only: a slot indirection would put a dependent load, and with it a wait
  // for every load in flight, in front of each chunk's requests)
  // (chunks past the item read its last token; their tokens are masked)
  auto chunk_slot = [&](int c) -> int64_t { return base + min(it.t0 + 16 * c + n, it.t1 - 1); };
  f16 *zt = sm.z[v];
  f32x4 o[32];
#pragma unroll
  for (int ct = 0; ct < 32; ++ct) o[ct] = f32x4{};
  float m_run = -INFINITY, l_run = 0.0f;
  // transposing-read position of lane l: rows (tokens) 4g + (l & 15) / 4,
  // columns 4 (l & 3) of each 16-column block
  const uint32_t ztr =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(zt + (4 * g + ((l & 15) >> 2)) * R16_ZS + 4 * (l & 3)));
  // two register sets for the chunk tiles, used in turn (two chunks per
  // trip), so the next chunk's loads stay in flight while one is processed:
  // copying a tile between registers would wait for its loads
  RawTile ta0, ta1, tb0, tb1;
  if (v < n_chunks) {
    const int64_t s0 = chunk_slot(v);
    ta0 = load_tile<G, RQ>(a, s0, g, 0);
    ta1 = load_tile<G, RQ>(a, s0, g, 1);
  }
  lds_barrier();  // the query operands (the chunk loads in flight stay in flight)
  // one chunk: request the wave's next chunk c + 8 into (rn0, rn1), then
  // process chunk c from (rc0, rc1).  The request is unconditional (past
  // the item it re-reads the item's last token): with a branch around it
  // the waits for the chunk in hand would also wait for the request.  A
  // chunk past the item stops after its request.
  auto chunk = [&](int c, const RawTile &rc0, const RawTile &rc1, RawTile &rn0, RawTile &rn1) {
    const int64_t sn = chunk_slot(c + 8);
    rn0 = load_tile<G, RQ>(a, sn, g, 0);
    rn1 = load_tile<G, RQ>(a, sn, g, 1);
    if (c >= n_chunks) return;  // a pair's second chunk past the item: its request only
    // ---- scores: one K-block (8 channels of the lane's quarter) at a time ----
    f32x4 sacc = f32x4{};
    f16 *zrow = zt + n * R16_ZS + 128 * g;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const RawTile &t = hf ? rc1 : rc0;
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const f16x8 zv = dequant_block<G>(t, kb);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(zv, sm.q[(KB * hf + kb) * 64 + l], sacc, 0, 0, 0);
        *reinterpret_cast<f16x8 *>(zrow + 64 * hf + 8 * kb) = zv;
      }
      // rope dims 16 g + 8 hf ..
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(dequant_rope<RQ>(t), sm.q[(KB * hf + KB - 1) * 64 + l], sacc, 0,
                                                    0, 0);
    }
    // ---- online softmax of row n over tokens 4g .. 4g + 3 of the chunk ----
    float s[4];
    const int tok0 = it.t0 + 16 * c + 4 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = (tok0 + i < s_lim) ? sacc[i] : -INFINITY;
    const float lmax = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    if (__any(lmax > m_run + kRescaleThreshold ? 1 : 0)) {
      float tmax = fmaxf(lmax, __shfl_xor(lmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      if (tmax > m_run + kRescaleThreshold) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - tmax);  // 0 on the first visible chunk
        if (m_run != -INFINITY) {
#pragma unroll
          for (int ct = 0; ct < 32; ++ct) o[ct] *= alpha;
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
    // the Z tile crosses lanes: its stores above the transposing reads below
    __builtin_amdgcn_wave_barrier();
    // ---- O^T += Z^T P^T ----
    // (an opaque copy of the LDS address: hoisted out of the loop, the 32
    // read addresses would each hold a register; per chunk they fold into
    // the instructions' offsets)
    uint32_t zb = ztr;
    asm volatile("" : "+v"(zb));
#pragma unroll
    for (int ct = 0; ct < 32; ++ct) {
      const f16x4 za = ds_read_tr16_lds(zb + 32 * ct);
      o[ct] = __builtin_amdgcn_mfma_f32_16x16x16f16(za, pb, o[ct], 0, 0, 0);
    }
    // the next chunk's Z stores after these reads
    __builtin_amdgcn_wave_barrier();
  };
  // chunks in pairs, the two register sets in turn (a branch around a
  // pair's second chunk would let the compiler share the sets; past the
  // item it issues its request and stops)
  for (int c = v; c < n_chunks; c += 16) {
    chunk(c, ta0, ta1, tb0, tb1);
    chunk(c + 8, tb0, tb1, ta0, ta1);
  }
  // ---- merge the eight waves ----
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  // the wave's O / l in fp16 into its own Z region, free now (one wave's LDS
  // operations complete in order, so its last transposing reads come first):
  // column 16 ct + 4 g + i of row n
  {
    const float inv_l = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    f16 *ob = zt + n * R16_OS + 4 * g;
#pragma unroll
    for (int ct = 0; ct < 32; ++ct)
      *reinterpret_cast<f16x4 *>(ob + 16 * ct) =
          f16x4{static_cast<f16>(o[ct][0] * inv_l), static_cast<f16>(o[ct][1] * inv_l),
                static_cast<f16>(o[ct][2] * inv_l), static_cast<f16>(o[ct][3] * inv_l)};
  }
  if (g == 0) {
    sm.m[v][n] = m_run;
    sm.l[v][n] = l_run;
  }
  // an LDS-only barrier: __syncthreads would also wait for the partial's
  // global stores of the other waves
  lds_barrier();
  // thread (row rn, 16-column block ct): weights exp2(m_w - mx) l_w / den of
  // the eight waves, then their weighted sum
  const int rn = tid & 15, ct = tid >> 4;
  float mw[8], ew[8];
  float mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    mw[w] = sm.m[w][rn];
    mx = fmaxf(mx, mw[w]);
  }
  float den = 0.0f;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    ew[w] = (mw[w] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw[w] - mx) * sm.l[w][rn];
    den += ew[w];
  }
  const float rden = den > 0.0f ? 1.0f / den : 0.0f;
  float acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const float wt = ew[w] * rden;
    const f16 *src = sm.z[w] + rn * R16_OS + 16 * ct;
    const f16x8 a0 = *reinterpret_cast<const f16x8 *>(src);
    const f16x8 a1 = *reinterpret_cast<const f16x8 *>(src + 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[e] = fmaf(static_cast<float>(a0[e]), wt, acc[e]);
      acc[8 + e] = fmaf(static_cast<float>(a1[e]), wt, acc[8 + e]);
    }
  }
  if (ct == 0 && rn < M) {
    a.part_ml[(static_cast<int64_t>(item) * M + rn) * 2 + 0] = mx;
    a.part_ml[(static_cast<int64_t>(item) * M + rn) * 2 + 1] = den;
  }
  // column block ct = (quarter q, half hf, K-block pair j) = 8 q + 4 hf + j
  // covers channels 128 q + 64 hf + 16 j .. + 16; its column 8 b + e is
  // K-block kb = 2 j + b, channel slot_channel(hf, kb, e) = 64 hf + 16 j +
  // slot_channel(0, b, e): the same permutation in every block, with indices
  // known at compile time (a register array indexed at run time would be
  // lowered to a compare and a select per element)
  if (rn < M) {
    const int q = ct >> 3, hf = (ct >> 2) & 1, j = ct & 3;
    f16 outv[16];
#pragma unroll
    for (int col = 0; col < 16; ++col) outv[slot_channel(0, col >> 3, col & 7)] = static_cast<f16>(acc[col]);
    f16 *dst = reinterpret_cast<f16 *>(a.part_o) + (static_cast<int64_t>(item) * M + rn) * R + 128 * q + 64 * hf + 16 * j;
    *reinterpret_cast<f16x8 *>(dst) = f16x8{outv[0], outv[1], outv[2], outv[3], outv[4], outv[5], outv[6], outv[7]};
    *reinterpret_cast<f16x8 *>(dst + 8) =
        f16x8{outv[8], outv[9], outv[10], outv[11], outv[12], outv[13], outv[14], outv[15]};
  }
}
}  // namespace

SplitK splitk_kernel_for(int rows, bool sparse) {
  return (!sparse && rows <= 16) ? SplitK::kRows16 : SplitK::kWarpSpec;
}

int splitk_target_items(int rows, bool sparse, int ncu) {
  // one workgroup per compute unit: the 16-row kernel's eight waves, or a
  // 64-row block of the warp-specialised kernel
  const int t = splitk_kernel_for(rows, sparse) == SplitK::kRows16 ? ncu : ncu / ((rows + ROWS - 1) / ROWS);
  return t < 1 ? 1 : t;
}

hipError_t launch_splitk_mfma(const DecodeArgs &a, hipStream_t s) {
  TimedLaunch tl("splitk_decode", s);
  const int M = a.d.num_heads * a.Tq;
  const int mt = M <= 32 ? 1 : 2;  // 32-row blocks when all rows fit one
  const int rb_count = (M + 32 * mt - 1) / (32 * mt);
  const int rb_count64 = (M + ROWS - 1) / ROWS;
  // the plan holds at most max(target, sequences) items: size the grid by
  // that, not by the workspace's item capacity, or the XCD-ordered block
  // numbering would hand whole XCDs only blocks past the plan
  const int n_items = std::min(a.max_items, std::max(a.target_items, a.B));
  const int n_logical = n_items * rb_count;
  const int grid = ((n_logical + 7) / 8) * 8;
  const bool rq = a.d.rope_bits == 4;
  if (splitk_kernel_for(M, a.sel != nullptr) == SplitK::kRows16) {
    const int n_items16 = std::min(a.max_items, std::max(a.target_items, a.B));
    const int grid16 = ((n_items16 + 7) / 8) * 8;
#define MLA_ROWS16_LAUNCH(G_, RQ_) splitk_rows16_kernel<G_, RQ_><<<grid16, 512, 0, s>>>(a, n_items16)
    if (a.d.group_size == 32) {
      if (rq) MLA_ROWS16_LAUNCH(32, true); else MLA_ROWS16_LAUNCH(32, false);
    } else {
      if (rq) MLA_ROWS16_LAUNCH(16, true); else MLA_ROWS16_LAUNCH(16, false);
    }
#undef MLA_ROWS16_LAUNCH
    return hipGetLastError();
  }
#define MLA_SPLITK_LAUNCH(G_, RQ_, MT_) \
  splitk_ws_kernel<G_, RQ_, MT_><<<grid, 512, 0, s>>>(a, rb_count, rb_count64, n_logical)
  if (a.d.group_size == 32) {
    if (mt == 1) {
      if (rq) MLA_SPLITK_LAUNCH(32, true, 1); else MLA_SPLITK_LAUNCH(32, false, 1);
    } else {
      if (rq) MLA_SPLITK_LAUNCH(32, true, 2); else MLA_SPLITK_LAUNCH(32, false, 2);
    }
  } else {
    if (mt == 1) {
      if (rq) MLA_SPLITK_LAUNCH(16, true, 1); else MLA_SPLITK_LAUNCH(16, false, 1);
    } else {
      if (rq) MLA_SPLITK_LAUNCH(16, true, 2); else MLA_SPLITK_LAUNCH(16, false, 2);
    }
  }
#undef MLA_SPLITK_LAUNCH
  return hipGetLastError();
}

}  // namespace mla
