// Device pieces of the quantise-on-append path shared by the append kernels
// and by the decode-step launch that runs a small append next to the query
// absorb: the argument block, the side-key copy, the quantiser epilogue of
// one 32-channel x 32-token rotation tile, and the one-wave small-append tile.
//
// [OSCAR issue #10, maintainer reply, "How the rotation adapts to the
// latent"]: the cache holds the rotated, INT2-quantised latent; low-variance
// eigen-directions (the first channels of z, ascending order) share groups.
#pragma once

#include "kernels.hpp"

namespace mla {
namespace {

constexpr int kSkinnyMaxTokens = 1024;  // appends of at most this many tokens use the small-append tile

// Copy the bf16 side keys (width values each) of tokens [t0, t0 + cnt) into
// their cache slots, one wave, all lanes moving 16-byte pieces (4-byte pieces
// when width is not a multiple of 8); slots outside the cache are skipped.
__device__ __forceinline__ void copy_side_keys(uint16_t *__restrict__ dst, const uint16_t *__restrict__ src,
                                               int width, const int64_t *__restrict__ slots, int64_t t0,
                                               int cnt, int64_t capacity, int lane) {
  if ((width & 7) == 0) {
    const int per = width / 8, total = cnt * per;
    for (int e0 = lane; e0 < total; e0 += 64 * 4) {
      uint4 v[4];
      int64_t sl[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = min(e0 + 64 * j, total - 1), t = e / per;
        sl[j] = slots[t0 + t];
        v[j] = reinterpret_cast<const uint4 *>(src + (t0 + t) * width)[e % per];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = e0 + 64 * j;
        if (e < total && sl[j] >= 0 && sl[j] < capacity)
          reinterpret_cast<uint4 *>(dst + sl[j] * width)[e % per] = v[j];
      }
    }
  } else {
    const int per = width / 2, total = cnt * per;
    for (int e = lane; e < total; e += 64) {
      const int t = e / per;
      const int64_t sl = slots[t0 + t];
      if (sl >= 0 && sl < capacity)
        reinterpret_cast<uint32_t *>(dst + sl * width)[e % per] =
            reinterpret_cast<const uint32_t *>(src + (t0 + t) * width)[e % per];
    }
  }
}

struct AppendParams {
  const void *latent;
  const uint16_t *k_rope;
  const uint16_t *idx_key;
  const int64_t *slots;
  int64_t n;
  const uint16_t *Rt;
  const float *alpha;
  mla_cache cache;
  float *z_out;
  int64_t lat_stride;  // elements from one token's latent row to the next
  int r, G, d_r, d_idx;
  int rope_bits;       // 0: bf16 rope keys copied; 4: quantised (rope_quant_group)
};

// Rope-key variant: token tok's rope dims 16 g .. 16 g + 15 to 4-bit codes
// with an fp16 (scale, zero) [OSCAR issue #10, maintainer's later reply: two
// designs for the rope and non-rope parts; the reading is the latent
// quantiser without clipping, 15 levels, rope key unrotated]: 16 bf16 values
// in (two 16-byte loads), 8 code bytes and one (scale, zero) word out into
// the slot's entry (d_r / 2 code bytes, then d_r / 16 words; entries are
// 4-byte aligned).  Every step in IEEE fp32 with no contraction, the division
// correctly rounded, as the latent quantiser.
__device__ __forceinline__ void rope_quant_group(const uint16_t *__restrict__ k_rope, int64_t tok, int g, int d_r,
                                                 int64_t slot, uint8_t *__restrict__ entries) {
  const uint4 *src = reinterpret_cast<const uint4 *>(k_rope + tok * d_r + 16 * g);
  const uint4 v0 = src[0], v1 = src[1];
  const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  float x[16];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[2 * j] = __uint_as_float(w[j] << 16);
    x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
  float mx = x[0], mn = x[0];
#pragma unroll
  for (int j = 1; j < 16; ++j) {
    mx = fmaxf(mx, x[j]);
    mn = fminf(mn, x[j]);
  }
  const float mid = __fmul_rn(0.5f, __fadd_rn(mx, mn));
  const float half = __fmul_rn(0.5f, __fsub_rn(mx, mn));
  const float lo = __fsub_rn(mid, half);
  const float hi = __fadd_rn(mid, half);
  const f16 scale = f32_to_f16(__fdiv_rn(__fsub_rn(hi, lo), 15.0f));
  const f16 zero = f32_to_f16(lo);
  const float sf = static_cast<float>(scale), zf = static_cast<float>(zero);
  uint32_t packed[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    uint32_t c = 0u;
    if (sf != 0.0f) {  // fmaxf/fminf drop a NaN quotient: code 0
      const float u = __fdiv_rn(__fsub_rn(x[j], zf), sf);
      c = static_cast<uint32_t>(fminf(fmaxf(rintf(u), 0.0f), 15.0f));
    }
    packed[j >> 3] |= c << (4 * (j & 7));
  }
  uint8_t *e = entries + slot * (d_r / 2 + d_r / 4);
  reinterpret_cast<uint32_t *>(e + 8 * g)[0] = packed[0];
  reinterpret_cast<uint32_t *>(e + 8 * g)[1] = packed[1];
  *reinterpret_cast<uint32_t *>(e + d_r / 2 + 4 * g) =
      static_cast<uint32_t>(f16_bits(scale)) | (static_cast<uint32_t>(f16_bits(zero)) << 16);
}

// Epilogue of one 32-channel x 32-token rotation tile in MFMA C layout (lane
// l holds channels ch0 + 8q + 4hf + s, v = 4q + s, of token tok): the fp32
// rotated latent for a rotation-only launch, else the group min/max
// (exchanged with the partner lane l ^ 32), fp16 scale/zero, INT2 codes and
// their stores into the token's cache slot.
template <int R, int G>
__device__ __forceinline__ void tile_epilogue(const AppendParams &p, const f32x16 &z, int64_t tok, bool write,
                                              int64_t slot, int ch0, const float (&alpha)[32 / G], int hf) {
  constexpr int NGT = 32 / G;    // groups per tile: 1 (G=32) or 2 (G=16)
  constexpr int VPG = 16 / NGT;  // values per lane per group
  if (p.z_out != nullptr) {
    if (write) {
      float *dst = p.z_out + tok * R + ch0 + 4 * hf;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4 *>(dst + 8 * q) = f32x4{z[4 * q], z[4 * q + 1], z[4 * q + 2], z[4 * q + 3]};
    }
    return;
  }
  QuantParams qp[NGT];
#pragma unroll
  for (int g = 0; g < NGT; ++g) {
    float mx = z[g * VPG], mn = z[g * VPG];
#pragma unroll
    for (int v = 1; v < VPG; ++v) {
      mx = fmaxf(mx, z[g * VPG + v]);
      mn = fminf(mn, z[g * VPG + v]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    mn = fminf(mn, __shfl_xor(mn, 32));
    qp[g] = quant_params(mx, mn, alpha[g]);
  }
  // quotient estimates u for all 16 values and their nearest integers; the
  // exact division runs only where some estimate of this lane lies within
  // 2e-6 of a half-integer (a code boundary, or one the clamp makes
  // harmless); NaN and infinite estimates take that path too.
  float xs[16], rs[16];
  bool near = false;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const QuantParams &qq = qp[v / VPG];
    xs[v] = __fsub_rn(z[v], qq.zero_f);
    const float u = quant_u_estimate(xs[v], qq);
    rs[v] = rintf(u);
    near |= !(fabsf(u - rs[v]) < 0.5f - 2e-6f);  // (NaN: near)
  }
  if (near) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const QuantParams &qq = qp[v / VPG];
      const float u = quant_u_estimate(xs[v], qq);
      if (!(fabsf(u - rs[v]) < 0.5f - 2e-6f)) rs[v] = rintf(__fdiv_rn(xs[v], qq.scale_f));
    }
  }
  // four clamped codes c0..c3 make the byte c0 + 4 c1 + 16 c2 + 64 c3, an
  // integer that fp32 holds exactly; the conversion places it in the dword
  uint32_t dword = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float b = fminf(fmaxf(rs[4 * k + 3], 0.0f), 3.0f);
#pragma unroll
    for (int j = 2; j >= 0; --j) b = fmaf(b, 4.0f, fminf(fmaxf(rs[4 * k + j], 0.0f), 3.0f));
    dword = __builtin_amdgcn_cvt_pk_u8_f32(b, k, dword);
  }
  // a group with scale 0 (all values equal) gets code 0 throughout
#pragma unroll
  for (int g = 0; g < NGT; ++g)
    if (qp[g].scale_f == 0.0f) dword &= VPG == 16 ? 0u : ~(0xffffu << (16 * g));
  // lane hf=0 holds bytes 0,2,4,6 of the tile's 8 code bytes, hf=1 holds 1,3,5,7
  const uint32_t partner = __shfl_xor(dword, 32);
  const uint32_t packed = __builtin_amdgcn_perm(partner, dword, hf ? 0x03070206u : 0x05010400u);
  if (write) {
    reinterpret_cast<uint32_t *>(p.cache.codes + slot * (R / 4) + ch0 / 4)[hf] = packed;
    if (NGT == 1) {
      if (hf == 0) {
        const uint32_t sz = static_cast<uint32_t>(f16_bits(qp[0].scale)) |
                            (static_cast<uint32_t>(f16_bits(qp[0].zero)) << 16);
        reinterpret_cast<uint32_t *>(p.cache.scale_zero)[slot * (R / G) + ch0 / G] = sz;
      }
    } else {
      // lane half hf stores group hf's side info (selects, not a lane-indexed array)
      const uint32_t sz0 = static_cast<uint32_t>(f16_bits(qp[0].scale)) |
                           (static_cast<uint32_t>(f16_bits(qp[0].zero)) << 16);
      const uint32_t sz1 = static_cast<uint32_t>(f16_bits(qp[NGT - 1].scale)) |
                           (static_cast<uint32_t>(f16_bits(qp[NGT - 1].zero)) << 16);
      const uint32_t sz = hf ? sz1 : sz0;
      reinterpret_cast<uint32_t *>(p.cache.scale_zero)[slot * (R / G) + ch0 / G + hf] = sz;
    }
  }
}

// One 32-channel x 32-token tile of a small append (a decode step's few new
// tokens) by one wave: R_apply^T rows and latents go straight from memory
// into the MFMA operands, all at once (ALL) or in double-buffered chunks.
// Every accumulator sees the same MFMA sequence as in the LDS-staged kernel
// (K-steps in order, even/odd partial sums added at the end), so a token
// gets bit-identical codes whichever kernel appends it.
template <int R, int G, int NACC, bool ALL>
__device__ __forceinline__ void skinny_tile(const AppendParams &p, int ct, int ty, int l) {
  constexpr int KS = R / 16;
  constexpr int NGT = 32 / G;
  const int hf = l >> 5, l32 = l & 31;  // channels [32 ct, 32 ct + 32), tokens [32 ty, 32 ty + 32)
  const int64_t tok = static_cast<int64_t>(ty) * 32 + l32;
  const bool valid = tok < p.n;
  const bf16x8 *arow = reinterpret_cast<const bf16x8 *>(p.Rt + static_cast<int64_t>(32 * ct + l32) * R);
  const bf16x8 *brow =
      reinterpret_cast<const bf16x8 *>(static_cast<const uint16_t *>(p.latent) + (valid ? tok : 0) * p.lat_stride);
  int64_t slot = -1;
  float alpha[NGT] = {};
  if (p.z_out == nullptr) {
    if (valid) slot = p.slots[tok];
#pragma unroll
    for (int g = 0; g < NGT; ++g) alpha[g] = p.alpha[(32 * ct) / G + g];
  }
  f32x16 acc[NACC];
#pragma unroll
  for (int a = 0; a < NACC; ++a) acc[a] = f32x16{};
  // lanes of tokens past the end read token 0's row (their columns are never
  // stored), so the loads carry no branches
  if constexpr (ALL) {
    // every operand of the tile requested at once (one memory round trip;
    // 2 x KS loads per lane)
    bf16x8 aq[KS], bq[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      aq[ks] = arow[2 * ks + hf];
      bq[ks] = brow[2 * ks + hf];
    }
    __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the products
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      acc[ks % NACC] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[ks], bq[ks], acc[ks % NACC], 0, 0, 0);
  } else {
    // operands in chunks of 16 K-steps, one chunk of registers (for a wave
    // that shares its workgroup's register budget with other work): a
    // chunk's loads are issued as soon as the previous chunk's products are
    constexpr int PD = KS < 16 ? KS : 16;
    static_assert(KS % PD == 0, "K-steps come in whole chunks");
#pragma unroll
    for (int c = 0; c < KS / PD; ++c) {
      bf16x8 aq[PD], bq[PD];
#pragma unroll
      for (int j = 0; j < PD; ++j) {
        aq[j] = arow[2 * (c * PD + j) + hf];
        bq[j] = brow[2 * (c * PD + j) + hf];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < PD; ++j) {
        const int ks = c * PD + j;
        acc[ks % NACC] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[j], bq[j], acc[ks % NACC], 0, 0, 0);
      }
    }
  }
  f32x16 z = acc[0];
#pragma unroll
  for (int a = 1; a < NACC; ++a) z += acc[a];
  const bool write = valid && (p.z_out != nullptr || (slot >= 0 && slot < p.cache.capacity));
  tile_epilogue<R, G>(p, z, tok, write, slot, 32 * ct, alpha, hf);
  // side keys: the first channel tile copies its 32 tokens' keys
  if (ct == 0 && p.z_out == nullptr) {
    const int64_t t0 = static_cast<int64_t>(ty) * 32;
    const int cnt = static_cast<int>(min<int64_t>(32, p.n - t0));
    copy_side_keys(p.cache.k_rope, p.k_rope, p.d_r, p.slots, t0, cnt, p.cache.capacity, l);
    if (p.d_idx > 0) copy_side_keys(p.cache.idx_key, p.idx_key, p.d_idx, p.slots, t0, cnt, p.cache.capacity, l);
  }
}

// The same tile computed by wave 0 of a workgroup of four waves: all four
// stage the 32-token tile's latent rows in LDS (`lat`, 32 rows x R / 8
// pieces of 16 bytes, piece p of row t at p ^ (t & 15): the 16 lanes of a
// read hit separate banks) while wave 0 holds the R_apply^T rows of channel
// tile ct for all K-steps in registers, so all operands arrive in one memory
// round trip; the other waves return after the staging.  One channel tile
// per workgroup keeps the R_apply^T bytes each CU fetches at 32 rows.  The
// MFMA sequence is the one above, so the codes are the same bytes.  Side
// keys are not copied here (side_key_block).  Called by all threads of the
// workgroup.
template <int R, int G, int NACC>
__device__ __forceinline__ void staged_skinny_tile(const AppendParams &p, int ct, int ty, int tid,
                                                   u32x4 *__restrict__ lat) {
  const bool active = tid < 64;
  constexpr int KS = R / 16, PR = R / 8, PER = 32 * PR / 256;
  constexpr int NGT = 32 / G;
  static_assert(PER * 256 == 32 * PR, "whole rows per workgroup");
  const int l = tid & 63, hf = l >> 5, l32 = l & 31;
  const int64_t t0 = static_cast<int64_t>(ty) * 32, tok = t0 + l32;
  const bool valid = tok < p.n;
  // the tile's latent rows, piece tid + 256 j each (row 0 stands in for
  // tokens past the end: their columns are never stored)
  u32x4 lv[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = tid + 256 * j, t = e / PR, pc = e % PR;
    const int64_t row = t0 + t < p.n ? t0 + t : 0;
    lv[j] = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(p.latent) + row * p.lat_stride + 8 * pc);
  }
  const bf16x8 *arow = reinterpret_cast<const bf16x8 *>(p.Rt + static_cast<int64_t>(32 * ct + l32) * R);
  bf16x8 aq[KS];
  if (active) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) aq[ks] = arow[2 * ks + hf];
  }
  int64_t slot = -1;
  if (valid) slot = p.slots[tok];
  float alpha[NGT];
#pragma unroll
  for (int g = 0; g < NGT; ++g) alpha[g] = p.alpha[(32 * ct) / G + g];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = tid + 256 * j, t = e / PR, pc = e % PR;
    lat[t * PR + (pc ^ (t & 15))] = lv[j];
  }
  __syncthreads();
  if (!active) return;
  f32x16 acc[NACC];
#pragma unroll
  for (int a = 0; a < NACC; ++a) acc[a] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bf16x8 bq = __builtin_bit_cast(bf16x8, lat[l32 * PR + ((2 * ks + hf) ^ (l32 & 15))]);
    acc[ks % NACC] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[ks], bq, acc[ks % NACC], 0, 0, 0);
  }
  f32x16 z = acc[0];
#pragma unroll
  for (int a = 1; a < NACC; ++a) z += acc[a];
  const bool write = valid && slot >= 0 && slot < p.cache.capacity;
  tile_epilogue<R, G>(p, z, tok, write, slot, 32 * ct, alpha, hf);
}

// Side keys of the 32-token tile ty by a workgroup of four waves: wave 0 the
// bf16 rope keys (copied) or waves 0-1 the 4-bit rope keys (one thread per
// token and group of 16 dims, rope_quant_group); waves 2 and 3 the indexer
// keys of the tile's first and second 16 tokens.
__device__ __forceinline__ void side_key_block(const AppendParams &p, int ty, int tid) {
  const int64_t t0 = static_cast<int64_t>(ty) * 32;
  const int cnt = static_cast<int>(min<int64_t>(32, p.n - t0));
  const int wv = tid >> 6, lane = tid & 63;
  if (p.rope_bits == 4) {
    const int groups = p.d_r / 16;
    for (int u = tid; tid < 128 && u < cnt * groups; u += 128) {
      const int64_t tok = t0 + u / groups;
      const int64_t slot = p.slots[tok];
      if (slot >= 0 && slot < p.cache.capacity)
        rope_quant_group(p.k_rope, tok, u % groups, p.d_r, slot, reinterpret_cast<uint8_t *>(p.cache.k_rope));
    }
  } else if (wv == 0) {
    copy_side_keys(p.cache.k_rope, p.k_rope, p.d_r, p.slots, t0, cnt, p.cache.capacity, lane);
  }
  if (wv >= 2 && p.d_idx > 0) {
    const int h0 = 16 * (wv - 2), hc = min(16, cnt - h0);
    if (hc > 0) copy_side_keys(p.cache.idx_key, p.idx_key, p.d_idx, p.slots, t0 + h0, hc, p.cache.capacity, lane);
  }
}

}  // namespace
}  // namespace mla
