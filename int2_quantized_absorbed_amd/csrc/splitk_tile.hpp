// Tile machinery shared by the MFMA decode kernels (r = 512, d_r = 64
// latent layers; the grouped-query kernel reuses the dequantisation and the
// Z tile layout): constants, cache-tile loads, the exact INT2 -> fp16
// dequantisation, LDS layout and small wave-level helpers.
//
// [OSCAR issue #10, maintainer reply, "How the rotation adapts to the
// latent"]: the cached latent is the rotated INT2 latent, dequantised as
// zero + scale * code with the group's fp16 side information.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace mla {
namespace {


constexpr int R = 512;
constexpr int DR = 64;
constexpr int ROWS = 64;        // query rows per workgroup
constexpr int TT = 32;          // tokens per tile
constexpr int KB = 9;           // K-blocks of 16 per wave: 8 latent + 1 rope
// Z tile rows: 128 halves + 16 pad, so the four rows a transposing load
// reads fall in separate banks.  The 16-byte chunks of a row are stored
// XOR-swizzled by row bits (each kernel states its rule where it stores and
// reads the tile).
constexpr int ZSTRIDE = 144;
constexpr float kRescaleThreshold = 8.0f;  // log2 units
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008;     // MFMA
constexpr int kSchedDsWrite = 0x200;  // LDS write

// Orders the scheduling region that ends here as N pairs of one MFMA and
// one LDS store (the store first if STORE_FIRST), the rest after them.
// Issued in a burst, a wave's LDS stores queue at the LDS and hold up its
// next instructions; one per MFMA they drain while the MFMAs run.
template <int N, bool STORE_FIRST>
__device__ __forceinline__ void interleave_stores() {
#pragma unroll
  for (int k = 0; k < N; ++k) {
    if constexpr (STORE_FIRST) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    } else {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 1, 0);
    }
  }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f16x4 ds_read_tr16(const f16 *p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<s16x4 __attribute__((address_space(3))) *>(
          reinterpret_cast<uintptr_t>(p)));
  return __builtin_bit_cast(f16x4, v);
}

// ds_read_b64_tr_b16 at an LDS byte address
__device__ __forceinline__ f16x4 ds_read_tr16_lds(uint32_t addr) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<s16x4 __attribute__((address_space(3))) *>(static_cast<uintptr_t>(addr)));
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

// Tile state of the split-K kernel:
//   z   per channel slice, dequantised latent tile [token][slot] (PV B
//       operand), double-buffered
//   sp  partial scores [slice][acc slot][lane (+4 for hf = 1)]
//   p   P [row][token] (PV A operand), alpha per row, per-slice rescale flags
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
  uint4 rope;   // 8 bf16 rope values, or (4-bit rope key) .x 8 codes, .y (scale, zero)
};

// Bytes of one token's 4-bit rope-key entry at d_r = 64: 32 code bytes, then
// the (scale, zero) words of its 4 groups of 16 dims.
constexpr int kRopeEntry = DR / 2 + DR / 4;

// Tile operands of lane (token, lane half hf) of channel slice w: 64 latent
// channels' codes, their groups' side information and 8 rope dims (16w +
// 8hf ..).  RQ: the rope key is stored as 4-bit codes of group w.
template <int G, bool RQ = false>
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
  if (RQ) {
    const uint8_t *e = reinterpret_cast<const uint8_t *>(a.cache.k_rope) + slot * kRopeEntry;
    t.rope = uint4{*reinterpret_cast<const uint32_t *>(e + 8 * w + 4 * hf),
                   *reinterpret_cast<const uint32_t *>(e + DR / 2 + 4 * w), 0u, 0u};
  } else {
    t.rope = *reinterpret_cast<const uint4 *>(a.cache.k_rope + slot * DR + 16 * w + 8 * hf);
  }
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

// codes -> fp16.  Per code word (16 channels): two masks split the codes of
// channels (4j, 4j+2) and (4j+1, 4j+3) into nibbles, then per pair one
// conversion and one fused fp16 multiply-add with the group's (scale, zero):
// z_hat = zero + scale * c with one rounding.  Latent K-block kb (0..7) of
// the tile is code word kb / 2, pairs kb % 2: the eight channels
// slot_channel(hf, kb, 0..7) of the lane's slice.
template <int G>
__device__ __forceinline__ f16x8 dequant_block(const RawTile &t, int kb) {
  const uint32_t cws[4] = {t.codes.x, t.codes.y, t.codes.z, t.codes.w};
  const uint32_t szw[4] = {t.sz.x, t.sz.y, t.sz.z, t.sz.w};
  const int q = kb >> 1, odd = kb & 1;
  const uint32_t sz = szw[(G == 32) ? (q >> 1) : q];
  const f16x2 sc = __builtin_bit_cast(f16x2, (sz & 0xffffu) * 0x10001u);
  const f16x2 zr = __builtin_bit_cast(f16x2, (sz >> 16) * 0x10001u);
  const uint32_t u = (cws[q] >> (2 * odd)) & 0x33333333u;
  const f16x2 c0 = __builtin_elementwise_fma(code_pair<0>(u), sc, zr);
  const f16x2 c1 = __builtin_elementwise_fma(code_pair<1>(u), sc, zr);
  const f16x2 c2 = __builtin_elementwise_fma(code_pair<2>(u), sc, zr);
  const f16x2 c3 = __builtin_elementwise_fma(code_pair<3>(u), sc, zr);
  return f16x8{c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
}

// The rope K-block of the tile (8 rope dims) as fp16.
template <bool RQ>
__device__ __forceinline__ f16x8 dequant_rope(const RawTile &t) {
  f16x8 v;
  if (RQ) {
    // 4-bit rope codes: byte j holds dims 2j (low nibble) and 2j+1.  The
    // fp16 with bits 0x6400 | n is 1024 + n exactly, so subtracting 1024
    // gives the code; then k_hat = zero + scale * code with one rounding.
    const uint32_t c = t.rope.x, sz = t.rope.y;
    const f16x2 sc = __builtin_bit_cast(f16x2, (sz & 0xffffu) * 0x10001u);
    const f16x2 zr = __builtin_bit_cast(f16x2, (sz >> 16) * 0x10001u);
    const f16x2 k1024 = f16x2{static_cast<f16>(1024.0f), static_cast<f16>(1024.0f)};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t b = c >> (8 * j);
      const uint32_t pair = (b & 0xfu) | (((b >> 4) & 0xfu) << 16) | 0x64006400u;
      const f16x2 h = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, pair) - k1024, sc, zr);
      v[2 * j] = h[0];
      v[2 * j + 1] = h[1];
    }
  } else {
    const uint32_t rws[4] = {t.rope.x, t.rope.y, t.rope.z, t.rope.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = static_cast<f16>(__uint_as_float(rws[j] << 16));
      v[2 * j + 1] = static_cast<f16>(__uint_as_float(rws[j] & 0xffff0000u));
    }
  }
  return v;
}

// The whole tile: the score operands of the lane's slice (8 latent K-blocks
// and the rope K-block).
template <int G, bool RQ = false>
__device__ __forceinline__ void dequant(const RawTile &t, f16x8 (&bz)[KB]) {
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) bz[kb] = dequant_block<G>(t, kb);
  bz[8] = dequant_rope<RQ>(t);
}

}  // namespace
}  // namespace mla
