// Quantise-on-append: rotate each incoming latent token by R_apply, clip and
// INT2-quantise it group by group, pack 2-bit codes with fp16 scale/zero,
// and copy the bf16 rope key (and indexer key) into its cache slot.
//
// [OSCAR issue #10, maintainer reply, "How the rotation adapts to the
// latent"]: the cache holds the rotated, INT2-quantised latent; low-variance
// eigen-directions (the first channels of z, ascending order) share groups.
// [llm-helper PR #64, PR description]: a latent layer stores the latent, the
// rotary key and (GLM-5.3-Flash) the indexer key per token.
//
// Kernels, chosen by input dtype and shape; for bf16 latents the token count
// only picks between two kernels that give bit-identical results, so one
// layer always quantises a token the same way:
//  * append_mfma_kernel: bf16 latents, r in {128, 256, 384, 512}.  The
//    rotation z^T = R_apply^T c^T is a bf16 MFMA GEMM (32x32x16, fp32
//    accumulate) with channels as the M dimension: each lane then holds 16
//    channels of one token, so a 32-channel group is two lanes (one cross-lane
//    exchange for min/max) and the 2-bit codes of 4 consecutive channels form
//    one byte in-lane.  The R_apply^T slice (128 channels x r) stays in LDS;
//    latents stream from HBM straight into MFMA B operands.
//  * append_skinny_kernel: the same shapes for appends of at most 1024 tokens
//    (a decode step's new tokens): one wave per 32-channel x 32-token tile,
//    operands straight from memory, the same MFMA sequence per accumulator.
//  * append_valu_kernel: any other shape and fp32 latents; the dot products
//    run in fp64 (exact products, fp64 sum) and are rounded once to fp32.
#include "kernels.hpp"

namespace mla {
namespace {

// Copy one token's bf16 side key (width values) with the widest aligned moves.
__device__ __forceinline__ void copy_key(uint16_t *__restrict__ dst, const uint16_t *__restrict__ src,
                                         int width, int lane, int nlanes) {
  if ((width & 7) == 0) {
    const uint4 *s4 = reinterpret_cast<const uint4 *>(src);
    uint4 *d4 = reinterpret_cast<uint4 *>(dst);
    for (int e = lane; e < width / 8; e += nlanes) d4[e] = s4[e];
  } else {
    const uint32_t *s1 = reinterpret_cast<const uint32_t *>(src);
    uint32_t *d1 = reinterpret_cast<uint32_t *>(dst);
    for (int e = lane; e < width / 2; e += nlanes) d1[e] = s1[e];
  }
}

template <typename T>
__device__ __forceinline__ double latent_f64(const T *p, int64_t i);
template <>
__device__ __forceinline__ double latent_f64<float>(const float *p, int64_t i) {
  return static_cast<double>(p[i]);
}
template <>
__device__ __forceinline__ double latent_f64<uint16_t>(const uint16_t *p, int64_t i) {
  return static_cast<double>(bf16_to_f32(p[i]));
}

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
};

// One block per token, one thread per output channel (blockDim == r <= 1024).
template <typename T>
__global__ __launch_bounds__(1024) void append_valu_kernel(AppendParams p) {
  extern __shared__ double cs[];
  const int64_t tok = blockIdx.x;
  const int j = threadIdx.x;
  const int r = p.r;
  const T *lat = static_cast<const T *>(p.latent);
  int64_t slot = -1;
  if (p.z_out == nullptr) {
    slot = p.slots[tok];
    if (slot < 0 || slot >= p.cache.capacity) return;  // uniform per block
  }
  for (int i = j; i < r; i += blockDim.x) cs[i] = latent_f64<T>(lat, tok * p.lat_stride + i);
  __syncthreads();
  const uint16_t *row = p.Rt + static_cast<int64_t>(j) * r;
  double acc = 0.0;
  for (int i = 0; i < r; i += 8) {
    const uint4 w = *reinterpret_cast<const uint4 *>(row + i);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc = fma(cs[i + 2 * k], static_cast<double>(bf16_to_f32(static_cast<uint16_t>(ww[k] & 0xffffu))), acc);
      acc = fma(cs[i + 2 * k + 1], static_cast<double>(bf16_to_f32(static_cast<uint16_t>(ww[k] >> 16))), acc);
    }
  }
  const float z = static_cast<float>(acc);  // one rounding, to nearest even
  if (p.z_out != nullptr) {
    p.z_out[tok * r + j] = z;
    return;
  }
  const int G = p.G;
  float mx = z, mn = z;
  for (int off = G / 2; off > 0; off >>= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, off));
    mn = fminf(mn, __shfl_xor(mn, off));
  }
  const QuantParams q = quant_params(mx, mn, p.alpha[j / G]);
  const uint32_t code = quant_code(z, q);
  const uint32_t c1 = __shfl_down(code, 1), c2 = __shfl_down(code, 2), c3 = __shfl_down(code, 3);
  if ((j & 3) == 0)
    p.cache.codes[slot * (r / 4) + j / 4] = static_cast<uint8_t>(code | (c1 << 2) | (c2 << 4) | (c3 << 6));
  if (j % G == 0) {
    const uint32_t sz = static_cast<uint32_t>(f16_bits(q.scale)) | (static_cast<uint32_t>(f16_bits(q.zero)) << 16);
    reinterpret_cast<uint32_t *>(p.cache.scale_zero)[slot * (r / G) + j / G] = sz;
  }
  copy_key(p.cache.k_rope + slot * p.d_r, p.k_rope + tok * p.d_r, p.d_r, j, blockDim.x);
  if (p.d_idx > 0)
    copy_key(p.cache.idx_key + slot * p.d_idx, p.idx_key + tok * p.d_idx, p.d_idx, j, blockDim.x);
}

// ---------------------------------------------------------------------------
// MFMA path
// ---------------------------------------------------------------------------
constexpr int kSlice = 128;       // channels per block (4 M-tiles of 32)
constexpr int kWaves = 8;         // two waves per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kTokPerWave = 32;   // one N-tile of 32 tokens
constexpr int kTokPerBlock = kWaves * kTokPerWave;
constexpr int kSkinnyMaxTokens = 1024;  // appends of at most this many tokens use append_skinny_kernel

template <int R>
constexpr int lds_stride() { return R + 8; }  // +16 B per row: rows rotate banks

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
  // quotient estimates for all 16 values; the exact division runs only
  // when some value of the wave lies next to a code boundary
  float xs[16], us[16];
  bool near = false;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const QuantParams &qq = qp[v / VPG];
    xs[v] = __fsub_rn(z[v], qq.zero_f);
    us[v] = quant_u_estimate(xs[v], qq);
    near |= qq.scale_f != 0.0f && quant_u_near_boundary(us[v]);
  }
  if (near) {
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if (quant_u_near_boundary(us[v])) us[v] = __fdiv_rn(xs[v], qp[v / VPG].scale_f);
  }
  uint32_t dword = 0;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const uint32_t code = qp[v / VPG].scale_f == 0.0f ? 0u : quant_code_from_u(us[v]);
    dword |= code << (2 * v);
  }
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
      const QuantParams &qh = qp[hf & (NGT - 1)];
      const uint32_t sz = static_cast<uint32_t>(f16_bits(qh.scale)) |
                          (static_cast<uint32_t>(f16_bits(qh.zero)) << 16);
      reinterpret_cast<uint32_t *>(p.cache.scale_zero)[slot * (R / G) + ch0 / G + hf] = sz;
    }
  }
}

template <int R, int G, int NACC>
__global__ __launch_bounds__(kThreads) void append_mfma_kernel(AppendParams p, int n_logical) {
  extern __shared__ __attribute__((aligned(16))) uint16_t rt_s[];
  constexpr int KS = R / 16;
  constexpr int NSLICE = R / kSlice;
  constexpr int LS = lds_stride<R>();
  // XCD-aware order: blocks b, b + 8, ... run on one XCD (one L2); give them
  // consecutive logical indices, so the NSLICE channel-slice blocks of a
  // token tile read its latents through the same L2
  const int per_xcd = static_cast<int>(gridDim.x / 8);
  const int logical = static_cast<int>(blockIdx.x % 8) * per_xcd + static_cast<int>(blockIdx.x / 8);
  if (logical >= n_logical) return;  // grid padding (whole block)
  const int cs = logical % NSLICE;
  const int tb = logical / NSLICE;
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, hf = l >> 5, l32 = l & 31;

  // this wave's 32 tokens; lanes of tokens past the end read token 0's row
  // (their output columns are never stored), so every load is unconditional
  const int64_t wave_tok0 = static_cast<int64_t>(tb) * kTokPerBlock + w * kTokPerWave;
  const int64_t tok = wave_tok0 + l32;
  const bool valid = tok < p.n;
  const bf16x8 *brow = reinterpret_cast<const bf16x8 *>(static_cast<const uint16_t *>(p.latent) + (valid ? tok : 0) * p.lat_stride);
  // epilogue inputs, fetched now so their latency hides under the GEMM
  constexpr int NGT = 32 / G;  // groups per M-tile: 1 (G=32) or 2 (G=16)
  int64_t slot = -1;
  float alpha_of[4][NGT] = {};  // (the rotation-only launch, z_out != nullptr, has no alpha)
  if (p.z_out == nullptr) {
    if (valid) slot = p.slots[tok];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int g = 0; g < NGT; ++g) alpha_of[mt][g] = p.alpha[(cs * kSlice + mt * 32) / G + g];
  }
  const bool live = wave_tok0 < p.n;  // a wave with no token in range skips the products

  f32x16 acc[NACC][4];
#pragma unroll
  for (int a = 0; a < NACC; ++a)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[a][mt] = f32x16{};

  // latent operands stream from HBM in chunks of PD K-steps, double-buffered:
  // chunk c + 1 is in flight while chunk c is multiplied
  constexpr int PD = 8;
  static_assert(KS % PD == 0, "K-steps come in whole chunks");
  bf16x8 bq[2][PD];
#pragma unroll
  for (int j = 0; j < PD; ++j) bq[0][j] = brow[2 * j + hf];
  // stage R_apply^T rows [cs*128, +128) into LDS (16-byte chunks, several
  // loads in flight per thread) while the first latent chunk is in flight
  {
    const uint4 *src = reinterpret_cast<const uint4 *>(p.Rt + static_cast<int64_t>(cs) * kSlice * R);
    constexpr int CPR = R / 8;  // chunks per row
    constexpr int TOTAL = kSlice * CPR;
    constexpr int SU = TOTAL % (kThreads * 16) == 0 ? 16 : (TOTAL % (kThreads * 8) == 0 ? 8 : 4);
    static_assert(TOTAL % (kThreads * SU) == 0, "staging loop has no tail");
    for (int e0 = tid; e0 < TOTAL; e0 += kThreads * SU) {
      uint4 v[SU];
#pragma unroll
      for (int j = 0; j < SU; ++j) v[j] = src[e0 + kThreads * j];
#pragma unroll
      for (int j = 0; j < SU; ++j) {
        const int e = e0 + kThreads * j, row = e / CPR, c = e % CPR;
        *reinterpret_cast<uint4 *>(rt_s + row * LS + c * 8) = v[j];
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < KS / PD; ++c) {
    if (!live) break;
    const int cur = c & 1;
    if (c + 1 < KS / PD) {
#pragma unroll
      for (int j = 0; j < PD; ++j) bq[cur ^ 1][j] = brow[2 * ((c + 1) * PD + j) + hf];
    }
#pragma unroll
    for (int j = 0; j < PD; ++j) {
      const int ks = c * PD + j;
      bf16x8 a[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        a[mt] = *reinterpret_cast<const bf16x8 *>(rt_s + (mt * 32 + l32) * LS + ks * 16 + hf * 8);
      const int par = ks % NACC;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        acc[par][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mt], bq[cur][j], acc[par][mt], 0, 0, 0);
    }
  }

  // epilogue: lane holds channels 32mt + 8q + 4hf + s (v = 4q + s) of token tok
  const bool write = valid && (p.z_out != nullptr || (slot >= 0 && slot < p.cache.capacity));
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    f32x16 z = acc[0][mt];
#pragma unroll
    for (int a = 1; a < NACC; ++a) z += acc[a][mt];
    tile_epilogue<R, G>(p, z, tok, write, slot, cs * kSlice + mt * 32, alpha_of[mt], hf);
  }
  // side keys: channel-slice block cs copies its share of this 256-token
  // tile (ceil(256 / NSLICE) tokens), an eighth of that per wave, every lane
  // moving 16-byte pieces
  if (p.z_out == nullptr) {
    constexpr int PB = (kTokPerBlock + NSLICE - 1) / NSLICE, PW = (PB + kWaves - 1) / kWaves;
    const int64_t tile_end = min<int64_t>(static_cast<int64_t>(tb + 1) * kTokPerBlock, p.n);
    const int64_t t0 = static_cast<int64_t>(tb) * kTokPerBlock + cs * PB + w * PW;
    const int64_t t1 = min<int64_t>(min<int64_t>(t0 + PW, static_cast<int64_t>(tb) * kTokPerBlock + (cs + 1) * PB), tile_end);
    const int cnt = static_cast<int>(t1 - t0);
    if (cnt > 0) {
      copy_side_keys(p.cache.k_rope, p.k_rope, p.d_r, p.slots, t0, cnt, p.cache.capacity, l);
      if (p.d_idx > 0) copy_side_keys(p.cache.idx_key, p.idx_key, p.d_idx, p.slots, t0, cnt, p.cache.capacity, l);
    }
  }
}

// Small appends (a decode step's few new tokens): one wave per (32-channel
// tile, 32-token tile).  R_apply^T rows and latents go straight from memory
// into the MFMA operands (8 K-steps per double-buffered chunk), and every
// accumulator sees the same MFMA sequence as in append_mfma_kernel (K-steps
// in order, even/odd partial sums added at the end), so a token gets
// bit-identical codes whichever kernel appends it.
template <int R, int G, int NACC>
__global__ __launch_bounds__(64) void append_skinny_kernel(AppendParams p) {
  constexpr int KS = R / 16, PD = 8;
  static_assert(KS % PD == 0, "K-steps come in whole chunks");
  constexpr int NGT = 32 / G;
  const int ct = blockIdx.x;  // channels [32 ct, 32 ct + 32)
  const int l = threadIdx.x, hf = l >> 5, l32 = l & 31;
  const int64_t tok = static_cast<int64_t>(blockIdx.y) * 32 + l32;
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
  // lanes of tokens past the end read token 0's row (their columns are never
  // stored), so the loads carry no branches
  bf16x8 aq[2][PD], bq[2][PD];
#pragma unroll
  for (int j = 0; j < PD; ++j) {
    aq[0][j] = arow[2 * j + hf];
    bq[0][j] = brow[2 * j + hf];
  }
  f32x16 acc[NACC];
#pragma unroll
  for (int a = 0; a < NACC; ++a) acc[a] = f32x16{};
#pragma unroll
  for (int c = 0; c < KS / PD; ++c) {
    const int cur = c & 1;
    if (c + 1 < KS / PD) {
#pragma unroll
      for (int j = 0; j < PD; ++j) {
        aq[cur ^ 1][j] = arow[2 * ((c + 1) * PD + j) + hf];
        bq[cur ^ 1][j] = brow[2 * ((c + 1) * PD + j) + hf];
      }
    }
#pragma unroll
    for (int j = 0; j < PD; ++j) {
      const int ks = c * PD + j;
      acc[ks % NACC] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[cur][j], bq[cur][j], acc[ks % NACC], 0, 0, 0);
    }
  }
  f32x16 z = acc[0];
#pragma unroll
  for (int a = 1; a < NACC; ++a) z += acc[a];
  const bool write = valid && (p.z_out != nullptr || (slot >= 0 && slot < p.cache.capacity));
  tile_epilogue<R, G>(p, z, tok, write, slot, 32 * ct, alpha, hf);
  // side keys: the first channel tile copies its 32 tokens' keys
  if (ct == 0 && p.z_out == nullptr) {
    const int64_t t0 = static_cast<int64_t>(blockIdx.y) * 32;
    const int cnt = static_cast<int>(min<int64_t>(32, p.n - t0));
    copy_side_keys(p.cache.k_rope, p.k_rope, p.d_r, p.slots, t0, cnt, p.cache.capacity, l);
    if (p.d_idx > 0) copy_side_keys(p.cache.idx_key, p.idx_key, p.d_idx, p.slots, t0, cnt, p.cache.capacity, l);
  }
}

template <int R, int G>
hipError_t launch_mfma_rg(const AppendParams &p, hipStream_t s) {
  constexpr int NACC = 2;
  if (p.n <= kSkinnyMaxTokens) {
    const dim3 grid(R / 32, static_cast<unsigned>((p.n + 31) / 32));
    append_skinny_kernel<R, G, NACC><<<grid, 64, 0, s>>>(p);
    return hipGetLastError();
  }
  const size_t lds = static_cast<size_t>(kSlice) * lds_stride<R>() * sizeof(uint16_t);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&append_mfma_kernel<R, G, NACC>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t blocks = ((p.n + kTokPerBlock - 1) / kTokPerBlock) * (R / kSlice);
  if (blocks > (int64_t{1} << 30)) return hipErrorInvalidValue;
  const int64_t grid = (blocks + 7) / 8 * 8;  // a multiple of 8 (XCD-aware order)
  append_mfma_kernel<R, G, NACC><<<static_cast<unsigned>(grid), kThreads, lds, s>>>(p, static_cast<int>(blocks));
  return hipGetLastError();
}

template <int R>
hipError_t launch_mfma_r(const AppendParams &p, hipStream_t s) {
  return p.G == 32 ? launch_mfma_rg<R, 32>(p, s) : launch_mfma_rg<R, 16>(p, s);
}

}  // namespace

bool append_uses_mfma(const mla_dims &d, mla_dtype dt) {
  const int r = d.kv_lora_rank;
  return dt == MLA_DTYPE_BF16 && (r == 128 || r == 256 || r == 384 || r == 512);
}

hipError_t launch_append(const mla_dims &d, const void *latent, mla_dtype dt, const uint16_t *k_rope,
                         const uint16_t *idx_key, const int64_t *slots, int64_t n, const uint16_t *Rt,
                         const float *alpha, const mla_cache &cache, float *z_out, hipStream_t s,
                         int64_t lat_stride) {
  if (n <= 0) return hipSuccess;
  TimedLaunch tl("append_quant", s);
  AppendParams p;
  p.latent = latent;
  p.k_rope = k_rope;
  p.idx_key = idx_key;
  p.slots = slots;
  p.n = n;
  p.Rt = Rt;
  p.alpha = alpha;
  p.cache = cache;
  p.z_out = z_out;
  p.lat_stride = lat_stride > 0 ? lat_stride : d.kv_lora_rank;
  p.r = d.kv_lora_rank;
  p.G = d.group_size;
  p.d_r = d.qk_rope_head_dim;
  p.d_idx = d.index_head_dim;
  if (append_uses_mfma(d, dt)) {
    switch (p.r) {
      case 128: return launch_mfma_r<128>(p, s);
      case 256: return launch_mfma_r<256>(p, s);
      case 384: return launch_mfma_r<384>(p, s);
      default: return launch_mfma_r<512>(p, s);
    }
  }
  const size_t lds = static_cast<size_t>(p.r) * sizeof(double);
  if (dt == MLA_DTYPE_FP32)
    append_valu_kernel<float><<<static_cast<unsigned>(n), p.r, lds, s>>>(p);
  else
    append_valu_kernel<uint16_t><<<static_cast<unsigned>(n), p.r, lds, s>>>(p);
  return hipGetLastError();
}

}  // namespace mla
