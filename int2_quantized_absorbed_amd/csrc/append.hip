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
//  * append_staged_kernel: bf16 latents, r in {128, 256, 384, 512}, more
//    than 1024 tokens.  The rotation z^T = R_apply^T c^T is a bf16 MFMA GEMM
//    (32x32x16, fp32 accumulate) with channels as the M dimension: each lane
//    then holds 16 channels of one token, so a 32-channel group is two lanes
//    (one cross-lane exchange for min/max) and the 2-bit codes of 4
//    consecutive channels form one byte in-lane.  The R_apply^T slice (128
//    channels x r) stays in LDS; latents arrive with coalesced loads and pass
//    through a per-wave LDS buffer into the MFMA B operands.
//  * append_skinny_kernel: the same shapes for appends of at most 1024 tokens
//    (a decode step's new tokens): one wave per 32-channel x 32-token tile,
//    operands straight from memory, the same MFMA sequence per accumulator.
//  * append_valu_kernel: any other shape and fp32 latents; the dot products
//    run in fp64 (exact products, fp64 sum) and are rounded once to fp32.
#include <atomic>

#include "append_tile.hpp"

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
constexpr int kSlice = 128;             // channels per block of the staged kernel (4 M-tiles of 32)
constexpr int kTokPerBlock = 256;       // tokens per block of the staged kernel

// Appends of more than kSkinnyMaxTokens tokens.  A block owns one 128-channel
// slice of R_apply^T, which stays in LDS for the whole block, and kTokPerBlock
// tokens.  Each of its WAVES waves owns 32 * NT tokens and computes all four
// 32-channel M-tiles of the slice for its NT token tiles, so an A operand
// read from LDS feeds NT products.  Latents reach the MFMA B operands through
// a per-wave LDS buffer, one K-chunk (64 values, 128 bytes of a token row) at
// a time: a chunk is fetched with fully coalesced 16-byte loads (8 lanes per
// token row), PF chunks ahead of the one being multiplied, and read back in
// operand order.  Both LDS regions are XOR-swizzled rather than padded, so
// the 16-byte operand reads of 16 consecutive lanes hit 64 distinct banks.
// Accumulation order per output: K-steps in order into even/odd partial sums
// added at the end, the same as append_skinny_kernel.
template <int R, int WAVES, int NT>
struct StagedCfg {
  static constexpr int KS = R / 16;           // MFMA K-steps
  static constexpr int KC = 4;                // K-steps per staged chunk
  static constexpr int NCH = KS / KC;         // chunks per token row
  static constexpr int TOKW = 32 * NT;        // tokens per wave
  static constexpr int NLD = TOKW / 8;        // 16-byte loads per lane per chunk
  static constexpr int THREADS = 64 * WAVES;
  static constexpr size_t RT_BYTES = static_cast<size_t>(kSlice) * R * 2;
  static constexpr size_t LDS = RT_BYTES + static_cast<size_t>(WAVES) * TOKW * 128;
  static_assert(WAVES * TOKW == kTokPerBlock, "a block covers one token tile");
};

// element offset of 16-byte chunk c of row `row` in the swizzled R_apply^T slice
template <int R>
__device__ __forceinline__ int rt_off(int row, int c) {
  return row * R + ((c ^ (row & 15)) << 3);
}
// byte offset of 16-byte piece j (0..7) of token t's row in a wave's chunk buffer
__device__ __forceinline__ int lat_off(int t, int j) {
  return t * 128 + ((j ^ ((t >> 1) & 7)) << 4);
}

template <int R, int G, int WAVES, int NT, int PF>
__global__ __launch_bounds__(64 * WAVES) void append_staged_kernel(AppendParams p,
                                                                                        int n_logical) {
  using C = StagedCfg<R, WAVES, NT>;
  constexpr int KS = C::KS, KC = C::KC, NCH = C::NCH, TOKW = C::TOKW, NLD = C::NLD, NSLICE = R / kSlice;
  static_assert(PF >= 1 && PF <= NCH, "prefetch depth within the row");
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
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
  uint16_t *rt_s = smem;
  uint8_t *lat_s = reinterpret_cast<uint8_t *>(smem) + C::RT_BYTES + static_cast<size_t>(w) * TOKW * 128;
  const int64_t wave_tok0 = static_cast<int64_t>(tb) * kTokPerBlock + w * TOKW;
  const uint16_t *lat = static_cast<const uint16_t *>(p.latent);

  // this thread's pieces of the R_apply^T slice (rows [cs*128, +128)) are
  // requested first: the products need them before anything else
  constexpr int CPR = R / 8;  // 16-byte pieces per row
  constexpr int RPT = kSlice * CPR / C::THREADS;  // pieces per thread
  static_assert(kSlice * CPR % C::THREADS == 0, "the slice splits evenly over the threads");
  u32x4 rv[RPT];
  {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(p.Rt + static_cast<int64_t>(cs) * kSlice * R);
#pragma unroll
    for (int j = 0; j < RPT; ++j) rv[j] = src[tid + C::THREADS * j];
  }
  // chunk loads: load i of a chunk brings 16 bytes (piece l & 7) of the
  // chunk's 128 bytes of token wave_tok0 + 8i + (l >> 3); tokens past the end
  // read the last token's row (their outputs are never stored)
  const uint16_t *rowp[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int64_t t = min<int64_t>(wave_tok0 + 8 * i + (l >> 3), p.n - 1);
    rowp[i] = lat + t * p.lat_stride + (l & 7) * 8;
  }
  uint4 buf[PF][NLD];
#pragma unroll
  for (int c = 0; c < PF; ++c)
#pragma unroll
    for (int i = 0; i < NLD; ++i) buf[c][i] = *reinterpret_cast<const uint4 *>(rowp[i] + c * 64);

  // epilogue inputs, fetched now so their latency hides under the GEMM
  constexpr int NGT = 32 / G;  // groups per M-tile: 1 (G=32) or 2 (G=16)
  int64_t slot[NT];
  float alpha_of[4][NGT] = {};  // (the rotation-only launch, z_out != nullptr, has no alpha)
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) slot[nt] = -1;
  if (p.z_out == nullptr) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int64_t tok = wave_tok0 + nt * 32 + l32;
      if (tok < p.n) slot[nt] = p.slots[tok];
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int g = 0; g < NGT; ++g) alpha_of[mt][g] = p.alpha[(cs * kSlice + mt * 32) / G + g];
  }

  // side keys: channel-slice block cs copies its share of this token tile
  // (ceil(kTokPerBlock / NSLICE) tokens), split over the waves.  When the
  // wave's share is at most one 16-byte piece per lane (the usual shapes),
  // the pieces are loaded here, in flight with the rotation staging below,
  // and stored after it; otherwise they are copied here.
  bool keys_deferred = false;
  uint4 kr_v = {}, ix_v = {};
  int64_t kr_sl = -1, ix_sl = -1;  // cache slots of the pieces (checked at store time)
  int kr_pc = 0, ix_pc = 0;        // piece index within the key
  if (p.z_out == nullptr) {
    constexpr int PB = (kTokPerBlock + NSLICE - 1) / NSLICE, PW = (PB + WAVES - 1) / WAVES;
    const int64_t tile_end = min<int64_t>(static_cast<int64_t>(tb + 1) * kTokPerBlock, p.n);
    const int64_t t0 = static_cast<int64_t>(tb) * kTokPerBlock + cs * PB + w * PW;
    const int64_t t1 = min<int64_t>(min<int64_t>(t0 + PW, static_cast<int64_t>(tb) * kTokPerBlock + (cs + 1) * PB), tile_end);
    const int cnt = static_cast<int>(t1 - t0);
    const int pr = p.d_r / 8, pi = p.d_idx / 8;  // 16-byte pieces per token
    keys_deferred = (p.d_r & 7) == 0 && (p.d_idx & 7) == 0 && cnt * pr <= 64 && cnt * pi <= 64;
    if (cnt > 0 && keys_deferred) {
      if (l < cnt * pr) {
        const int64_t t = t0 + l / pr;
        kr_sl = p.slots[t];
        kr_pc = l % pr;
        kr_v = reinterpret_cast<const uint4 *>(p.k_rope + t * p.d_r)[kr_pc];
      }
      if (pi > 0 && l < cnt * pi) {
        const int64_t t = t0 + l / pi;
        ix_sl = p.slots[t];
        ix_pc = l % pi;
        ix_v = reinterpret_cast<const uint4 *>(p.idx_key + t * p.d_idx)[ix_pc];
      }
    } else if (cnt > 0) {
      copy_side_keys(p.cache.k_rope, p.k_rope, p.d_r, p.slots, t0, cnt, p.cache.capacity, l);
      if (p.d_idx > 0) copy_side_keys(p.cache.idx_key, p.idx_key, p.d_idx, p.slots, t0, cnt, p.cache.capacity, l);
    }
  }

  // the R_apply^T slice into LDS
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int e = tid + C::THREADS * j;
    *reinterpret_cast<u32x4 *>(rt_s + rt_off<R>(e / CPR, e % CPR)) = rv[j];
  }
  __syncthreads();
  if (keys_deferred) {
    if (kr_sl >= 0 && kr_sl < p.cache.capacity)
      reinterpret_cast<uint4 *>(p.cache.k_rope + kr_sl * p.d_r)[kr_pc] = kr_v;
    if (ix_sl >= 0 && ix_sl < p.cache.capacity)
      reinterpret_cast<uint4 *>(p.cache.idx_key + ix_sl * p.d_idx)[ix_pc] = ix_v;
  }

  f32x16 acc[2][4][NT];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[a][mt][nt] = f32x16{};

  // a wave with no token in range skips the products
  if (wave_tok0 < p.n) {
    // A chunk goes registers -> this wave's LDS buffer, then the chunk PF
    // places further on is requested into the freed registers (the chunks in
    // flight move down one slot, so every register index is static).  LDS
    // instructions of one wave execute in order: a chunk's writes land after
    // the previous chunk's operand reads, and its operand reads after its
    // writes; the wave barriers only keep the compiler from moving LDS
    // accesses across them.  Software pipeline: the operands of a K-step are
    // requested before the products of the previous K-step issue (scheduling
    // fences keep that order), so LDS latency hides under the MFMAs.
    bf16x8 opa0[4], opb0[NT], opa1[4], opb1[NT];  // even / odd K-step operands
    static_assert(KC % 2 == 0, "K-steps come in even/odd pairs within a chunk");
#pragma unroll
    for (int ks = 0; ks < KS; ks += 2) {
      if (ks == 0) {
        // chunk 0: registers -> LDS, chunk PF requested into the freed
        // registers, then the operands of K-step 0
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < NLD; ++i)
          *reinterpret_cast<uint4 *>(lat_s + lat_off(8 * i + (l >> 3), l & 7)) = buf[0][i];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int f = 0; f + 1 < PF; ++f)
#pragma unroll
          for (int i = 0; i < NLD; ++i) buf[f][i] = buf[f + 1][i];
        if (PF < NCH) {
#pragma unroll
          for (int i = 0; i < NLD; ++i) buf[PF - 1][i] = *reinterpret_cast<const uint4 *>(rowp[i] + PF * 64);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          opa0[mt] = *reinterpret_cast<const bf16x8 *>(rt_s + rt_off<R>(mt * 32 + l32, hf));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          opb0[nt] = *reinterpret_cast<const bf16x8 *>(lat_s + lat_off(nt * 32 + l32, hf));
      }
      // odd K-step ks + 1 (same chunk)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        opa1[mt] = *reinterpret_cast<const bf16x8 *>(rt_s + rt_off<R>(mt * 32 + l32, 2 * (ks + 1) + hf));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        opb1[nt] = *reinterpret_cast<const bf16x8 *>(lat_s + lat_off(nt * 32 + l32, 2 * ((ks + 1) % KC) + hf));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[0][mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa0[mt], opb0[nt], acc[0][mt][nt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      // even K-step ks + 2, unless it starts a new chunk (then it is read
      // right after that chunk is staged)
      if (ks + 2 < KS && (ks + 2) % KC != 0) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          opa0[mt] = *reinterpret_cast<const bf16x8 *>(rt_s + rt_off<R>(mt * 32 + l32, 2 * (ks + 2) + hf));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          opb0[nt] = *reinterpret_cast<const bf16x8 *>(lat_s + lat_off(nt * 32 + l32, 2 * ((ks + 2) % KC) + hf));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[1][mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa1[mt], opb1[nt], acc[1][mt][nt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (ks + 2 < KS && (ks + 2) % KC == 0) {
        // the next chunk's first K-step: stage it now, then read its operands
        // while the odd products above run
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < NLD; ++i)
          *reinterpret_cast<uint4 *>(lat_s + lat_off(8 * i + (l >> 3), l & 7)) = buf[0][i];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int f = 0; f + 1 < PF; ++f)
#pragma unroll
          for (int i = 0; i < NLD; ++i) buf[f][i] = buf[f + 1][i];
        if ((ks + 2) / KC + PF < NCH) {
#pragma unroll
          for (int i = 0; i < NLD; ++i)
            buf[PF - 1][i] = *reinterpret_cast<const uint4 *>(rowp[i] + ((ks + 2) / KC + PF) * 64);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          opa0[mt] = *reinterpret_cast<const bf16x8 *>(rt_s + rt_off<R>(mt * 32 + l32, 2 * (ks + 2) + hf));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          opb0[nt] = *reinterpret_cast<const bf16x8 *>(lat_s + lat_off(nt * 32 + l32, hf));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // epilogue: lane holds channels 32mt + 8q + 4hf + s (v = 4q + s) of token
  // wave_tok0 + 32nt + l32
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int64_t tok = wave_tok0 + nt * 32 + l32;
    const bool write = tok < p.n && (p.z_out != nullptr || (slot[nt] >= 0 && slot[nt] < p.cache.capacity));
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const f32x16 z = acc[0][mt][nt] + acc[1][mt][nt];
      tile_epilogue<R, G>(p, z, tok, write, slot[nt], cs * kSlice + mt * 32, alpha_of[mt], hf);
    }
  }
}

// Small appends: one wave per (32-channel tile, 32-token tile), every
// operand requested at once.
template <int R, int G, int NACC>
__global__ __launch_bounds__(64) void append_skinny_kernel(AppendParams p) {
  skinny_tile<R, G, NACC, true>(p, blockIdx.x, blockIdx.y, threadIdx.x);
}

template <int R, int G, int WAVES, int NT, int PF>
hipError_t launch_staged(const AppendParams &p, hipStream_t s) {
  using C = StagedCfg<R, WAVES, NT>;
  constexpr int PFC = PF < C::NCH ? PF : C::NCH;
  const void *fn = reinterpret_cast<const void *>(&append_staged_kernel<R, G, WAVES, NT, PFC>);
  // the dynamic LDS limit is a per-device attribute of the function: set it
  // once on each device this instantiation launches on (devices past 63 set
  // it on every launch)
  static std::atomic<uint64_t> attr_set{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? uint64_t{1} << dev : 0;
  if (bit == 0 || (attr_set.load(std::memory_order_acquire) & bit) == 0) {
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(C::LDS));
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit, std::memory_order_release);
  }
  const int64_t blocks = ((p.n + kTokPerBlock - 1) / kTokPerBlock) * (R / kSlice);
  if (blocks > (int64_t{1} << 30)) return hipErrorInvalidValue;
  const int64_t grid = (blocks + 7) / 8 * 8;  // a multiple of 8 (XCD-aware order)
  append_staged_kernel<R, G, WAVES, NT, PFC>
      <<<static_cast<unsigned>(grid), C::THREADS, C::LDS, s>>>(p, static_cast<int>(blocks));
  return hipGetLastError();
}

template <int R, int G>
hipError_t launch_mfma_rg(const AppendParams &p, hipStream_t s) {
  constexpr int NACC = 2;
  if (p.n <= kSkinnyMaxTokens) {
    const dim3 grid(R / 32, static_cast<unsigned>((p.n + 31) / 32));
    append_skinny_kernel<R, G, NACC><<<grid, 64, 0, s>>>(p);
    return hipGetLastError();
  }
  // eight waves (two per SIMD), one 32-token tile each, three chunks in flight
  return launch_staged<R, G, 8, 1, 3>(p, s);
}

template <int R>
hipError_t launch_mfma_r(const AppendParams &p, hipStream_t s) {
  return p.G == 32 ? launch_mfma_rg<R, 32>(p, s) : launch_mfma_rg<R, 16>(p, s);
}

}  // namespace

bool append_fusable(const mla_dims &d, mla_dtype dt, int64_t n) {
  return dt == MLA_DTYPE_BF16 && d.kv_lora_rank == 512 && (d.rope_bits == 0 || d.rope_bits == 4) && n > 0 &&
         n <= kSkinnyMaxTokens;
}

// Rope-key variant: one thread per (token, group of 16 rope dims), see
// rope_quant_group.
__global__ __launch_bounds__(256) void rope_quant_kernel(const uint16_t *__restrict__ k_rope,
                                                         const int64_t *__restrict__ slots, int64_t n, int d_r,
                                                         uint8_t *__restrict__ entries, int64_t capacity) {
  const int groups = d_r / 16;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t tok = gid / groups;
  const int g = static_cast<int>(gid % groups);
  if (tok >= n) return;
  const int64_t slot = slots[tok];
  if (slot < 0 || slot >= capacity) return;
  rope_quant_group(k_rope, tok, g, d_r, slot, entries);
}

bool append_uses_mfma(const mla_dims &d, mla_dtype dt) {
  const int r = d.kv_lora_rank;
  return dt == MLA_DTYPE_BF16 && (r == 128 || r == 256 || r == 384 || r == 512);
}

hipError_t launch_append(const mla_dims &d, const void *latent, mla_dtype dt, const uint16_t *k_rope,
                         const uint16_t *idx_key, const int64_t *slots, int64_t n, const uint16_t *Rt,
                         const float *alpha, const mla_cache &cache, float *z_out, hipStream_t s,
                         int64_t lat_stride) {
  if (n <= 0) return hipSuccess;
  if (d.rope_bits == 4) {
    // the latent (and indexer key) through the latent kernels, the rope key
    // quantised on its own
    mla_dims dl = d;
    dl.rope_bits = 0;
    dl.qk_rope_head_dim = 0;
    hipError_t e = launch_append(dl, latent, dt, nullptr, idx_key, slots, n, Rt, alpha, cache, z_out, s, lat_stride);
    if (e != hipSuccess || z_out != nullptr) return e;
    TimedLaunch tl("append_rope", s);
    const int64_t threads = n * (d.qk_rope_head_dim / 16);
    rope_quant_kernel<<<static_cast<unsigned>((threads + 255) / 256), 256, 0, s>>>(
        k_rope, slots, n, d.qk_rope_head_dim, reinterpret_cast<uint8_t *>(cache.k_rope), cache.capacity);
    return hipGetLastError();
  }
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
  p.rope_bits = 0;
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
