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
//      registers straight into the fp16 B operands of the score MFMA
//      (v_mfma_f32_32x32x16_f16): z_hat = zero + scale * code with one fp16
//      rounding (codes enter as exact small integers);
//   2. partial scores S_w[64 rows x 32 tokens] = Q~_w Z_w^T (K = 128 + 16);
//   3. the partials are summed through LDS (each lane's accumulator slots
//      line up across waves), each wave runs the online softmax for 16 rows
//      (32-lane max/sum via DPP within 16 lanes + one lane swap), writes P^T
//      in fp16 to LDS;
//   4. O_w[64 x 128] += P Z_w with P and Z read back through the gfx950
//      transposing LDS load (ds_read_b64_tr_b16).
// The running max is only moved when a tile's max exceeds it by more than
// 8 (log2 units); otherwise p = 2^(s - m) <= 256 stays exact enough in fp16
// and O needs no rescaling.
#include "kernels.hpp"

namespace mla {
namespace {

constexpr int R = 512;
constexpr int DR = 64;
constexpr int ROWS = 64;        // query rows per workgroup
constexpr int TT = 32;          // tokens per tile
constexpr int KB = 9;           // K-blocks of 16 per wave: 8 latent + 1 rope
constexpr int ZSTRIDE = 144;    // halves per token row of the Z tile (128 + pad)
constexpr int PSTRIDE = 80;     // halves per token row of P^T (64 + pad)
constexpr float kRescaleThreshold = 8.0f;  // log2 units

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f16x4 ds_read_tr16(const f16 *p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<s16x4 __attribute__((address_space(3))) *>(
          reinterpret_cast<uintptr_t>(p)));
  return __builtin_bit_cast(f16x4, v);
}

// 16-lane all-reduce via DPP (xor 1, xor 2, half-row mirror, row mirror),
// then the two 16-lane rows of each 32-lane half are combined with a swap.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

template <bool kMax>
__device__ __forceinline__ float reduce32(float x) {
  auto op = [](float a, float b) { return kMax ? fmaxf(a, b) : a + b; };
  x = op(x, dpp_mov<0xB1>(x));     // quad_perm [1,0,3,2]
  x = op(x, dpp_mov<0x4E>(x));     // quad_perm [2,3,0,1]
  x = op(x, dpp_mov<0x141>(x));    // row_half_mirror
  x = op(x, dpp_mov<0x140>(x));    // row_mirror
  x = op(x, __shfl_xor(x, 16));
  return x;
}

// Channel of latent K-slot e (0..7) in K-block kb (0..7) for lane half hf,
// relative to the wave's first channel.  Matches the dequantisation below:
// half2 j of block kb holds the codes of channels 16*(kb/2) + 4*(kb%2) + j
// and that + 8.
__device__ __forceinline__ int slot_channel(int hf, int kb, int e) {
  return 64 * hf + 16 * (kb >> 1) + 4 * (kb & 1) + (e >> 1) + 8 * (e & 1);
}

struct __align__(16) Smem {
  float sp[4][32][64];              // partial scores, [wave][acc slot][lane]
  f16 z[4][TT * ZSTRIDE];           // dequantised latent tile per wave
  f16 pt[TT * PSTRIDE];             // P^T [token][row]
  float alpha[ROWS];
};

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

  // ---- softmax rows owned by this wave: acc slots rho = 8w .. 8w+7 ----
  // slot rho -> (mt = rho/16, v = rho%16) -> row 32mt + 8(v/4) + 4hf + v%4
  int srow[8], svis[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rho = 8 * w + i, mt = rho >> 4, v = rho & 15;
    srow[i] = 32 * mt + 8 * (v >> 2) + 4 * hf + (v & 3);
    const int m = rb * ROWS + srow[i];
    if (m < M) {
      const int t = m / H;
      svis[i] = a.causal ? (L - a.Tq + t + 1) : L;
    } else {
      svis[i] = -1;  // padding row: never visible
    }
  }
  float m_run[8], l_run[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.0f;
  }

  f32x16 o[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) o[mt][nt] = f32x16{};

  const uint32_t *codes32 = reinterpret_cast<const uint32_t *>(a.cache.codes);
  const uint16_t *sz16 = a.cache.scale_zero;
  const uint16_t *rope = a.cache.k_rope;
  constexpr int NG = R / G;                 // groups per token
  constexpr int GPL = 64 / G;               // groups per lane (2 or 4)
  const f16x2 k1024 = {static_cast<f16>(-1024.0f), static_cast<f16>(-1024.0f)};

  for (int t0 = it.t0; t0 < it.t1; t0 += TT) {
    // ---- 1. load + dequantise this lane's token into score B operands ----
    const int tau = t0 + l32;
    const bool tok_ok = tau < it.t1;
    const int64_t slot = base + (tok_ok ? tau : it.t0);
    const uint4 cw = *reinterpret_cast<const uint4 *>(codes32 + slot * (R / 16) + w * 8 + hf * 4);
    uint32_t szw[GPL];
    if (GPL == 2) {
      const uint2 s2 = *reinterpret_cast<const uint2 *>(sz16 + (slot * NG + (4 * w + 2 * hf)) * 2);
      szw[0] = s2.x;
      szw[1] = s2.y;
    } else {
      const uint4 s4 = *reinterpret_cast<const uint4 *>(sz16 + (slot * NG + (8 * w + 4 * hf)) * 2);
      szw[0] = s4.x;
      szw[1] = s4.y;
      szw[2 % GPL] = s4.z;
      szw[3 % GPL] = s4.w;
    }
    const uint4 rw = *reinterpret_cast<const uint4 *>(rope + slot * DR + 16 * w + 8 * hf);

    f16x8 bz[KB];
    const uint32_t cws[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const int q = kb >> 1;                       // dword: channels 16q..16q+15
      const int gi = (G == 32) ? (q >> 1) : q;     // group within the lane
      const uint32_t sz = szw[gi];
      const f16x2 sc = __builtin_bit_cast(f16x2, (sz & 0xffffu) * 0x10001u);
      const f16x2 zr = __builtin_bit_cast(f16x2, (sz >> 16) * 0x10001u);
      f16x8 v;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t x = ((cws[q] >> (2 * (4 * (kb & 1) + j))) & 0x00030003u) | 0x64006400u;
        const f16x2 c = __builtin_bit_cast(f16x2, x) + k1024;     // exact small integers
        const f16x2 z2 = __builtin_elementwise_fma(c, sc, zr);   // one rounding
        v[2 * j] = z2[0];
        v[2 * j + 1] = z2[1];
      }
      bz[kb] = v;
    }
    {
      const uint32_t rws[4] = {rw.x, rw.y, rw.z, rw.w};
      f16x8 v;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = static_cast<f16>(bf16_to_f32(static_cast<uint16_t>(rws[j] & 0xffffu)));
        v[2 * j + 1] = static_cast<f16>(bf16_to_f32(static_cast<uint16_t>(rws[j] >> 16)));
      }
      bz[8] = v;
    }

    // ---- 2. partial scores ----
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aq[mt][kb], bz[kb], sacc[mt], 0, 0, 0);

    // latent tile to LDS (wave-private), row = token, slots 64hf + 8kb + e
    f16 *zt = sm.z[w] + l32 * ZSTRIDE + 64 * hf;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) *reinterpret_cast<f16x8 *>(zt + 8 * kb) = bz[kb];
    // partial scores to LDS, slot-major and lane-contiguous
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) sm.sp[w][mt * 16 + v][l] = sacc[mt][v];
    __syncthreads();

    // ---- 3. reduce partials + online softmax for this wave's 16 rows ----
    bool any_rescale = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rho = 8 * w + i;
      float s = sm.sp[0][rho][l] + sm.sp[1][rho][l] + sm.sp[2][rho][l] + sm.sp[3][rho][l];
      if (!(tok_ok && tau < svis[i])) s = -INFINITY;
      const float tmax = reduce32<true>(s);
      float m_use = m_run[i];
      float alpha = 1.0f;
      if (tmax > m_use + kRescaleThreshold) {  // also true for the first visible tile
        alpha = (m_use == -INFINITY) ? 0.0f : exp2f(m_use - tmax);
        m_use = tmax;
        any_rescale = true;
      }
      const float p = (s == -INFINITY) ? 0.0f : exp2f(s - m_use);
      const float psum = reduce32<false>(p);
      l_run[i] = l_run[i] * alpha + psum;
      m_run[i] = m_use;
      sm.pt[l32 * PSTRIDE + srow[i]] = static_cast<f16>(p);
      if (l32 == 0) sm.alpha[srow[i]] = alpha;
    }
    // barrier that also tells every wave whether any row moved its max
    const int rescale = __syncthreads_or(any_rescale ? 1 : 0);

    // ---- 4. O = alpha * O + P Z ----
    if (rescale) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float al = sm.alpha[32 * mt + 8 * (v >> 2) + 4 * hf + (v & 3)];
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) o[mt][nt][v] *= al;
        }
    }
    const int g = l >> 4, s16 = l & 15;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      // source-lane addresses for the transposing loads: 4 tokens x 16 columns
      const int krow = 16 * ks + 8 * (g >> 1) + (s16 >> 2);
      const int col = 16 * (g & 1) + 4 * (s16 & 3);
      f16x8 pa[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const f16 *p0 = sm.pt + krow * PSTRIDE + 32 * mt + col;
        const f16x4 lo = ds_read_tr16(p0);
        const f16x4 hi = ds_read_tr16(p0 + 4 * PSTRIDE);
        pa[mt] = f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const f16 *z0 = sm.z[w] + krow * ZSTRIDE + 32 * nt + col;
        const f16x4 lo = ds_read_tr16(z0);
        const f16x4 hi = ds_read_tr16(z0 + 4 * ZSTRIDE);
        const f16x8 zb = f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          o[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa[mt], zb, o[mt][nt], 0, 0, 0);
      }
    }
  }

  // ---- write the partial (O, m, l) of this work item ----
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int sl = 32 * nt + l32;  // slot of the wave's Z tile
    const int ch = 128 * w + slot_channel(sl >> 6, (sl & 63) >> 3, sl & 7);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = rb * ROWS + 32 * mt + 8 * (v >> 2) + 4 * hf + (v & 3);
        if (m < M) a.part_o[(static_cast<int64_t>(item) * M + m) * R + ch] = o[mt][nt][v];
      }
  }
  if (l32 == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = rb * ROWS + srow[i];
      if (m < M) {
        a.part_ml[(static_cast<int64_t>(item) * M + m) * 2 + 0] = m_run[i];
        a.part_ml[(static_cast<int64_t>(item) * M + m) * 2 + 1] = l_run[i];
      }
    }
  }
}

// q~ = W~_UK[h]^T q_nope and q_rope, both times scale*log2(e), written in fp16
// straight into the per-lane operand order of splitk_mfma_kernel:
// [b][row block][wave][mt][kb][lane][8], zero for padding rows.
__global__ __launch_bounds__(256) void absorb_mfma_kernel(DecodeArgs a, int rb_count) {
  constexpr int RC = 16;
  extern __shared__ float qs_dyn[];
  const int h = blockIdx.x;
  const int H = a.d.num_heads, dn = a.d.qk_nope_head_dim;
  const int M = H * a.Tq;
  const int nrows = a.B * a.Tq;
  const int QP = dn + 1;
  f16 *qb = static_cast<f16 *>(a.qbuf);
  const uint16_t *wk = a.w_uk_f + static_cast<int64_t>(h) * dn * R;
  auto pos = [&](int b, int m, int w, int hf, int kb, int e) -> int64_t {
    const int rb = m / ROWS, mt = (m % ROWS) / 32, lane = (m % 32) + 32 * hf;
    return ((((static_cast<int64_t>(b) * rb_count + rb) * 4 + w) * 2 + mt) * KB + kb) * 512 + lane * 8 + e;
  };
  for (int q0 = 0; q0 < nrows; q0 += RC) {
    const int nr = min(RC, nrows - q0);
    __syncthreads();
    for (int e = threadIdx.x; e < nr * dn; e += 256) {
      const int i = e / dn, k = e % dn;
      qs_dyn[i * QP + k] = bf16_to_f32(a.q_nope[(static_cast<int64_t>(q0 + i) * H + h) * dn + k]);
    }
    __syncthreads();
    for (int j = threadIdx.x; j < R; j += 256) {
      float acc[RC];
#pragma unroll
      for (int i = 0; i < RC; ++i) acc[i] = 0.0f;
      for (int k = 0; k < dn; ++k) {
        const float wv = static_cast<float>(bits_f16(wk[static_cast<int64_t>(k) * R + j]));
#pragma unroll
        for (int i = 0; i < RC; ++i) acc[i] = fmaf(wv, qs_dyn[i * QP + k], acc[i]);
      }
      // inverse of slot_channel
      const int w = j >> 7, jj = j & 127, hf = jj >> 6, r6 = jj & 63;
      const int q = r6 >> 4, idx = r6 & 15, i8 = idx >> 3, rem = idx & 7;
      const int kb = 2 * q + (rem >> 2), e = 2 * (rem & 3) + i8;
      for (int i = 0; i < nr; ++i) {
        const int row = q0 + i, b = row / a.Tq, t = row % a.Tq, m = t * H + h;
        qb[pos(b, m, w, hf, kb, e)] = static_cast<f16>(acc[i] * a.scale_log2);
      }
    }
    for (int e = threadIdx.x; e < nr * DR; e += 256) {
      const int i = e / DR, k = e % DR;
      const int row = q0 + i, b = row / a.Tq, t = row % a.Tq, m = t * H + h;
      const float v = bf16_to_f32(a.q_rope[(static_cast<int64_t>(row) * H + h) * DR + k]) * a.scale_log2;
      qb[pos(b, m, k >> 4, (k >> 3) & 1, 8, k & 7)] = static_cast<f16>(v);
    }
  }
  // zero the padding rows of the last row block (one block does it)
  if (h == 0 && M % ROWS != 0) {
    const int pad = rb_count * ROWS - M;
    for (int b = 0; b < a.B; ++b)
      for (int e = threadIdx.x; e < pad * 4 * KB * 16; e += 256) {
        const int m = M + e / (4 * KB * 16);
        const int rest = e % (4 * KB * 16);
        const int w = rest / (KB * 16), kb = (rest / 16) % KB, hfe = rest % 16;
        qb[pos(b, m, w, hfe >> 3, kb, hfe & 7)] = static_cast<f16>(0.0f);
      }
  }
}

}  // namespace

bool mfma_decode_supported(const mla_dims &d, int rows) {
  return d.kv_lora_rank == R && d.qk_rope_head_dim == DR && (d.group_size == 32 || d.group_size == 16) &&
         rows >= 1;
}

int mfma_row_block() { return ROWS; }

hipError_t launch_absorb_mfma_layout(const DecodeArgs &a, hipStream_t s) {
  TimedLaunch tl("absorb_q", s);
  const int M = a.d.num_heads * a.Tq;
  const int rb_count = (M + ROWS - 1) / ROWS;
  const size_t lds = static_cast<size_t>(16) * (a.d.qk_nope_head_dim + 1) * sizeof(float);
  absorb_mfma_kernel<<<a.d.num_heads, 256, lds, s>>>(a, rb_count);
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

}  // namespace mla
