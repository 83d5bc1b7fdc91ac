// Shared device helpers and host-side plumbing of libmla (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "mla.h"

namespace mla {

// ---------------------------------------------------------------------------
// vector types for MFMA operands
// ---------------------------------------------------------------------------
typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// number formats
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// bf16 round-to-nearest-even (NaN kept quiet)
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint16_t f16_bits(f16 h) {
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ f16 bits_f16(uint16_t b) {
  return __builtin_bit_cast(f16, b);
}
// fp32 -> fp16 round to nearest even (the hardware default rounding mode)
__device__ __forceinline__ f16 f32_to_f16(float x) { return static_cast<f16>(x); }

// ---------------------------------------------------------------------------
// The INT2 group quantiser, step by step in IEEE fp32 with no contraction:
// every product and sum is rounded on its own (__f*_rn intrinsics), and the
// division is the correctly rounded one.  Both append paths and the clip fit
// use exactly these two functions.
// ---------------------------------------------------------------------------
struct QuantParams {
  f16 scale;
  f16 zero;
  float scale_f;  // f32(scale)
  float zero_f;   // f32(zero)
  float rcp;      // approximate 1 / scale_f (hardware reciprocal, within 1 ulp)
};

__device__ __forceinline__ QuantParams quant_params(float mx, float mn, float alpha) {
  const float mid = __fmul_rn(0.5f, __fadd_rn(mx, mn));
  const float half = __fmul_rn(0.5f, __fsub_rn(mx, mn));
  const float ah = __fmul_rn(alpha, half);
  const float lo = __fsub_rn(mid, ah);
  const float hi = __fadd_rn(mid, ah);
  const float scale32 = __fdiv_rn(__fsub_rn(hi, lo), 3.0f);
  QuantParams q;
  q.scale = f32_to_f16(scale32);
  q.zero = f32_to_f16(lo);
  q.scale_f = static_cast<float>(q.scale);
  q.zero_f = static_cast<float>(q.zero);
  q.rcp = __builtin_amdgcn_rcpf(q.scale_f);
  return q;
}

// code = clamp(rint(fl(x / scale)), 0, 3) with x = fl(z - zero) and fl()
// IEEE round-to-nearest division.  The code only depends on which side of
// the boundaries 0.5, 1.5, 2.5 the rounded quotient lies, so the quotient is
// first estimated as fl(x * rcp(scale)): for |u| < 4 it lies within 1e-6 of
// fl(x / scale) (reciprocal within 1 ulp, product and quotient each rounded
// once).  Only an estimate within 2e-6 of a boundary (or NaN) needs the
// exact division; the code is then the same as with exact division always.
__device__ __forceinline__ float quant_u_estimate(float x, const QuantParams &q) {
  return __fmul_rn(x, q.rcp);
}
__device__ __forceinline__ bool quant_u_near_boundary(float u) {
  const float dist = fminf(fminf(fabsf(u - 0.5f), fabsf(u - 1.5f)), fabsf(u - 2.5f));
  return !(dist > 2e-6f);
}
// fmaxf/fminf drop a NaN operand, so NaN maps to code 0
__device__ __forceinline__ uint32_t quant_code_from_u(float u) {
  return static_cast<uint32_t>(fminf(fmaxf(rintf(u), 0.0f), 3.0f));
}

__device__ __forceinline__ uint32_t quant_code(float z, const QuantParams &q) {
  if (q.scale_f == 0.0f) return 0u;
  const float x = __fsub_rn(z, q.zero_f);
  float u = quant_u_estimate(x, q);
  if (quant_u_near_boundary(u)) u = __fdiv_rn(x, q.scale_f);
  return quant_code_from_u(u);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
void set_error(const std::string &msg);
void clear_error();
mla_status fail(mla_status st, const std::string &msg);
mla_status hip_fail(hipError_t e, const char *what);
bool dims_valid(const mla_dims *d, std::string *why);
int device_cu_count();

// per-kernel event timing (no-ops unless enabled)
struct TimedLaunch {
  TimedLaunch(const char *name, hipStream_t s);
  ~TimedLaunch();
  const char *name_;
  hipStream_t stream_;
  void *start_;
};

}  // namespace mla

#define MLA_HIP_CHECK(expr, what)                          \
  do {                                                     \
    hipError_t _e = (expr);                                \
    if (_e != hipSuccess) return ::mla::hip_fail(_e, what); \
  } while (0)
