// ga_device.h -- device-side helpers shared by the gfx950 kernels of this
// library: bf16 packing and rounding, the exact bf16 sigmoid gate, wave-level
// reductions.  Written for CDNA4 (wave64) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ga {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// ---------------------------------------------------------------------------
// bf16 <-> fp32 / fp64
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even on the 16 dropped bits (the bf16 format is
// the upper half of binary32, so subnormals and the overflow to infinity follow
// from the same carry).  NaN stays NaN.
__device__ __forceinline__ uint16_t bf16_rne_f32(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp64 -> bf16, round to nearest even, with bf16 subnormals and overflow.
// Normal range: round the 52-bit fraction to 7 bits on the integer image of the
// value (a carry out of the fraction bumps the exponent, as it should).
// Subnormal range (|x| < 2^-126): the bf16 grid is the multiples of 2^-133, so
// scale by 2^133 (exact) and round to an integer with the hardware's
// ties-to-even rounding.
__device__ __forceinline__ uint16_t bf16_rne_f64(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
  uint64_t a = u & 0x7fffffffffffffffull;
  if (a > 0x7ff0000000000000ull) return (uint16_t)(sign | 0x7fc0u);
  double ad = __longlong_as_double((long long)a);
  if (ad < 0x1p-126) {
    double r = __builtin_rint(ad * 0x1p133);  // 0..128; 128 is the smallest normal
    return (uint16_t)(sign | (uint16_t)r);
  }
  uint64_t rounded = (a + 0x00000fffffffffffull + ((a >> 45) & 1ull)) >> 45;
  int64_t e = (int64_t)(rounded >> 7) - 1023 + 127;
  if (e >= 255) return (uint16_t)(sign | 0x7f80u);
  return (uint16_t)(sign | (uint16_t)((e << 7) | (int64_t)(rounded & 0x7fu)));
}

// bf16(sigmoid(g)) for a bf16 gate g, correctly rounded.
//
// Reference evaluation: sigmoid in fp64 (relative error a few 2^-53), rounded
// once to bf16.  The closest any of the 65,536 gates comes to a bf16 rounding
// midpoint is ~2.5e-9 relative, far above the fp64 error.
__device__ __forceinline__ uint16_t sigmoid_bf16_f64(uint16_t gate) {
  double g = (double)bf16_to_f32(gate);
  double s = 1.0 / (1.0 + exp(-g));
  return bf16_rne_f64(s);
}

// Fast path: sigmoid in fp32 for |g| <= 80, a few fp32 ulp of error.
// exp(-g) = 2^(-g log2 e) with Cody and Waite's two-part constant: log2 e =
// kLog2eHi + kLog2eLo, kLog2eHi = 23637 / 2^14 (15 significant bits), so
// -g kLog2eHi is exact for a bf16 g (8 significant bits); its nearest integer
// n splits it exactly into n + (t - n), and 2^(t - n - g kLog2eLo) (argument
// within +-0.51) comes from the hardware exp2, scaled by 2^n exactly.
// 1 / (1 + e) is the hardware reciprocal refined by one Newton step.
// Rounding the result to bf16 gives the correctly rounded sigmoid whenever it
// lies more than kSigmoidSlack fp32 ulps from a bf16 rounding midpoint, i.e.
// when its low 16 bits are not within kSigmoidSlack of 0x8000; the function
// then returns true.  Otherwise (about 0.05% of gates, every one whose
// sigmoid lies close to a midpoint among them), and for |g| > 80 or NaN, it
// returns false and the fp64 evaluation must decide.  Branch-free, so a
// caller can run it over many elements and fix the rare misses afterwards
// (the fp64 path for every element cost the prefill epilogue about 11% of
// the kernel's time).  All 65,536 gates are checked through both public entry
// points that apply the gate.
constexpr int kSigmoidSlack = 16;
constexpr float kLog2eHi = 23637.0f / 16384.0f;
constexpr float kLog2eLo = 7.052607543300837e-06f;  // log2(e) - kLog2eHi, rounded

__device__ __forceinline__ bool sigmoid_bf16_fast(uint16_t gate, uint16_t& res) {
  const float g = bf16_to_f32(gate);
  const float gc = __builtin_fminf(__builtin_fmaxf(g, -80.f), 80.f);  // keeps n finite
  const float t = -gc * kLog2eHi;  // exact
  const float n = __builtin_rintf(t);
  const float f = __builtin_fmaf(-gc, kLog2eLo, t - n);
  const float e = __builtin_ldexpf(__builtin_amdgcn_exp2f(f), (int)n);
  const float den = 1.0f + e;
  float s = __builtin_amdgcn_rcpf(den);
  s = __builtin_fmaf(__builtin_fmaf(-den, s, 1.0f), s, s);
  res = bf16_rne_f32(s);
  const int low = (int)(__float_as_uint(s) & 0xffffu) - 0x8000;
  return __builtin_fabsf(g) <= 80.f && (low > kSigmoidSlack || low < -kSigmoidSlack);
}

__device__ __forceinline__ uint16_t sigmoid_bf16(uint16_t gate) {
  uint16_t r;
  return sigmoid_bf16_fast(gate, r) ? r : sigmoid_bf16_f64(gate);
}

// bf16(Ob * sigma_b) for bf16 Ob and sigma_b: their product has at most 16
// significant bits, so it is exact in fp32 whenever it is a normal fp32 value
// and exact in fp64 at every magnitude (subnormals included); either way the
// only rounding is the final one.
__device__ __forceinline__ uint16_t gate_product(uint16_t ob, uint16_t sb) {
  const float p = bf16_to_f32(ob) * bf16_to_f32(sb);
  if (__builtin_fabsf(p) >= 0x1p-126f && __builtin_fabsf(p) <= 0x1p127f) return bf16_rne_f32(p);
  const double pd = (double)bf16_to_f32(ob) * (double)bf16_to_f32(sb);
  return bf16_rne_f64(pd);
}

// The gate epilogue: out = bf16(Ob * bf16(sigmoid(g))).
__device__ __forceinline__ uint16_t gate_output(uint16_t ob, uint16_t gate) {
  return gate_product(ob, sigmoid_bf16(gate));
}

// ---------------------------------------------------------------------------
// wave-level reductions
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}
// DPP controls (gfx9): quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_mirror.  Applied in this order to a value, they sum it over each aligned
// group of 16 lanes: after the two quad steps every quad holds one value, so the
// half-row mirror pairs quad 0 with quad 1, and the row mirror then pairs the
// two halves of the row.
constexpr int kDppXor1 = 0xb1;
constexpr int kDppXor2 = 0x4e;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

__device__ __forceinline__ float sum16(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  return v;
}

__device__ __forceinline__ float shfl_xor(float v, int mask) {
  int lane = __lane_id();
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(v)));
}

}  // namespace ga
