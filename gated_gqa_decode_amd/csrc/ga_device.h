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

// bf16(sigmoid(g)) for a bf16 gate g, correctly rounded: sigmoid is evaluated in
// fp64 (relative error a few 2^-53) and rounded once to bf16.  The closest any
// of the 65,536 gates comes to a bf16 rounding midpoint is ~2.5e-9 relative,
// far above the fp64 error, so the result equals the correctly rounded value
// for every gate (checked exhaustively through the public entry point).
__device__ __forceinline__ uint16_t sigmoid_bf16(uint16_t gate) {
  double g = (double)bf16_to_f32(gate);
  double s = 1.0 / (1.0 + exp(-g));
  return bf16_rne_f64(s);
}

// The gate epilogue: out = bf16(Ob * sigma_b).  The product of two bf16 values
// has at most 16 significant bits and is exact in fp64 at every magnitude,
// subnormal operands included, so the only rounding is the final one.
__device__ __forceinline__ uint16_t gate_output(uint16_t ob, uint16_t gate) {
  uint16_t sb = sigmoid_bf16(gate);
  double prod = (double)bf16_to_f32(ob) * (double)bf16_to_f32(sb);
  return bf16_rne_f64(prod);
}

// ---------------------------------------------------------------------------
// dot products and reductions
// ---------------------------------------------------------------------------
// acc + a.lo*b.lo + a.hi*b.hi on packed bf16 pairs, fp32 accumulate.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

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

// Reduce-scatter of 8 per-lane partial sums over an aligned group of 16 lanes
// (c16 = lane % 16): afterwards lane c16 holds the complete sum of entry
// c16 >> 1 (the two lanes c16 = 2h, 2h + 1 both hold entry h).  Three halving
// rounds pair lane i with 15 - i (row mirror: splits entries 0-3 / 4-7 by bit
// 3), with 7 - i inside each half-row (bit 2) and with i ^ 3 inside each quad
// (bit 1); each lane keeps the half it owns and adds the partner's copy of it.
// A last round sums the two lanes of a pair.  22 VALU operations instead of
// the 32 of eight separate all-reduces, and no select of the lane's entry.
constexpr int kDppQuadReverse = 0x1b;  // quad_perm [3,2,1,0]

__device__ __forceinline__ float reduce_scatter8(const float (&x)[8], int c16) {
  const bool b3 = (c16 & 8) != 0, b2 = (c16 & 4) != 0, b1 = (c16 & 2) != 0;
  float y[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float keep = b3 ? x[k + 4] : x[k];
    const float send = b3 ? x[k] : x[k + 4];
    y[k] = keep + dpp<kDppMirror>(send);
  }
  float z[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float keep = b2 ? y[k + 2] : y[k];
    const float send = b2 ? y[k] : y[k + 2];
    z[k] = keep + dpp<kDppHalfMirror>(send);
  }
  const float keep = b1 ? z[1] : z[0];
  const float send = b1 ? z[0] : z[1];
  float w = keep + dpp<kDppQuadReverse>(send);
  return w + dpp<kDppXor1>(w);
}

__device__ __forceinline__ float shfl_xor(float v, int mask) {
  int lane = __lane_id();
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(v)));
}

// Orders this wave's LDS writes before its later LDS reads of other lanes' data.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace ga
