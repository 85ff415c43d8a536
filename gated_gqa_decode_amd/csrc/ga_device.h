// ga_device.h -- device-side helpers shared by the gfx950 kernels of this
// library: bf16 packing and rounding, the exact bf16 sigmoid gate, wave-level
// reductions.  Written for CDNA4 (wave64) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ga {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even on the 16 dropped bits (the bf16 format is
// the upper half of binary32, so subnormals and the overflow to infinity follow
// from the same carry).  NaN stays NaN.
__device__ __forceinline__ uint16_t bf16_rne_f32(float f) {
  // both results computed and one selected: no branch per element
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t quiet_nan = (u >> 16) | 0x0040u;
  return (uint16_t)(((u & 0x7fffffffu) > 0x7f800000u) ? quiet_nan : rounded);
}

// bf16(sigmoid(g)) for a bf16 gate g, correctly rounded.  A table holds the
// 4,096 gates of biased exponent 118..133 (|g| in [2^-9, 128)), written by
// gen_sigmoid_table.py with 60-digit decimal arithmetic and exact rational
// rounding; every other gate has a closed form the generator checks:
// |g| < 2^-9 -> 0.5, g >= 128 -> 1, g <= -128 -> +0, NaN -> NaN.  Entry
// (sign << 11) | ((exponent - 118) << 7) | mantissa.  All 65,536 gates are
// checked through the public entry points.
static __device__ const uint16_t kSigmoidTable[4096] = {
#include "sigmoid_bf16_table.inc"
};
constexpr uint32_t kSigmoidExpLo = 118, kSigmoidExpHi = 133;

__device__ __forceinline__ uint32_t sigmoid_table_slot(uint16_t gate) {
  const uint32_t e = (gate >> 7) & 0xffu;
  return ((uint32_t)(gate >> 15) << 11) | (((e - kSigmoidExpLo) & 15u) << 7) | (gate & 0x7fu);
}

// The result given the table entry at sigmoid_table_slot(gate) (ignored
// outside the table's range).
__device__ __forceinline__ uint16_t sigmoid_from_entry(uint16_t gate, uint16_t entry) {
  const uint32_t e = (gate >> 7) & 0xffu;
  uint16_t r = entry;
  if (e < kSigmoidExpLo) r = 0x3f00;
  if (e > kSigmoidExpHi) r = (gate & 0x8000u) ? 0 : 0x3f80;
  if (e == 0xffu && (gate & 0x7fu) != 0) r = 0x7fc0;
  return r;
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
