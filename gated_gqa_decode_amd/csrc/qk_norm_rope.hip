// qk_norm_rope.hip -- the step before attention on gfx950: per-head
// QK-RMSNorm and partial rotate-half RoPE on q and k, with each token's K and
// V written to its slot of the paged pools (or to dense outputs).
//
// cuDNN FE-OSS "Gated Attention Block (SM107)", Overview stages (2)+(3): one
// kernel normalises each Q / K head row (optional) and applies RoPE to its
// first rope_dim dims; Weights and tables: cos, sin [.., rope_dim] in the
// activation dtype with the rotate-half convention, w_q_norm / w_k_norm [D];
// Fusion knobs: the rows are normed and rotated in fp32 and written once.
//
// One wave per (token, pair of head rows) -- H_q query rows, then H_kv key
// rows -- one row per half-wave: lane l handles dims 8(l % 32) .. +7 of its
// row, so every load and store moves a 512-byte row in 16-byte pieces, and
// all of a wave's loads (row, norm weights, cos / sin, V, and the RoPE
// partner dims d +- rope_dim/2 of the row and the weights) are issued before
// any is used; the only cross-lane step left is the norm's sum.  Key rows also
// carry that kv head's V row to the slot.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ga_device.h"
#include "ga_internal.h"

namespace ga {

namespace {

constexpr int kD = 256;

struct RopeArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* w_q;  // null: no norm
  const uint16_t* w_k;
  const uint16_t* cos;  // [T][rope_dim]
  const uint16_t* sin;
  const int64_t* slot_mapping;  // null: dense K / V outputs
  uint16_t* q_out;
  uint16_t* k_out;
  uint16_t* v_out;  // may be null in dense mode
  float eps;
  long long num_tokens;
  long long num_slots;  // pool slots (num_pages * page_size) in slot mode
  int num_q_heads;
  int num_kv_heads;
  int rope_dim;
};

__device__ __forceinline__ void unpack8(uint2 lo, uint2 hi, float (&f)[8]) {
  f[0] = bf16_lo(lo.x);
  f[1] = bf16_hi(lo.x);
  f[2] = bf16_lo(lo.y);
  f[3] = bf16_hi(lo.y);
  f[4] = bf16_lo(hi.x);
  f[5] = bf16_hi(hi.x);
  f[6] = bf16_lo(hi.y);
  f[7] = bf16_hi(hi.y);
}

__device__ __forceinline__ uint32_t pack2(float x, float y) {
  return (uint32_t)bf16_rne_f32(x) | ((uint32_t)bf16_rne_f32(y) << 16);
}

// 16 bytes at p (16-byte aligned), as two halves of 4 bf16 each.
struct Piece {
  uint2 lo, hi;
};
__device__ __forceinline__ Piece load16(const uint16_t* p) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  return {make_uint2(u.x, u.y), make_uint2(u.z, u.w)};
}
__device__ __forceinline__ void store16(uint16_t* p, Piece v) {
  *reinterpret_cast<uint4*>(p) = make_uint4(v.lo.x, v.lo.y, v.hi.x, v.hi.y);
}

}  // namespace

// Sum over each half-wave (32 lanes): DPP sums within each 16-lane row, then
// the two row sums of the lane's half read into scalar registers.
__device__ __forceinline__ float half_sum(float v, int half) {
  v = sum16(v);
  const int b = __float_as_int(v);
  const float h0 = __int_as_float(__builtin_amdgcn_readlane(b, 0)) +
                   __int_as_float(__builtin_amdgcn_readlane(b, 16));
  const float h1 = __int_as_float(__builtin_amdgcn_readlane(b, 32)) +
                   __int_as_float(__builtin_amdgcn_readlane(b, 48));
  return half ? h1 : h0;
}

// One (token, row pair) unit of work: what its loads bring, then what is
// stored.  load_pair issues every load; finish_pair uses them.
struct PairLoads {
  long long t;
  int row_raw;
  Piece x, xp, w, wp, c, s, v;
};

__device__ __forceinline__ PairLoads load_pair(const RopeArgs& a, long long w, int lane) {
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int rows = Hq + Hkv;
  const int pairs = (rows + 1) >> 1;
  const int half = lane >> 5;
  const int p = lane & 31;  // dims 8p .. 8p + 7
  PairLoads L;
  L.t = w / pairs;
  L.row_raw = 2 * (int)(w - L.t * pairs) + half;
  const int row = min(L.row_raw, rows - 1);  // past the end: a repeat, not stored
  const bool is_q = row < Hq;
  const int kvh = row - Hq;
  const int R = a.rope_dim;
  const bool rotated = 8 * p < R;
  const uint16_t* wn = is_q ? a.w_q : a.w_k;  // both or neither are given
  // The row, its norm weights, the token's tables, the V row, and -- instead
  // of a cross-lane exchange after the norm -- the RoPE partner dims of the
  // row and of the weights straight from memory (the partner's value is
  // formed from them with the same operations the partner lane applies, so it
  // is bitwise the same).  Dims 8p + 4g .. +3 (g = 0, 1) have partners
  // 4g-aligned at +- R/2 (R/2 is a multiple of 4).
  const uint16_t* xrow =
      is_q ? a.q + ((size_t)L.t * Hq + row) * kD : a.k + ((size_t)L.t * Hkv + kvh) * kD;
  L.x = load16(xrow + 8 * p);
  const Piece zero = {make_uint2(0, 0), make_uint2(0, 0)};
  L.xp = L.w = L.wp = L.c = L.s = L.v = zero;
  if (wn != nullptr) L.w = load16(wn + 8 * p);
  if (rotated) {
    const int hr = R >> 1;
    int pofs[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int gd = 8 * p + 4 * g;
      pofs[g] = gd < hr ? gd + hr : gd - hr;
    }
    L.c = load16(a.cos + (size_t)L.t * R + 8 * p);
    L.s = load16(a.sin + (size_t)L.t * R + 8 * p);
    if ((hr & 4) == 0) {  // the partners of all 8 dims are 8 contiguous dims
      L.xp = load16(xrow + pofs[0]);
      if (wn != nullptr) L.wp = load16(wn + pofs[0]);
    } else {              // two groups of 4 in different places
      L.xp = {*reinterpret_cast<const uint2*>(xrow + pofs[0]),
              *reinterpret_cast<const uint2*>(xrow + pofs[1])};
      if (wn != nullptr)
        L.wp = {*reinterpret_cast<const uint2*>(wn + pofs[0]),
                *reinterpret_cast<const uint2*>(wn + pofs[1])};
    }
  }
  if (!is_q && a.v_out != nullptr) L.v = load16(a.v + ((size_t)L.t * Hkv + kvh) * kD + 8 * p);
  return L;
}

__device__ __forceinline__ void finish_pair(const RopeArgs& a, const PairLoads& L, int lane) {
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int rows = Hq + Hkv;
  const int half = lane >> 5;
  const int p = lane & 31;
  const int row = min(L.row_raw, rows - 1);
  const bool is_q = row < Hq;
  const int kvh = row - Hq;
  const int R = a.rope_dim;
  const bool rotated = 8 * p < R;
  const int hr = R >> 1;
  float x[8], xp[8];
  unpack8(L.x.lo, L.x.hi, x);
  unpack8(L.xp.lo, L.xp.hi, xp);
  // RMSNorm over the row's D values, in fp32
  float y[8], yp[8];
  if (a.w_q != nullptr) {  // wave-uniform
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
    ss = half_sum(ss, half);
    const float rr = 1.0f / sqrtf(ss / (float)kD + a.eps);
    float wf[8], wpf[8];
    unpack8(L.w.lo, L.w.hi, wf);
    unpack8(L.wp.lo, L.wp.hi, wpf);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      y[e] = x[e] * rr * wf[e];
      yp[e] = xp[e] * rr * wpf[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      y[e] = x[e];
      yp[e] = xp[e];
    }
  }
  // rotate-half RoPE on dims < R: first half z = y c - y' s, second half
  // z = y c + y' s, y' the partner dim d +- R/2
  float c[8], sn[8];
  unpack8(L.c.lo, L.c.hi, c);
  unpack8(L.s.lo, L.s.hi, sn);
  float z[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const bool first = 8 * p + 4 * (e >> 2) < hr;
    z[e] = !rotated ? y[e] : first ? y[e] * c[e] - yp[e] * sn[e] : y[e] * c[e] + yp[e] * sn[e];
  }
  if (L.row_raw >= rows) return;  // the repeated last row: nothing to store
  const Piece zo = {make_uint2(pack2(z[0], z[1]), pack2(z[2], z[3])),
                    make_uint2(pack2(z[4], z[5]), pack2(z[6], z[7]))};
  if (is_q) {
    store16(a.q_out + ((size_t)L.t * Hq + row) * kD + 8 * p, zo);
    return;
  }
  // key row: K and V to the token's slot (or dense position)
  long long slot = L.t;
  if (a.slot_mapping != nullptr) {
    slot = a.slot_mapping[L.t];
    if (slot < 0 || slot >= a.num_slots) return;  // padded token / outside the pools
  }
  const size_t off = ((size_t)slot * Hkv + kvh) * kD + 8 * p;
  store16(a.k_out + off, zo);
  if (a.v_out != nullptr) store16(a.v_out + off, L.v);
}

// One row pair per wave, all its loads issued before any is used.  (Two or
// four pairs per wave keep more bytes in flight per wave but need so many
// registers that fewer waves fit: measured slower at T = 4096.)
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(RopeArgs a) {
  const long long units = a.num_tokens * ((a.num_q_heads + a.num_kv_heads + 1) >> 1);
  const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= units) return;
  const int lane = __lane_id();
  finish_pair(a, load_pair(a, w, lane), lane);
}

hipError_t launch_qk_norm_rope(const RopeLaunch& p, hipStream_t stream) {
  RopeArgs a;
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.w_q = p.w_q;
  a.w_k = p.w_k;
  a.cos = p.cos;
  a.sin = p.sin;
  a.slot_mapping = p.slot_mapping;
  a.q_out = p.q_out;
  a.k_out = p.k_out;
  a.v_out = p.v_out;
  a.eps = p.eps;
  a.num_tokens = p.num_tokens;
  a.num_slots = p.num_slots;
  a.num_q_heads = p.num_q_heads;
  a.num_kv_heads = p.num_kv_heads;
  a.rope_dim = p.rope_dim;
  // one (token, pair of head rows) unit per wave, four waves per workgroup
  const long long units = p.num_tokens * ((p.num_q_heads + p.num_kv_heads + 1) / 2);
  hipLaunchKernelGGL(qk_norm_rope_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, stream,
                     a);
  return hipGetLastError();
}

}  // namespace ga
