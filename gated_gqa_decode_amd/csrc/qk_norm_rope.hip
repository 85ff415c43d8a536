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
// all of a wave's loads (row, norm weights, cos / sin, V) are issued before
// any is used.  At T = 4096 the kernel is bound by its vector instructions,
// not by memory, so the work per lane is kept small and free of divergent
// branches: the mean of squares takes one multiply by 1/D, the reciprocal
// square root is the hardware's, the bf16 rounding is the hardware's packed
// round-to-nearest-even conversion, and every lane loads the tables (lanes
// past rope_dim / 8 at a clamped, in-bounds address) and selects its result.
// The RoPE partner dims d +- rope_dim/2 sit rope_dim/16 lanes away; when that
// distance is a power of two they come from the partner lane's own normalised
// values by a swizzle (lane i reads lane i ^ (rope_dim/16) within its 32 lanes,
// bitwise what that lane computed); otherwise the partner's row and weights
// are loaded from memory and normalised with the same operations.  Key rows
// also carry that kv head's V row to the slot.
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
  uint32_t units;   // num_tokens * pairs (< 2^32: rows are at most 2^30)
  DivU32 by_pairs;  // division by pairs = ceil((H_q + H_kv) / 2)
};

__device__ __forceinline__ void unpack8(uint4 u, float (&f)[8]) {
  f[0] = bf16_lo(u.x);
  f[1] = bf16_hi(u.x);
  f[2] = bf16_lo(u.y);
  f[3] = bf16_hi(u.y);
  f[4] = bf16_lo(u.z);
  f[5] = bf16_hi(u.z);
  f[6] = bf16_lo(u.w);
  f[7] = bf16_hi(u.w);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (v_cvt_pk_bf16_f32: round to nearest even, denormals kept)
__device__ __forceinline__ uint32_t pack2(float x, float y) {
  const f32x2 v = {x, y};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint4 zero4() { return make_uint4(0, 0, 0, 0); }
__device__ __forceinline__ uint4 load16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
// the same from an address the compiler cannot see through (an integer made
// opaque, then a global pointer, so the load stays a global, not a flat, one)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef const u32x4 __attribute__((address_space(1)))* global_u32x4_ptr;
__device__ __forceinline__ uint4 load16_opaque(const uint16_t* p) {
  uint64_t u = reinterpret_cast<uintptr_t>(p);
  asm volatile("" : "+v"(u));
  const u32x4 v = *reinterpret_cast<global_u32x4_ptr>(u);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// every output row is written once and not read again by this kernel: the
// non-temporal hint (T = 4096 dense: 19.3-20.1 -> 17.7-17.9 us)
__device__ __forceinline__ void store16(uint16_t* p, uint4 v) {
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}

// lane i reads lane i ^ X of its 32-lane group (ds_swizzle, bit mode:
// and-mask 0x1f, or-mask 0, xor-mask X)
template <int X>
__device__ __forceinline__ float swizzle_xor(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1f | (X << 10)));
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

// kXor > 0: the RoPE partner is lane p ^ kXor (rope_dim = 16 kXor); 0: the
// partner dims are loaded from memory; -1: no rotation (rope_dim = 0).
template <int kXor>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(RopeArgs a) {
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int rows = Hq + Hkv;
  const int pairs = (rows + 1) >> 1;
  const uint32_t w = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (w >= a.units) return;
  const uint32_t t = divu32(w, a.by_pairs);  // wave-uniform
  const int pr = (int)(w - t * (uint32_t)pairs);
  const int lane = __lane_id();
  const int half = lane >> 5;
  const int p = lane & 31;  // dims 8p .. 8p + 7
  const int row_raw = 2 * pr + half;
  const int row = min(row_raw, rows - 1);  // past the end: a repeat, not stored
  const bool is_q = row < Hq;
  const int kvh = row - Hq;
  const int R = a.rope_dim;
  const int hr = R >> 1;
  const bool norm = a.w_q != nullptr;  // both or neither are given
  const uint16_t* xrow = is_q ? a.q + ((size_t)t * Hq + row) * kD : a.k + ((size_t)t * Hkv + kvh) * kD;
  const uint16_t* wn = is_q ? a.w_q : a.w_k;

  // ---- loads ------------------------------------------------------------------
  // All unconditional, so they are all in flight before the first wait: an
  // input that is not used this time (no norm, no rotation, no V) is replaced
  // by a second read of the lane's own row piece.  Lanes past R / 8 read the
  // last table group and ignore it.
  // (The selected addresses are made opaque: otherwise the compiler turns a
  // select of addresses into a select of a load and the row it already has,
  // and waits for that row before the branch.)
  const uint16_t* own = xrow + 8 * p;
  const bool copy_v = !is_q && a.v_out != nullptr;
  const size_t tab = (size_t)t * R + 8 * min(p, max((R >> 3) - 1, 0));
  const uint16_t* vsrc = copy_v ? a.v + ((size_t)t * Hkv + kvh) * kD + 8 * p : own;
  const uint16_t* wsrc = norm ? wn + 8 * p : own;
  const uint16_t* csrc = kXor >= 0 ? a.cos + tab : own;
  const uint16_t* ssrc = kXor >= 0 ? a.sin + tab : own;
  const uint4 xv = load16(own);
  const uint4 vv = load16_opaque(vsrc);
  const uint4 wv = load16_opaque(wsrc);
  uint4 cv = zero4(), sv = zero4();
  if constexpr (kXor >= 0) {
    cv = load16_opaque(csrc);
    sv = load16_opaque(ssrc);
  }
  // the token's slot (key rows), read from q's start when there is no mapping
  uint64_t su = a.slot_mapping != nullptr ? reinterpret_cast<uintptr_t>(a.slot_mapping + t)
                                          : reinterpret_cast<uintptr_t>(a.q);
  asm volatile("" : "+v"(su));
  const long long slot_read = *reinterpret_cast<const long long __attribute__((address_space(1)))*>(su);
  // kXor = 0: the partner dims of the row and the weights from memory.  Dims
  // 8p + 4g .. +3 (g = 0, 1) have partners 4g-aligned at +- R/2 (R/2 is a
  // multiple of 4); lanes past R / 8 read their own dims.
  uint4 xpv = xv, wpv = wv;
  if constexpr (kXor == 0) {  // (R > 0)
    int pofs[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int gd = 8 * p + 4 * g;
      pofs[g] = gd >= R ? gd : gd < hr ? gd + hr : gd - hr;  // lanes past R: their own dims
    }
    const uint16_t* wrow = norm ? wn : xrow;
    const uint2 x0 = *reinterpret_cast<const uint2*>(xrow + pofs[0]);
    const uint2 x1 = *reinterpret_cast<const uint2*>(xrow + pofs[1]);
    const uint2 w0 = *reinterpret_cast<const uint2*>(wrow + pofs[0]);
    const uint2 w1 = *reinterpret_cast<const uint2*>(wrow + pofs[1]);
    xpv = make_uint4(x0.x, x0.y, x1.x, x1.y);
    wpv = make_uint4(w0.x, w0.y, w1.x, w1.y);
  }
  // nothing below moves above the loads
  __builtin_amdgcn_sched_barrier(0);

  // ---- RMSNorm over the row's D values, in fp32 -------------------------------
  float x[8], y[8];
  unpack8(xv, x);
  float rr = 1.f;
  if (norm) {  // wave-uniform
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(x[e], x[e], ss);
    ss = half_sum(ss, half);
    rr = __builtin_amdgcn_rsqf(ss * (1.0f / kD) + a.eps);
    float wf[8];
    unpack8(wv, wf);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = x[e] * rr * wf[e];
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = x[e];
  }

  // ---- rotate-half RoPE on dims < R ---------------------------------------------
  // first half (d < R/2): z = y c - y' s; second half: z = y c + y' s, y' the
  // partner dim's normalised value
  float z[8];
  if constexpr (kXor >= 0) {
    float yp[8];
    if constexpr (kXor > 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) yp[e] = swizzle_xor<kXor>(y[e]);
    } else {
      float xp[8];
      unpack8(xpv, xp);
      if (norm) {
        float wpf[8];
        unpack8(wpv, wpf);
#pragma unroll
        for (int e = 0; e < 8; ++e) yp[e] = xp[e] * rr * wpf[e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) yp[e] = xp[e];
      }
    }
    float c[8], sn[8];
    unpack8(cv, c);
    unpack8(sv, sn);
    const bool rotated = 8 * p < R;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool first = 8 * p + 4 * (e >> 2) < hr;
      const float r = __builtin_fmaf(first ? -yp[e] : yp[e], sn[e], y[e] * c[e]);
      z[e] = rotated ? r : y[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = y[e];
  }

  // ---- stores -----------------------------------------------------------------------
  if (row_raw >= rows) return;  // the repeated last row: nothing to store
  const uint4 zo = make_uint4(pack2(z[0], z[1]), pack2(z[2], z[3]), pack2(z[4], z[5]), pack2(z[6], z[7]));
  if (is_q) {
    store16(a.q_out + ((size_t)t * Hq + row) * kD + 8 * p, zo);
    return;
  }
  // key row: K and V to the token's slot (or dense position)
  long long slot = t;
  if (a.slot_mapping != nullptr) {
    slot = slot_read;
    if (slot < 0 || slot >= a.num_slots) return;  // padded token / outside the pools
  }
  const size_t off = ((size_t)slot * Hkv + kvh) * kD + 8 * p;
  store16(a.k_out + off, zo);
  if (copy_v) store16(a.v_out + off, vv);
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
  const int pairs = (p.num_q_heads + p.num_kv_heads + 1) / 2;
  const long long units = p.num_tokens * pairs;
  a.units = (uint32_t)units;
  a.by_pairs = divu32_make((uint32_t)pairs);
  const dim3 grid((unsigned)((units + 3) / 4));
  // partners by swizzle when rope_dim / 16 is a power of two; no table at all
  // for rope_dim 0
  const int xr = p.rope_dim == 0 ? -1 : (p.rope_dim % 16 == 0) ? p.rope_dim / 16 : 0;
  switch (xr) {
    case -1: hipLaunchKernelGGL(qk_norm_rope_kernel<-1>, grid, dim3(256), 0, stream, a); break;
    case 1: hipLaunchKernelGGL(qk_norm_rope_kernel<1>, grid, dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(qk_norm_rope_kernel<2>, grid, dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL(qk_norm_rope_kernel<4>, grid, dim3(256), 0, stream, a); break;
    case 8: hipLaunchKernelGGL(qk_norm_rope_kernel<8>, grid, dim3(256), 0, stream, a); break;
    case 16: hipLaunchKernelGGL(qk_norm_rope_kernel<16>, grid, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL(qk_norm_rope_kernel<0>, grid, dim3(256), 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace ga
