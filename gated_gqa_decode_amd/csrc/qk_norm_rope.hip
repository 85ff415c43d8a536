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
// Rows are (token, head row): H_q query rows, then H_kv key rows, each of
// which also copies that kv head's V row.  Lane l owns dims 4l .. 4l+3, so a
// row is one 8-byte load and one 8-byte store per lane; the RoPE partner of
// dim d (d +- rope_dim/2) sits in the lane rope_dim/8 away, at the same
// position, and is fetched with one cross-lane permute per element.
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

__device__ __forceinline__ void unpack4(uint2 u, float (&f)[4]) {
  f[0] = bf16_lo(u.x);
  f[1] = bf16_hi(u.x);
  f[2] = bf16_lo(u.y);
  f[3] = bf16_hi(u.y);
}

__device__ __forceinline__ uint2 pack4(const float (&f)[4]) {
  uint2 u;
  u.x = (uint32_t)bf16_rne_f32(f[0]) | ((uint32_t)bf16_rne_f32(f[1]) << 16);
  u.y = (uint32_t)bf16_rne_f32(f[2]) | ((uint32_t)bf16_rne_f32(f[3]) << 16);
  return u;
}

__device__ __forceinline__ float from_lane(float v, int src_lane) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src_lane << 2, __float_as_int(v)));
}

}  // namespace

// Rows per wave.  More than one keeps more bytes in flight but lengthens
// each wave's chain of cross-lane steps; measured at T = 4096 and T = 64, one
// row per wave is as fast or faster.
constexpr int kRows = 1;

// Sum over the wave: DPP sums within each 16-lane row, then the four row sums
// read into scalar registers (no LDS-routed permutes on the chain).
__device__ __forceinline__ float wave_sum_rows(float v) {
  v = sum16(v);
  const int b = __float_as_int(v);
  return (__int_as_float(__builtin_amdgcn_readlane(b, 0)) +
          __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(b, 32)) +
          __int_as_float(__builtin_amdgcn_readlane(b, 48)));
}

__global__ __launch_bounds__(256) void qk_norm_rope_kernel(RopeArgs a) {
  const int rows_per_token = a.num_q_heads + a.num_kv_heads;
  const long long total = a.num_tokens * rows_per_token;
  const long long row0 = ((long long)blockIdx.x * 4 + (threadIdx.x >> 6)) * kRows;
  if (row0 >= total) return;
  const int lane = __lane_id();
  const int R = a.rope_dim;
  const bool rotated = 4 * lane < R;

  long long tok[kRows];
  int hrow[kRows];
  uint2 xraw[kRows], wraw[kRows], craw[kRows], sraw[kRows];
#pragma unroll
  for (int j = 0; j < kRows; ++j) {
    const long long row = min(row0 + j, total - 1);  // past the end: redo the last row, unstored
    tok[j] = row / rows_per_token;
    hrow[j] = (int)(row - tok[j] * rows_per_token);
    const bool is_q = hrow[j] < a.num_q_heads;
    const uint16_t* src = is_q ? a.q + ((size_t)tok[j] * a.num_q_heads + hrow[j]) * kD
                               : a.k + ((size_t)tok[j] * a.num_kv_heads + (hrow[j] - a.num_q_heads)) * kD;
    xraw[j] = *reinterpret_cast<const uint2*>(src + 4 * lane);
    const uint16_t* w = is_q ? a.w_q : a.w_k;
    wraw[j] = w != nullptr ? *reinterpret_cast<const uint2*>(w + 4 * lane) : make_uint2(0, 0);
    craw[j] = sraw[j] = make_uint2(0, 0);
    if (rotated) {
      craw[j] = *reinterpret_cast<const uint2*>(a.cos + (size_t)tok[j] * R + 4 * lane);
      sraw[j] = *reinterpret_cast<const uint2*>(a.sin + (size_t)tok[j] * R + 4 * lane);
    }
  }

#pragma unroll
  for (int j = 0; j < kRows; ++j) {
    const long long t = tok[j];
    const int hr = hrow[j];
    const bool is_q = hr < a.num_q_heads;
    float x[4];
    unpack4(xraw[j], x);

    // RMSNorm over the head's D values, in fp32
    float y[4] = {x[0], x[1], x[2], x[3]};
    if ((is_q ? a.w_q : a.w_k) != nullptr) {
      const float ss = wave_sum_rows(x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3]);
      const float r = 1.0f / sqrtf(ss / (float)kD + a.eps);
      float wf[4];
      unpack4(wraw[j], wf);
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = x[e] * r * wf[e];
    }

    // rotate-half RoPE on dims < R: first half z = y c - y' s, second half
    // z = y c + y' s, with y' the partner dim R/2 away (R/8 lanes away)
    float z[4] = {y[0], y[1], y[2], y[3]};
    {
      const int half_lanes = R >> 3;
      const bool first = lane < half_lanes;
      const int partner = first ? lane + half_lanes : lane - half_lanes;
      float yp[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) yp[e] = from_lane(y[e], rotated ? partner : lane);
      if (rotated) {
        float c[4], s[4];
        unpack4(craw[j], c);
        unpack4(sraw[j], s);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          z[e] = first ? y[e] * c[e] - yp[e] * s[e] : y[e] * c[e] + yp[e] * s[e];
      }
    }
    if (row0 + j >= total) continue;  // a repeated last row: nothing to store
    const uint2 zout = pack4(z);
    if (is_q) {
      *reinterpret_cast<uint2*>(a.q_out + ((size_t)t * a.num_q_heads + hr) * kD + 4 * lane) = zout;
      continue;
    }
    // key row: K and V to the token's slot (or dense position)
    const int kvh = hr - a.num_q_heads;
    long long slot = t;
    if (a.slot_mapping != nullptr) {
      slot = a.slot_mapping[t];
      if (slot < 0 || slot >= a.num_slots) continue;  // padded token / outside the pools
    }
    const size_t off = ((size_t)slot * a.num_kv_heads + kvh) * kD + 4 * lane;
    *reinterpret_cast<uint2*>(a.k_out + off) = zout;
    if (a.v_out != nullptr)
      *reinterpret_cast<uint2*>(a.v_out + off) =
          *reinterpret_cast<const uint2*>(a.v + ((size_t)t * a.num_kv_heads + kvh) * kD + 4 * lane);
  }
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
  const long long rows = p.num_tokens * (p.num_q_heads + p.num_kv_heads);
  const long long waves = (rows + kRows - 1) / kRows;
  hipLaunchKernelGGL(qk_norm_rope_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ga
