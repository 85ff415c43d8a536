// ga_internal.h -- launch descriptors passed from the C ABI layer (capi.cpp)
// to the kernel launchers (decode.hip, prefill.hip).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ga {

// GQA groups (G = H_q / H_kv) the kernels take: 1..16.  Decode serves a
// whole group in one workgroup (idle MFMA columns past G).  Prefill runs up to
// 8 heads per workgroup (one wave each); groups of 9..16 run as two parts of
// ceil(G/2) and floor(G/2) heads, each part streaming the kv head's K/V.
constexpr int kMaxHeadsPerPart = 8;
inline int head_parts(int group) { return group > kMaxHeadsPerPart ? 2 : 1; }
inline bool group_supported(int group) { return group >= 1 && group <= 2 * kMaxHeadsPerPart; }

struct DecodeLaunch {
  const uint16_t* q;
  const uint16_t* gate;
  const void* k_pool;  // bf16, or e4m3 codes when kv_fp8
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* kv_indptr;   // CSR row pointers [B + 1] (page size 1) or null
  const int32_t* kv_indices;  // CSR token slots
  long long index_capacity;   // entries of kv_indices
  int page_size;              // 16, or 1 (token slots)
  uint16_t* out;
  float* part_acc;  // workspace: [B][H_q][num_splits][D] fp32
  float* part_ml;   // workspace: [B][H_q][num_splits][2] fp32
  float scale;
  int kv_fp8;        // pools hold e4m3 codes: K = k_descale * code, V = v_descale * code
  float k_descale;   // 1 for bf16 pools
  float v_descale;
  int batch;
  int num_q_heads;
  int num_kv_heads;
  int max_pages;
  long long num_pages;
  int tokens_per_split;
  int num_splits;
  int split_target;  // workgroups the split sizing rule aims for
  // attention-spec options (null / 0: plain attention)
  const float* sinks;  // [H_q] sink logits
  float* lse;          // [B][H_q] log-sum-exp output
  int window;          // > 0: sliding window of that many keys
};

struct PrefillLaunch {
  const uint16_t* q;
  const uint16_t* gate;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float scale;
  int causal;
  int batch;
  int seq_len;
  int num_q_heads;
  int num_kv_heads;
  // attention-spec options (null / 0: plain attention)
  const int32_t* kv_lens;  // [B] key lengths
  const float* sinks;      // [H_q] sink logits
  float* lse;              // [B][S][H_q] log-sum-exp output
  int window;              // > 0: row i sees keys j > i - window
};

struct RopeLaunch {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* w_q;  // null: no norm (then w_k is null too)
  const uint16_t* w_k;
  const uint16_t* cos;  // [T][rope_dim]
  const uint16_t* sin;
  const int64_t* slot_mapping;  // null: dense K / V outputs
  uint16_t* q_out;
  uint16_t* k_out;
  uint16_t* v_out;
  float eps;
  long long num_tokens;
  long long num_slots;
  int num_q_heads;
  int num_kv_heads;
  int rope_dim;
};

// Unsigned 32-bit division by a divisor fixed for a launch, through one high
// multiply (Granlund and Montgomery, "Division by Invariant Integers using
// Multiplication", PLDI 1994, the unsigned algorithm of section 4): with
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1 (< 2^32),
// n / d = (t + ((n - t) >> min(l, 1))) >> max(l - 1, 0), t = (m n) >> 32,
// for every n < 2^32 and 1 <= d < 2^32.  divu32_make runs on the host;
// divu32 on either side.
struct DivU32 {
  uint32_t m;
  uint32_t s1, s2;
};
inline DivU32 divu32_make(uint32_t d) {
  uint32_t l = 0;
  while (l < 32 && ((uint64_t)1 << l) < d) ++l;
  DivU32 r;
  r.m = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1);
  r.s1 = l < 1 ? l : 1;
  r.s2 = l > 1 ? l - 1 : 0;
  return r;
}
__host__ __device__ inline uint32_t divu32(uint32_t n, DivU32 c) {
  const uint32_t t = (uint32_t)(((uint64_t)c.m * n) >> 32);
  return (t + ((n - t) >> c.s1)) >> c.s2;
}

hipError_t launch_decode(const DecodeLaunch& d, hipStream_t stream);
hipError_t launch_qk_norm_rope(const RopeLaunch& p, hipStream_t stream);
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);
hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t stream);

}  // namespace ga
