// ga_internal.h -- launch descriptors passed from the C ABI layer (capi.cpp)
// to the kernel launchers (decode.hip, prefill.hip).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ga {

struct DecodeLaunch {
  const uint16_t* q;
  const uint16_t* gate;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  uint16_t* out;
  float* part_acc;  // workspace: [B][H_q][num_splits][D] fp32
  float* part_ml;   // workspace: [B][H_q][num_splits][2] fp32
  float scale;
  int batch;
  int num_kv_heads;
  int max_pages;
  long long num_pages;
  int tokens_per_split;
  int num_splits;
  hipEvent_t stage1_start;  // recorded around stage 1 when non-null
  hipEvent_t stage1_stop;
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
  int num_kv_heads;
};

hipError_t launch_decode(const DecodeLaunch& d, hipStream_t stream);
hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t stream);

}  // namespace ga
