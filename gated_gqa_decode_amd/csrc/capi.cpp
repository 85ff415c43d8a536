// capi.cpp -- the extern "C" boundary of libgated_attn.so (include/gated_attn.h):
// argument validation, split planning, workspace sizing, device check, launch.
//
// Every check that the host can make runs before anything is enqueued (cuDNN
// "Gated Attention Block", Forward: typed errors rather than a failed launch;
// FreeToken PR #781, Summary: validate before touching KV storage).  Nothing
// here allocates, synchronises or reads device memory.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "ga_internal.h"
#include "gated_attn.h"

#ifndef GA_DECODE_TARGET_BLOCKS
// Stage-1 workgroups a decode call aims for: one per compute unit of the
// 256-CU MI355X (stage 1 runs one 8-wave workgroup per CU), so long sequences
// run as few, long workgroups whose start-up and merge costs are amortised
// over many tokens.  Two 4-wave workgroups per CU were measured to finish far
// apart (the CU serves the older one first: 72 us vs 104 us at B=64, L=4096),
// leaving half the CU idle for the last third of the kernel.
#define GA_DECODE_TARGET_BLOCKS 256
#endif
static_assert((GA_DECODE_TARGET_BLOCKS & (GA_DECODE_TARGET_BLOCKS - 1)) == 0,
              "the device divides by the target with a shift");

namespace {

constexpr int kHeadDim = 256;
constexpr int kPageSize = 16;
constexpr int kSplitQuantum = 64;   // splits are whole 4-page groups
// The largest split.  At page size 1 the split's token slots are staged in
// LDS, which holds 2,048.  With 16-token pages and fewer (sequence, kv head)
// pairs than target workgroups: up to 16,384 tokens (a wave keeps the page ids
// of its up to 128 tiles in two registers), so the capacity-fixed grid holds
// few splits and a short sequence in a large capacity leaves few empty
// workgroups behind.  As many pairs as target workgroups or more: 4,096, so
// long sequences still split into several workgroups each, while each
// workgroup streams enough tokens to amortise its start (measured at B=224,
// L 4094..6142: 369 us per call with 4,096-token splits, 380 us with 2,048).
constexpr int kMaxSplitTokens = 4096;
constexpr int kMaxTokSplitTokens = 2048;
constexpr int kMaxLongSplitTokens = 16384;
// A launch's grid size times its workgroup size must stay below 2^32 threads:
// decode stage 1 and prefill have 512 threads per workgroup (2^22 workgroups:
// 2^31 threads), decode stage 2 has one 64-thread workgroup per (sequence,
// query head) row (2^25 rows: 2^31 threads).  These are the only limits on the
// batch.
constexpr int64_t kMaxStage1Workgroups = (int64_t)1 << 22;
constexpr int64_t kMaxPrefillWorkgroups = (int64_t)1 << 22;
constexpr int64_t kMaxDecodeRows = (int64_t)1 << 25;

thread_local int g_last_hip_error = 0;

// Device memory of gated_attn_decode_noalloc: the fp32 split partials that
// gated_attn_decode keeps in the caller's workspace.  Every GPU the library
// runs on holds its own copy from the code object's load until the process
// ends.  Host code never uses the name itself (on the host it stands for a
// host-side shadow, not a device address): the device address comes from
// hipGetSymbolAddress, once per device, and only that pointer is passed on.
constexpr size_t kScratchBytes = GA_DECODE_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

ga_status hip_fail(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return GA_ERR_HIP;
}

// gfx950 check for the current device, cached per device id.
ga_status check_device() {
  static std::atomic<int> cache[64];  // 0 unknown, 1 gfx950, 2 other
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev >= 0 && dev < 64) {
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c == 1) return GA_OK;
    if (c == 2) return GA_ERR_UNSUPPORTED;
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_fail(e);
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < 64) cache[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? GA_OK : GA_ERR_UNSUPPORTED;
}

// This device's copy of `scratch`: its address is looked up on the first call
// with the device current and kept.
ga_status device_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return GA_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e);
      if (p == nullptr) return hip_fail(hipErrorInvalidSymbol);
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return GA_OK;
}

ga_status check_heads(int32_t hq, int32_t hkv, int32_t d) {
  if (hq <= 0 || hkv <= 0 || d <= 0) return GA_ERR_INVALID_ARGUMENT;
  if (hq % hkv != 0) return GA_ERR_INVALID_ARGUMENT;
  if (!ga::group_supported(hq / hkv)) return GA_ERR_UNSUPPORTED;
  if (d != kHeadDim) return GA_ERR_UNSUPPORTED;
  return GA_OK;
}

ga_status check_decode_dims(const ga_decode_dims* d) {
  if (d == nullptr) return GA_ERR_INVALID_ARGUMENT;
  if (d->batch < 0 || d->page_size <= 0 || d->max_pages_per_seq <= 0 || d->num_pages <= 0)
    return GA_ERR_INVALID_ARGUMENT;
  ga_status st = check_heads(d->num_q_heads, d->num_kv_heads, d->head_dim);
  if (st != GA_OK) return st;
  if (d->page_size != kPageSize && d->page_size != 1) return GA_ERR_UNSUPPORTED;
  if ((int64_t)d->batch * d->num_q_heads > kMaxDecodeRows) return GA_ERR_UNSUPPORTED;
  // capacity in tokens must fit an int32
  if ((int64_t)d->max_pages_per_seq * d->page_size > INT32_MAX / 2) return GA_ERR_UNSUPPORTED;
  return GA_OK;
}

// Attention-spec options: pointers fp32 / int32 aligned, reserved flags zero,
// key lengths only for prefill (decode has its seq_lens argument).
ga_status check_options(const ga_attn_options* o, bool prefill) {
  if (o == nullptr) return GA_OK;
  if (o->flags != 0) return GA_ERR_INVALID_ARGUMENT;
  if (!aligned(o->sinks, 4) || !aligned(o->lse, 4) || !aligned(o->kv_lens, 4))
    return GA_ERR_INVALID_ARGUMENT;
  if (!prefill && o->kv_lens != nullptr) return GA_ERR_INVALID_ARGUMENT;
  return GA_OK;
}

// Split plan from the dims alone (allocated capacity, not current lengths).
// GA_ERR_UNSUPPORTED when the stage-1 grid would not fit one launch.
ga_status make_plan(const ga_decode_dims* d, ga_decode_plan* p) {
  const int64_t cap = (int64_t)d->max_pages_per_seq * d->page_size;
  // stage-1 workgroups per split: one per (sequence, kv head); a workgroup
  // serves all the group's query heads
  const int64_t bkv = (int64_t)d->batch * d->num_kv_heads;
  int64_t t = (cap * (bkv > 0 ? bkv : 1) + GA_DECODE_TARGET_BLOCKS - 1) / GA_DECODE_TARGET_BLOCKS;
  t = ((t + kSplitQuantum - 1) / kSplitQuantum) * kSplitQuantum;
  if (t < kSplitQuantum) t = kSplitQuantum;
  const int64_t t_max = d->page_size != kPageSize           ? kMaxTokSplitTokens
                        : bkv < GA_DECODE_TARGET_BLOCKS ? kMaxLongSplitTokens
                                                        : kMaxSplitTokens;
  if (t > t_max) t = t_max;
  const int64_t ns = (cap + t - 1) / t;
  // stage-1 grid: one workgroup per (split, sequence, kv head)
  const int64_t units = (int64_t)d->batch * d->num_kv_heads * ns;
  const int64_t wgs = units;
  if (units > INT32_MAX / 2 || wgs > kMaxStage1Workgroups) return GA_ERR_UNSUPPORTED;
  p->tokens_per_split = (int32_t)t;
  p->num_splits = (int32_t)ns;
  const int64_t rows = (int64_t)d->batch * d->num_q_heads * ns;
  size_t bytes = (size_t)rows * (size_t)(kHeadDim + 2) * sizeof(float);
  p->workspace_bytes = (bytes + 255) & ~(size_t)255;
  return GA_OK;
}

}  // namespace

extern "C" {

ga_status gated_attn_decode_plan(const ga_decode_dims* dims, ga_decode_plan* plan) {
  if (plan == nullptr) return GA_ERR_INVALID_ARGUMENT;
  ga_status st = check_decode_dims(dims);
  if (st != GA_OK) return st;
  return make_plan(dims, plan);
}

size_t gated_attn_decode_workspace_size(const ga_decode_dims* dims) {
  ga_decode_plan p;
  if (gated_attn_decode_plan(dims, &p) != GA_OK) return 0;
  return p.workspace_bytes;
}

}  // extern "C"

namespace {

// Shared by the bf16 and e4m3 decode entry points.
// Token / page addressing of a decode call: a block table with seq_lens, or
// CSR row pointers and token slots (page size 1).
struct Indexing {
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  int64_t index_capacity;
};

ga_status decode_impl(const uint16_t* q, const uint16_t* gate, const void* k_pool,
                      const void* v_pool, const Indexing& ix, float scale, int kv_fp8,
                      float k_descale, float v_descale, uint16_t* out, void* stream,
                      const ga_decode_dims* dims, void* workspace, size_t workspace_bytes,
                      const ga_attn_options* opts) {
  ga_status st = check_decode_dims(dims);
  if (st != GA_OK) return st;
  const bool csr = ix.kv_indptr != nullptr || ix.kv_indices != nullptr;
  if (csr && dims->page_size != 1) return GA_ERR_UNSUPPORTED;
  if (!(std::isfinite(scale) && scale > 0.f)) return GA_ERR_INVALID_ARGUMENT;
  if (!(std::isfinite(k_descale) && k_descale > 0.f && std::isfinite(v_descale) &&
        v_descale > 0.f))
    return GA_ERR_INVALID_ARGUMENT;
  st = check_options(opts, /*prefill=*/false);
  if (st != GA_OK) return st;
  if (dims->batch == 0) return GA_OK;
  const void* ptr16[] = {q, gate, k_pool, v_pool, out, workspace};
  for (const void* p : ptr16)
    if (p == nullptr || !aligned(p, 16)) return GA_ERR_INVALID_ARGUMENT;
  if (csr) {
    if (ix.kv_indptr == nullptr || ix.kv_indices == nullptr || !aligned(ix.kv_indptr, 4) ||
        !aligned(ix.kv_indices, 4) || ix.index_capacity < 0)
      return GA_ERR_INVALID_ARGUMENT;
  } else if (ix.block_table == nullptr || ix.seq_lens == nullptr ||
             !aligned(ix.block_table, 4) || !aligned(ix.seq_lens, 4)) {
    return GA_ERR_INVALID_ARGUMENT;
  }
  ga_decode_plan plan;
  st = make_plan(dims, &plan);
  if (st != GA_OK) return st;
  if (workspace_bytes < plan.workspace_bytes) return GA_ERR_WORKSPACE_TOO_SMALL;
  st = check_device();
  if (st != GA_OK) return st;

  ga::DecodeLaunch L;
  L.q = q;
  L.gate = gate;
  L.k_pool = k_pool;
  L.v_pool = v_pool;
  L.block_table = csr ? nullptr : ix.block_table;
  L.seq_lens = csr ? nullptr : ix.seq_lens;
  L.kv_indptr = csr ? ix.kv_indptr : nullptr;
  L.kv_indices = csr ? ix.kv_indices : nullptr;
  L.index_capacity = csr ? ix.index_capacity : 0;
  L.page_size = dims->page_size;
  L.out = out;
  const size_t rows = (size_t)dims->batch * dims->num_q_heads * plan.num_splits;
  L.part_acc = static_cast<float*>(workspace);
  L.part_ml = L.part_acc + rows * kHeadDim;
  L.scale = scale;
  L.kv_fp8 = kv_fp8;
  L.k_descale = k_descale;
  L.v_descale = v_descale;
  L.batch = dims->batch;
  L.num_q_heads = dims->num_q_heads;
  L.num_kv_heads = dims->num_kv_heads;
  L.max_pages = dims->max_pages_per_seq;
  L.num_pages = dims->num_pages;
  L.tokens_per_split = plan.tokens_per_split;
  L.num_splits = plan.num_splits;
  L.split_target = GA_DECODE_TARGET_BLOCKS;
  L.sinks = opts != nullptr ? opts->sinks : nullptr;
  L.lse = opts != nullptr ? opts->lse : nullptr;
  L.window = opts != nullptr && opts->window > 0 ? opts->window : 0;
  hipError_t e = ga::launch_decode(L, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  return GA_OK;
}

}  // namespace

extern "C" {

ga_status gated_attn_decode_ex(const uint16_t* q, const uint16_t* gate, const uint16_t* k_pool,
                               const uint16_t* v_pool, const int32_t* block_table,
                               const int32_t* seq_lens, float scale, uint16_t* out, void* stream,
                               const ga_decode_dims* dims, void* workspace,
                               size_t workspace_bytes, const ga_attn_options* opts) {
  const Indexing ix = {block_table, seq_lens, nullptr, nullptr, 0};
  return decode_impl(q, gate, k_pool, v_pool, ix, scale, 0, 1.f, 1.f, out, stream, dims,
                     workspace, workspace_bytes, opts);
}

ga_status gated_attn_decode_csr(const uint16_t* q, const uint16_t* gate, const uint16_t* k_pool,
                                const uint16_t* v_pool, const int32_t* kv_indptr,
                                const int32_t* kv_indices, int64_t index_capacity, float scale,
                                uint16_t* out, void* stream, const ga_decode_dims* dims,
                                void* workspace, size_t workspace_bytes,
                                const ga_attn_options* opts) {
  if (kv_indptr == nullptr || kv_indices == nullptr) return GA_ERR_INVALID_ARGUMENT;
  const Indexing ix = {nullptr, nullptr, kv_indptr, kv_indices, index_capacity};
  return decode_impl(q, gate, k_pool, v_pool, ix, scale, 0, 1.f, 1.f, out, stream, dims,
                     workspace, workspace_bytes, opts);
}

ga_status gated_attn_decode_fp8kv(const uint16_t* q, const uint16_t* gate, const uint8_t* k_pool,
                                  const uint8_t* v_pool, const int32_t* block_table,
                                  const int32_t* seq_lens, float scale, float k_descale,
                                  float v_descale, uint16_t* out, void* stream,
                                  const ga_decode_dims* dims, void* workspace,
                                  size_t workspace_bytes, const ga_attn_options* opts) {
  const Indexing ix = {block_table, seq_lens, nullptr, nullptr, 0};
  return decode_impl(q, gate, k_pool, v_pool, ix, scale, 1, k_descale, v_descale, out, stream,
                     dims, workspace, workspace_bytes, opts);
}

ga_status gated_attn_decode_fp8kv_csr(const uint16_t* q, const uint16_t* gate,
                                      const uint8_t* k_pool, const uint8_t* v_pool,
                                      const int32_t* kv_indptr, const int32_t* kv_indices,
                                      int64_t index_capacity, float scale, float k_descale,
                                      float v_descale, uint16_t* out, void* stream,
                                      const ga_decode_dims* dims, void* workspace,
                                      size_t workspace_bytes, const ga_attn_options* opts) {
  if (kv_indptr == nullptr || kv_indices == nullptr) return GA_ERR_INVALID_ARGUMENT;
  const Indexing ix = {nullptr, nullptr, kv_indptr, kv_indices, index_capacity};
  return decode_impl(q, gate, k_pool, v_pool, ix, scale, 1, k_descale, v_descale, out, stream,
                     dims, workspace, workspace_bytes, opts);
}

ga_status gated_attn_decode(const uint16_t* q, const uint16_t* gate, const uint16_t* k_pool,
                            const uint16_t* v_pool, const int32_t* block_table,
                            const int32_t* seq_lens, float scale, uint16_t* out, void* stream,
                            const ga_decode_dims* dims, void* workspace, size_t workspace_bytes) {
  return gated_attn_decode_ex(q, gate, k_pool, v_pool, block_table, seq_lens, scale, out, stream,
                              dims, workspace, workspace_bytes, nullptr);
}

ga_status gated_attn_decode_noalloc(const uint16_t* q, const uint16_t* gate,
                                    const uint16_t* k_pool, const uint16_t* v_pool,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    float scale, uint16_t* out, void* stream,
                                    const ga_decode_dims* dims) {
  ga_decode_plan plan;
  ga_status st = gated_attn_decode_plan(dims, &plan);
  if (st != GA_OK) return st;
  if (plan.workspace_bytes > kScratchBytes) return GA_ERR_WORKSPACE_TOO_SMALL;
  if (dims->batch == 0) return GA_OK;
  st = check_device();
  if (st != GA_OK) return st;
  void* ws = nullptr;
  st = device_scratch(&ws);
  if (st != GA_OK) return st;
  return gated_attn_decode_ex(q, gate, k_pool, v_pool, block_table, seq_lens, scale, out, stream,
                              dims, ws, kScratchBytes, nullptr);
}

ga_status gated_attn_prefill_ex(const uint16_t* q, const uint16_t* gate, const uint16_t* k,
                                const uint16_t* v, float scale, int causal, uint16_t* out,
                                void* stream, const ga_prefill_dims* dims,
                                const ga_attn_options* opts) {
  if (dims == nullptr) return GA_ERR_INVALID_ARGUMENT;
  if (dims->batch < 0 || dims->seq_len < 0) return GA_ERR_INVALID_ARGUMENT;
  ga_status st = check_heads(dims->num_q_heads, dims->num_kv_heads, dims->head_dim);
  if (st != GA_OK) return st;
  if (!(std::isfinite(scale) && scale > 0.f)) return GA_ERR_INVALID_ARGUMENT;
  st = check_options(opts, /*prefill=*/true);
  if (st != GA_OK) return st;
  if (dims->batch == 0 || dims->seq_len == 0) return GA_OK;
  // The kernel addresses q, gate and out with 64-bit offsets.  Two limits
  // remain: one sequence's K or V rows of all kv heads, S * H_kv * D bf16,
  // are read through a buffer descriptor of at most 2^31 - 1 bytes, and the
  // grid (one workgroup per sequence, kv head, head part and 16 query
  // positions) stays below 2^22 workgroups.
  if ((int64_t)dims->seq_len * dims->num_kv_heads * kHeadDim * 2 > INT32_MAX)
    return GA_ERR_UNSUPPORTED;
  const int parts = ga::head_parts(dims->num_q_heads / dims->num_kv_heads);
  if ((int64_t)dims->batch * dims->num_kv_heads * parts * ((dims->seq_len + 15) / 16) >
      kMaxPrefillWorkgroups)
    return GA_ERR_UNSUPPORTED;
  const void* ptr16[] = {q, gate, k, v, out};
  for (const void* p : ptr16)
    if (p == nullptr || !aligned(p, 16)) return GA_ERR_INVALID_ARGUMENT;
  st = check_device();
  if (st != GA_OK) return st;

  ga::PrefillLaunch P;
  P.q = q;
  P.gate = gate;
  P.k = k;
  P.v = v;
  P.out = out;
  P.scale = scale;
  P.causal = causal != 0;
  P.batch = dims->batch;
  P.seq_len = dims->seq_len;
  P.num_q_heads = dims->num_q_heads;
  P.num_kv_heads = dims->num_kv_heads;
  P.kv_lens = opts != nullptr ? opts->kv_lens : nullptr;
  P.sinks = opts != nullptr ? opts->sinks : nullptr;
  P.lse = opts != nullptr ? opts->lse : nullptr;
  P.window = opts != nullptr && opts->window > 0 ? opts->window : 0;
  hipError_t e = ga::launch_prefill(P, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  return GA_OK;
}

ga_status gated_attn_prefill(const uint16_t* q, const uint16_t* gate, const uint16_t* k,
                             const uint16_t* v, float scale, int causal, uint16_t* out,
                             void* stream, const ga_prefill_dims* dims) {
  return gated_attn_prefill_ex(q, gate, k, v, scale, causal, out, stream, dims, nullptr);
}

ga_status gated_attn_qk_norm_rope(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  const uint16_t* w_q_norm, const uint16_t* w_k_norm, float eps,
                                  const uint16_t* cos, const uint16_t* sin,
                                  const int64_t* slot_mapping, uint16_t* q_out, uint16_t* k_out,
                                  uint16_t* v_out, void* stream, const ga_qk_norm_rope_dims* dims) {
  if (dims == nullptr) return GA_ERR_INVALID_ARGUMENT;
  const int64_t T = dims->num_tokens;
  if (T < 0 || dims->num_q_heads <= 0 || dims->num_kv_heads <= 0 || dims->head_dim <= 0 ||
      dims->rope_dim < 0 || dims->rope_dim > dims->head_dim || (dims->rope_dim & 1))
    return GA_ERR_INVALID_ARGUMENT;
  if (dims->head_dim != kHeadDim || dims->rope_dim % 8 != 0) return GA_ERR_UNSUPPORTED;
  if (!(std::isfinite(eps) && eps >= 0.f)) return GA_ERR_INVALID_ARGUMENT;
  if ((w_q_norm == nullptr) != (w_k_norm == nullptr)) return GA_ERR_INVALID_ARGUMENT;
  const int64_t rows = T * ((int64_t)dims->num_q_heads + dims->num_kv_heads);
  if (rows > ((int64_t)1 << 30)) return GA_ERR_UNSUPPORTED;
  int64_t num_slots = 0;
  if (slot_mapping != nullptr) {
    if (dims->page_size != kPageSize) return GA_ERR_UNSUPPORTED;
    if (dims->num_pages <= 0) return GA_ERR_INVALID_ARGUMENT;
    num_slots = dims->num_pages * kPageSize;
  }
  if (T == 0) return GA_OK;
  const void* need16[] = {q, k, v, q_out, k_out};
  for (const void* p : need16)
    if (p == nullptr || !aligned(p, 16)) return GA_ERR_INVALID_ARGUMENT;
  if (slot_mapping != nullptr && (v_out == nullptr || !aligned(slot_mapping, 8)))
    return GA_ERR_INVALID_ARGUMENT;
  if (!aligned(v_out, 16) || !aligned(w_q_norm, 16) || !aligned(w_k_norm, 16))
    return GA_ERR_INVALID_ARGUMENT;
  if (dims->rope_dim > 0 &&
      (cos == nullptr || sin == nullptr || !aligned(cos, 16) || !aligned(sin, 16)))
    return GA_ERR_INVALID_ARGUMENT;
  ga_status st = check_device();
  if (st != GA_OK) return st;

  ga::RopeLaunch P;
  P.q = q;
  P.k = k;
  P.v = v;
  P.w_q = w_q_norm;
  P.w_k = w_k_norm;
  P.cos = cos;
  P.sin = sin;
  P.slot_mapping = slot_mapping;
  P.q_out = q_out;
  P.k_out = k_out;
  P.v_out = v_out;
  P.eps = eps;
  P.num_tokens = T;
  P.num_slots = num_slots;
  P.num_q_heads = dims->num_q_heads;
  P.num_kv_heads = dims->num_kv_heads;
  P.rope_dim = dims->rope_dim;
  hipError_t e = ga::launch_qk_norm_rope(P, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  return GA_OK;
}

ga_status gated_attn_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (src == nullptr || sink == nullptr || !aligned(src, 16) || !aligned(sink, 4) || bytes % 16 != 0)
    return GA_ERR_INVALID_ARGUMENT;
  ga_status st = check_device();
  if (st != GA_OK) return st;
  if (bytes == 0) return GA_OK;
  hipError_t e = ga::launch_stream_read(src, bytes, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  return GA_OK;
}

const char* gated_attn_status_string(ga_status status) {
  switch (status) {
    case GA_OK: return "GA_OK";
    case GA_ERR_INVALID_ARGUMENT: return "GA_ERR_INVALID_ARGUMENT";
    case GA_ERR_UNSUPPORTED: return "GA_ERR_UNSUPPORTED";
    case GA_ERR_WORKSPACE_TOO_SMALL: return "GA_ERR_WORKSPACE_TOO_SMALL";
    case GA_ERR_HIP: return "GA_ERR_HIP";
  }
  return "GA_ERR_UNKNOWN";
}

int gated_attn_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
