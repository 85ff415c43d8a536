// decode.hip -- split-KV gated GQA decode for gfx950 (CDNA4, wave64).
//
// Stage 1 (one 8-wave workgroup per (split s, sequence b, kv head g), sized so
// the grid is about one workgroup per CU): stream the split's tokens of the
// paged K/V pool once, score all query heads of the GQA group (up to 16)
// against every key on the matrix cores, and keep an fp32 online softmax
// state (running max, running sum, unnormalised O[256]) per head.  FreeToken
// PR #781, Summary: stage-1 partials are kept in fp32 for stage 2.
//
// Stage 2 (one wave per (b, query head)): merge the splits' partials by their
// log-sum-exp in fp32, round O to bf16, and apply the bf16 sigmoid gate with a
// rounded product -- the gate costs no launch of its own (FreeToken PR #781,
// Summary; cuDNN "Gated Attention Block", fuse_gate).
//
// Stage 1 in a wave.  The split's tokens form 16-token tiles (one page each);
// wave w takes tiles w, w + 8, w + 16, ... (a static assignment, so results do
// not depend on timing).  MFMA layouts (wave64): v_mfma_f32_16x16x32_bf16 A row
// = lane % 16, k = 8(lane / 16) + 0..7, B column = lane % 16, same k;
// v_mfma_f32_16x16x16_bf16 the same with k = 4(lane / 16) + 0..3; C row =
// 4(lane / 16) + r, column = lane % 16.  Per tile:
//   S^T (16 keys x 16 head columns) = K Q^T, 8 MFMAs 16x16x32.  A = K read
//       from HBM straight into registers (lane (li, lg): key li, 8 dims per
//       k-step), B = q (column = head; idle columns are zero).  Each lane then
//       holds head li's scores of keys 4lg .. 4lg+3 -- already the A layout of
//       P for the 16x16x16 product below.
//   online softmax per head in fp32 (lazy rescaling against a reference max);
//   P = Phi + Plo, two bf16 terms (~16 significant bits of the fp32 weight);
//   O (16 heads x 256) += P V, 16 column tiles x 2 MFMAs 16x16x16.  V needs
//       keys along k, but rows are stored dims-first, so it passes through a
//       per-wave LDS tile (rows of 512 B, 16-byte chunk c of row r stored at
//       c ^ 2(r & 7): conflict-free) and comes back transposed by the gfx950
//       read ds_read_b64_tr_b16 (within 16 lanes, lane i of the result gets
//       element i % 4 of source lane 4k + i / 4 in slot k; source lane s
//       points at V[key0 + s/4][d0 + 4(s%4)]).
// bf16 V is copied HBM -> LDS by direct global-to-LDS loads (no registers),
// alternating between two tiles; e4m3 K is converted to bf16 in registers
// before the score MFMAs, and e4m3 V is copied raw to LDS and converted into
// the bf16 tile just before its P V.  About two tiles per wave are in flight.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <cstdlib>
#include <cstring>

#include "ga_device.h"
#include "ga_internal.h"

namespace ga {

namespace {

constexpr int kD = 256;          // head dim
constexpr int kHeads = 16;       // query-head columns of an MFMA stage-1 workgroup
constexpr int kGroup = 8;        // query-head slots of a VALU stage-1 workgroup
constexpr int kStep = 8;         // tokens per VALU wave step
constexpr int kPage = 16;        // tokens per page = keys per tile
constexpr int kWaves = 8;        // waves per stage-1 workgroup (one workgroup per CU)
constexpr int kPageRegs = 2;     // page ids per lane: a split spans at most 128 pages
constexpr int kMaxSplit = 2048;  // tokens of the largest split
constexpr int kMinSplit = 64;    // tokens of the smallest split a sizing rule asks for
constexpr int kTileBytes = kPage * kD * 2;  // one bf16 V tile in LDS
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSlack = 8.f;    // lazy-rescale threshold, log2 units

struct Stage1Args {
  const uint16_t* q;
  const char* k_pool;  // bf16 or e4m3 elements, [P][16][H_kv][D]
  const char* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* kv_indptr;   // CSR (page size 1): [B + 1], or null for a block table
  const int32_t* kv_indices;  // CSR token slots
  long long index_capacity;   // entries of kv_indices
  float* part_acc;   // [B][H_q][NS][D]
  float* part_ml;    // [B][H_q][NS][2]  (m in log2 units, l)
  float scale_log2;  // scale * k factor * log2(e)
  int num_q_heads;
  int num_kv_heads;
  int num_units;     // NS * B * H_kv
  int max_pages;     // W: block-table columns (pages, or tokens at page size 1)
  long long num_pages;
  int tokens_per_split;  // the most tokens of one split
  int num_splits;
  int window;        // > 0: only the last `window` tokens of a sequence are visible
  int split_units;   // B * H_kv (the split sizing rule's units)
  int split_target;  // the workgroups the sizing rule aims for
};

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef s16x4_t __attribute__((address_space(3))) lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// K/V rows are read exactly once per call: non-temporal loads keep them from
// displacing reusable lines in L2 and the Infinity Cache (MALL).  kNt is the
// same policy for the direct global-to-LDS copies (cache-policy bit "nt").
constexpr int kNt = 2;
__device__ __forceinline__ uint4 ldg16_stream(const char* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// e4m3 codes -> bf16.  gfx950's conversion decodes the OCP e4m3 format
// exactly (checked on all 256 codes against an independent decoder); every
// e4m3 value is a bf16 value.  `hi` selects the codes in bytes 2-3 instead
// of 0-1.
template <bool hi>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t codes) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, hi));
}

// Two fp32 -> packed bf16 pair (round to nearest even); used for P only,
// whose precision the hi/lo split restores.
__device__ __forceinline__ uint32_t pk_bf16(float x, float y) {
  const f32x2_t v = {x, y};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// p must point into LDS (8-byte aligned).
__device__ __forceinline__ s16x4_t lds_tr_read(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
}

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint2 ldg8_stream(const char* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v[0], v[1]);
}

struct alignas(16) WaveSlot {
  float p[kStep][kGroup];  // probabilities of the step's 8 tokens x 8 heads
  float alpha[kGroup];     // rescale factor of the running state per head
};

struct alignas(16) MergeSlot {
  float acc[kWaves][kGroup][kD];
  float m[kWaves][kGroup];
  float l[kWaves][kGroup];
};

// How one sequence is split.  The grid and the workspace come from the
// capacity (num_splits splits of at most max_tokens tokens), so a call
// captured once serves every length.  Inside that, the sequence's visible
// keys [base, L) -- base is the window start rounded down to a page -- get
// the same sizing rule the capacity got (about target_blocks workgroups for
// `units` (sequence, kv head) pairs, at least kMinSplit tokens), cut into
// equal page-aligned parts: short sequences and windows spread over several
// splits, and no split is a sliver.
struct SplitRange {
  int base;    // first token of split 0
  int tokens;  // tokens per split (0 for an empty sequence)
  int count;   // non-empty splits (<= num_splits)
};

__device__ __forceinline__ SplitRange split_range(int L, int window, int num_splits,
                                                  int max_tokens, int units, int target_blocks) {
  SplitRange r;
  const int tok_lo = window > 0 ? max(0, L - window) : 0;
  r.base = tok_lo & ~(kPage - 1);
  const int n = L - r.base;
  if (n <= 0) {
    r.tokens = 0;
    r.count = 0;
    return r;
  }
  long long t = ((long long)n * units + target_blocks - 1) / target_blocks;
  t = max(t, (long long)kMinSplit);
  t = max(t, (long long)((n + num_splits - 1) / num_splits));  // at most num_splits splits
  t = min(t, (long long)max_tokens);
  const int count = (int)((n + t - 1) / t);
  r.tokens = (((n + count - 1) / count) + kPage - 1) & ~(kPage - 1);
  r.count = (n + r.tokens - 1) / r.tokens;
  return r;
}

}  // namespace

// The length of sequence b and where its token / page ids start: from the
// CSR row pointers, or seq_lens and the block-table row.  Clamped so that a
// violated precondition cannot lead outside the buffers.
__device__ __forceinline__ int seq_length(const int32_t* seq_lens, const int32_t* indptr,
                                          long long index_capacity, int b, int capacity,
                                          long long* first_index) {
  if (indptr != nullptr) {
    const long long lo = min(max((long long)indptr[b], 0LL), index_capacity);
    const long long hi = min(max((long long)indptr[b + 1], lo), index_capacity);
    *first_index = lo;
    return (int)min(hi - lo, (long long)capacity);
  }
  *first_index = 0;
  return min(seq_lens[b], capacity);
}

// The VALU stage-1 body (bf16 pools, groups of up to 8 heads), with 16-token
// pages (kTok = false) or one token per page (true: block-table entries or
// CSR indices are token slots).  Work layout inside a wave, per step of 8
// tokens, which all lie in one half of one 16-token page:
//   scores : lane = (token tq in 0..3) x (16-byte chunk c16 in 0..15).  A pass
//            covers 4 tokens; each lane holds q chunks c16 and c16+16 of all 8
//            heads (64 VGPRs) and forms 8 partial dot products with bf16 dot2
//            instructions; a 16-lane DPP reduce-scatter completes them (each
//            head's score lands in two lanes).  Two passes per step.
//   values : lane owns d = 4*lane .. 4*lane+3 of all 8 heads (32 fp32
//            accumulators) and takes every token of the step.
//   softmax: probabilities go through a 288-byte per-wave LDS slot from the
//            score lanes to the value lanes.
// Every K and V load instruction of a wave reads whole 256/512-byte row
// segments, and two steps' loads are in flight while a step is computed.
template <bool kTok>
__device__ __forceinline__ void stage1_valu_body(const Stage1Args& a) {
  __shared__ WaveSlot wslot[kWaves][2];
  __shared__ MergeSlot merge;
  __shared__ int progress[kWaves];  // last step each wave started
  __shared__ __align__(16) int tok_ids[kTok ? kMaxSplit : 4];  // page size 1: the split's token slots

  // Workgroup id -> (split s, sequence b, kv head g), split-major as in the
  // MFMA body.
  const int unit = blockIdx.x;  // (s * B + b) * H_kv + g
  if (unit >= a.num_units) return;
  const int seq_heads = a.num_units / a.num_splits;  // B * H_kv
  const int s = unit / seq_heads;
  const int g = (unit - s * seq_heads) % a.num_kv_heads;
  const int b = (unit - s * seq_heads) / a.num_kv_heads;
  const int lane = __lane_id();
  // wave-uniform by construction; readfirstlane lets the compiler keep the
  // step bookkeeping and the load base addresses in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int Hkv = a.num_kv_heads;
  const int Hq = a.num_q_heads;
  const int nh = Hq / Hkv;  // <= kGroup: head slots 0..nh-1 are real, the rest idle
  const int h0 = g * nh;    // first query head of this workgroup

  // Issued together, before the length is known: the page ids of split s as
  // it is when the sequence fills its capacity (page j of the split in lane
  // j % 64 of register j / 64; ids past the sequence's end are never used),
  // the length, and q.  Other lengths reload the page ids below.
  const int32_t* bt_row = a.block_table + (size_t)b * a.max_pages;
  auto load_pages = [&](int tok_first, int ntok, int (&pages)[kPageRegs]) {
    const int fp = tok_first / kPage;
    const int np = min(ntok / kPage, a.max_pages - fp);
#pragma unroll
    for (int r = 0; r < kPageRegs; ++r)
      pages[r] = lane + 64 * r < np ? bt_row[fp + lane + 64 * r] : 0;
  };
  int my_page[kPageRegs] = {0, 0};
  const int full_begin = s * a.tokens_per_split;  // < capacity, since s < num_splits
  if constexpr (!kTok) load_pages(full_begin, a.tokens_per_split, my_page);

  // score-lane coordinates
  const int tq = lane >> 4;    // token within a pass
  const int c16 = lane & 15;   // 16-byte chunk (and chunk + 16)
  const int hs = c16 >> 1;     // head whose score this lane keeps (see reduce_scatter8)

  // q of the workgroup's heads over the dims this lane's K pieces hold (bf16
  // pairs): d = 8 c16 .. +7 and 8 (c16 + 16) .. +7 (two 16-byte pieces of the
  // 512-byte row).  Idle head slots get q = 0 (their scores and sums are
  // computed and dropped).
  uint4 qa[kGroup], qb[kGroup];
  {
    const uint16_t* qbase = a.q + ((size_t)b * Hq + (size_t)h0) * kD;
    const int da = 8 * c16;
    const int db = 8 * (c16 + 16);
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      const int hh = min(h, nh - 1);
      qa[h] = ldg16(qbase + hh * kD + da);
      qb[h] = ldg16(qbase + hh * kD + db);
    }
#pragma unroll
    for (int h = 0; h < kGroup; ++h)
      if (h >= nh) qa[h] = qb[h] = make_uint4(0, 0, 0, 0);
  }

  // Lengths past the capacity and page ids outside the pool break the
  // documented preconditions; both are clamped so such input yields garbage
  // in its own row instead of an access outside the buffers.
  const int capacity = kTok ? a.max_pages : a.max_pages * kPage;
  long long first_index = 0;
  const int L = seq_length(a.seq_lens, a.kv_indptr, a.index_capacity, b, capacity, &first_index);
  // First visible token: the sliding window keeps the last `window` tokens.
  const int tok_lo = a.window > 0 ? max(0, L - a.window) : 0;
  const SplitRange sr = split_range(L, a.window, a.num_splits, a.tokens_per_split,
                                    a.split_units, a.split_target);
  if (s >= sr.count) return;  // empty split: stage 2 never reads its slot
  const int tok_begin = sr.base + s * sr.tokens;
  const int tok_end = min(L, tok_begin + sr.tokens);
  const int first_page = tok_begin / kPage;
  if constexpr (kTok) {
    // one slot per token: the split's slots go to LDS (at most kMaxSplit)
    const int32_t* ids = a.kv_indptr != nullptr ? a.kv_indices + first_index : bt_row;
    for (int i = threadIdx.x; i < sr.tokens; i += kWaves * 64) {
      const int tok = tok_begin + i;
      const int id = tok < tok_end ? ids[tok] : 0;
      tok_ids[i] = (int)min((long long)max(id, 0), a.num_pages - 1);
    }
  } else {
    if (tok_begin != full_begin) load_pages(tok_begin, sr.tokens, my_page);
#pragma unroll
    for (int r = 0; r < kPageRegs; ++r)
      my_page[r] = (int)min((long long)max(my_page[r], 0), a.num_pages - 1);
  }
  if (threadIdx.x < kWaves) progress[threadIdx.x] = 0;
  __syncthreads();

  // value lanes: lane owns d = 4*lane .. 4*lane+3 of all 8 heads
  float acc[kGroup][4];
#pragma unroll
  for (int h = 0; h < kGroup; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[h][e] = 0.f;
  float m_run = -INFINITY;  // reference max (log2 units) of head hs
  float l_run = 0.f;        // this lane's share of the running sum of head hs

  const int n_steps = (tok_end - tok_begin + kStep - 1) / kStep;
  constexpr int kElem = 2;                                  // bytes per K / V element
  const size_t row_bytes = (size_t)Hkv * kD * kElem;        // between tokens
  const size_t page_bytes = (size_t)kPage * row_bytes;      // between pages

  // Byte offsets of this lane's pieces inside one 8-token step (the same for
  // every step); the step's base address is wave-uniform.
  unsigned k_off[2];
#pragma unroll
  for (int pass = 0; pass < 2; ++pass)
    k_off[pass] = (unsigned)((pass * 4 + tq) * (int)row_bytes + c16 * 16);
  unsigned v_off[kStep];
#pragma unroll
  for (int t = 0; t < kStep; ++t) v_off[t] = (unsigned)(t * (int)row_bytes + lane * 4 * kElem);

  auto step_base = [&](int step, const char* pool) -> const char* {
    const int t0 = tok_begin + step * kStep;
    const int j = t0 / kPage - first_page;  // wave-uniform
    const int pg = j < 64 ? __builtin_amdgcn_readlane(my_page[0], j)
                          : __builtin_amdgcn_readlane(my_page[1], j - 64);
    return pool + (size_t)pg * page_bytes + (size_t)(t0 % kPage) * row_bytes +
           (size_t)g * kD * kElem;
  };

  // One step's data.  K: per pass of 4 tokens, 32 bytes per lane.  V: per
  // token, 8 bytes per lane -- a whole row segment per wave instruction.
  typedef uint2 VElem;
  struct KRegs {
    uint4 k[2][2];
  };
  struct VRegs {
    VElem v[kStep];
  };
  // Page size 1: every token has its own slot, so K takes a per-lane address
  // (the lane's token of the pass) and V one scalar base per token, both from
  // the slots in LDS.
  const size_t head_bytes = (size_t)g * kD * kElem;
  auto load_k = [&](int step, KRegs& r) {
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const char* kb;
      unsigned off;
      if constexpr (kTok) {
        kb = a.k_pool + (size_t)tok_ids[step * kStep + pass * 4 + tq] * row_bytes + head_bytes;
        off = (unsigned)(c16 * 16);
      } else {
        kb = step_base(step, a.k_pool);
        off = k_off[pass];
      }
      r.k[pass][0] = ldg16_stream(kb + off);
      r.k[pass][1] = ldg16_stream(kb + (off + 256u));
    }
  };
  auto load_v = [&](int step, VRegs& r) {
    int4 ids_lo = make_int4(0, 0, 0, 0), ids_hi = make_int4(0, 0, 0, 0);
    if constexpr (kTok) {
      ids_lo = *reinterpret_cast<const int4*>(&tok_ids[step * kStep]);
      ids_hi = *reinterpret_cast<const int4*>(&tok_ids[step * kStep + 4]);
    }
    const int ids[kStep] = {ids_lo.x, ids_lo.y, ids_lo.z, ids_lo.w,
                            ids_hi.x, ids_hi.y, ids_hi.z, ids_hi.w};
    const char* vb = kTok ? nullptr : step_base(step, a.v_pool);
#pragma unroll
    for (int t = 0; t < kStep; ++t) {
      const char* p;
      if constexpr (kTok)
        p = a.v_pool + (size_t)__builtin_amdgcn_readfirstlane(ids[t]) * row_bytes + head_bytes +
            lane * 4 * kElem;
      else
        p = vb + v_off[t];
      r.v[t] = ldg8_stream(p);
    }
  };

  // Two probability slots per wave: the scores of step i+1 are computed into
  // one while the values of step i are accumulated from the other, so the two
  // dependency chains can be interleaved; one fence per step separates a
  // slot's writes from its reads.
  WaveSlot* slots = wslot[wave];

  // Scores of one step -> probabilities in the step's slot.  Returns (wave-
  // uniform) whether the reference max was raised, in which case the slot's
  // alpha[] holds the factors the value accumulators must take before this
  // step's probabilities are added (l_run is rescaled here).
  auto score_step = [&](int step, const KRegs& r, WaveSlot& ws) -> bool {
    const int t0 = tok_begin + step * kStep;
    float sc[2];
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      // this lane's 16 K values as 8 bf16 pairs, in q's pair order
      const uint32_t kp[8] = {r.k[pass][0].x, r.k[pass][0].y, r.k[pass][0].z, r.k[pass][0].w,
                              r.k[pass][1].x, r.k[pass][1].y, r.k[pass][1].z, r.k[pass][1].w};
      float part[kGroup];
#pragma unroll
      for (int h = 0; h < kGroup; ++h) {
        float x = 0.f;
        x = dot2_bf16(qa[h].x, kp[0], x);
        x = dot2_bf16(qa[h].y, kp[1], x);
        x = dot2_bf16(qa[h].z, kp[2], x);
        x = dot2_bf16(qa[h].w, kp[3], x);
        x = dot2_bf16(qb[h].x, kp[4], x);
        x = dot2_bf16(qb[h].y, kp[5], x);
        x = dot2_bf16(qb[h].z, kp[6], x);
        x = dot2_bf16(qb[h].w, kp[7], x);
        part[h] = x;
      }
      const float mine = reduce_scatter8(part, c16);
      const int t = t0 + pass * 4 + tq;
      sc[pass] = (t < tok_end && t >= tok_lo) ? mine * a.scale_log2 : -INFINITY;
    }
    // Lazy rescaling: probabilities are taken relative to a reference max
    // m_run that is only raised (with a rescale of l and acc) when some score
    // of the step exceeds it by more than kSlack (log2 units), i.e. when a
    // probability would exceed 2^kSlack.  On the common path there is then no
    // cross-lane max and no rescale; any reference gives the same O, and
    // probabilities stay in [0, 2^kSlack].
    const bool raise = (sc[0] > m_run + kSlack) || (sc[1] > m_run + kSlack);
    const bool raised = __builtin_amdgcn_ballot_w64(raise) != 0;  // wave-uniform
    if (raised) {
      float mx = fmaxf(sc[0], sc[1]);
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
      if ((c16 & 1) == 0 && tq == 0) ws.alpha[hs] = alpha;
    }
    const float p0 = __builtin_amdgcn_exp2f(sc[0] - m_run);
    const float p1 = __builtin_amdgcn_exp2f(sc[1] - m_run);
    l_run += p0 + p1;
    if ((c16 & 1) == 0) {  // odd lanes hold the same (token, head) as their even neighbour
      ws.p[tq][hs] = p0;
      ws.p[4 + tq][hs] = p1;
    }
    return raised;
  };

  // Values of one step from its slot (after the rescale its scores asked for).
  auto value_step = [&](int step, const VRegs& r, const WaveSlot& ws, bool rescale) {
    const int t0 = tok_begin + step * kStep;
    if (rescale) {
      const float4 al0 = *reinterpret_cast<const float4*>(&ws.alpha[0]);
      const float4 al1 = *reinterpret_cast<const float4*>(&ws.alpha[4]);
      const float al[kGroup] = {al0.x, al0.y, al0.z, al0.w, al1.x, al1.y, al1.z, al1.w};
#pragma unroll
      for (int h = 0; h < kGroup; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[h][e] *= al[h];
    }
    VElem vv[kStep];
#pragma unroll
    for (int t = 0; t < kStep; ++t) vv[t] = r.v[t];
    if (t0 + kStep > tok_end || t0 < tok_lo) {
      // last step of the sequence (tail slots may hold anything) or the step
      // the window starts in: invisible rows take no part, whatever they hold
#pragma unroll
      for (int t = 0; t < kStep; ++t)
        if (t0 + t >= tok_end || t0 + t < tok_lo) vv[t] = VElem{};
    }
#pragma unroll
    for (int t = 0; t < kStep; ++t) {
      const float vf[4] = {bf16_lo(vv[t].x), bf16_hi(vv[t].x), bf16_lo(vv[t].y),
                           bf16_hi(vv[t].y)};
      const float4 pa = *reinterpret_cast<const float4*>(&ws.p[t][0]);
      const float4 pb = *reinterpret_cast<const float4*>(&ws.p[t][4]);
      const float pr[kGroup] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
#pragma unroll
      for (int h = 0; h < kGroup; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[h][e] = fmaf(pr[h], vf[e], acc[h][e]);
    }
  };

  // Steps of this wave: wave, wave + 8, ...; the assignment is static, so
  // the result does not depend on timing.  Each iteration scores step c1 and
  // accumulates the values of step c0; the K rows of a step are loaded one
  // iteration before its scores and its V rows one iteration before its
  // values, into two K and two V register sets used in turn (the loop is
  // unrolled twice, so no set is copied).  Loads are issued unconditionally
  // (past the end a wave re-reads the last step), so the wait before a step's
  // arithmetic covers only that step's own loads.
  //
  // A CU issues instructions of older waves first, which on its own lets the
  // first waves of the workgroup run well ahead of the last ones, and the
  // workgroup ends with its slowest wave.  So at every step a wave compares
  // its position with the other waves' and, while at least half of them are
  // ahead of it, runs at a raised issue priority (measured at B=64, L=4096:
  // stage 1 takes 89.4 us with this and 92.2 us without).
  auto balance = [&](int c) {
    if (lane == 0) progress[wave] = c;
    const int other = lane < kWaves ? progress[lane] : 0;
    const unsigned long long ahead = __builtin_amdgcn_ballot_w64(other > c);
    if (__builtin_popcountll(ahead) >= kWaves / 2)
      __builtin_amdgcn_s_setprio(2);
    else
      __builtin_amdgcn_s_setprio(0);
  };
  const int first_step = (max(tok_begin, tok_lo) - tok_begin) / kStep;
  int c0 = first_step + wave;
  if (c0 < n_steps) {
    const int last = n_steps - 1;
    int c1 = c0 + kWaves;
    int c2 = c0 + 2 * kWaves;
    KRegs kA, kB;
    VRegs vA, vB;
    load_k(c0, kA);
    load_v(c0, vA);
    load_k(min(c1, last), kB);
    bool resc = score_step(c0, kA, slots[0]);
    wave_lds_sync();
    for (;;) {
      // kB: K of c1; vA: V of c0 (scored, slot 0)
      balance(c0);
      load_k(min(c2, last), kA);
      load_v(min(c1, last), vB);
      bool resc_next = false;
      if (c1 < n_steps) resc_next = score_step(c1, kB, slots[1]);
      value_step(c0, vA, slots[0], resc);
      wave_lds_sync();
      c0 = c1;
      c1 = c2;
      c2 += kWaves;
      resc = resc_next;
      if (c0 >= n_steps) break;

      // kA: K of c1; vB: V of c0 (scored, slot 1)
      balance(c0);
      load_k(min(c2, last), kB);
      load_v(min(c1, last), vA);
      resc_next = false;
      if (c1 < n_steps) resc_next = score_step(c1, kA, slots[0]);
      value_step(c0, vB, slots[1], resc);
      wave_lds_sync();
      c0 = c1;
      c1 = c2;
      c2 += kWaves;
      resc = resc_next;
      if (c0 >= n_steps) break;
    }
    __builtin_amdgcn_s_setprio(0);
  }

  // ---- merge the waves' states and write the split's partial ---------------
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);
  if (lane < 2 * kGroup && (lane & 1) == 0) {  // tq == 0, c16 == 2h: one lane per head
    merge.m[wave][lane >> 1] = m_run;
    merge.l[wave][lane >> 1] = l_run;
  }
#pragma unroll
  for (int h = 0; h < kGroup; ++h)
    *reinterpret_cast<float4*>(&merge.acc[wave][h][lane * 4]) =
        make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
  __syncthreads();
  {
    const int h = threadIdx.x >> 6;   // 0..7
    const int c = threadIdx.x & 63;   // 4 values each
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, merge.m[w][h]);
    float wgt[kWaves];
    float lam = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      wgt[w] = __builtin_amdgcn_exp2f(merge.m[w][h] - M);  // 0 for a wave without tokens
      lam += merge.l[w][h] * wgt[w];
    }
    float out[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float4 x = *reinterpret_cast<const float4*>(&merge.acc[w][h][c * 4]);
      out[0] = fmaf(x.x, wgt[w], out[0]);
      out[1] = fmaf(x.y, wgt[w], out[1]);
      out[2] = fmaf(x.z, wgt[w], out[2]);
      out[3] = fmaf(x.w, wgt[w], out[3]);
    }
    if (h < nh) {
      const size_t row = ((size_t)b * Hq + (size_t)(h0 + h)) * a.num_splits + s;
      *reinterpret_cast<float4*>(a.part_acc + row * kD + c * 4) =
          make_float4(out[0], out[1], out[2], out[3]);
      if (c == 0) {
        a.part_ml[row * 2 + 0] = M;
        a.part_ml[row * 2 + 1] = lam;
      }
    }
  }
}

// The MFMA stage-1 body for bf16 pools (kFp8 = false) or e4m3 pools (true),
// with 16-token pages (kTok = false) or one token per page (true).
template <bool kFp8, bool kTok>
__device__ __forceinline__ void stage1_mma_body(const Stage1Args& a) {
  // Per-wave LDS tiles.  bf16 pools: vA / vB = two V tiles, used in turn.
  // e4m3 pools: vA = the converted bf16 tile, vB / vC = two raw e4m3 tiles.
  // Separate objects, so the compiler can see that a copy into one does not
  // touch the others.  After the loop they hold the waves' O for the merge.
  __shared__ __align__(16) char vA[kWaves][kTileBytes];
  __shared__ __align__(16) char vB[kWaves][kFp8 ? kTileBytes / 2 : kTileBytes];
  __shared__ __align__(16) char vC[kWaves][kFp8 ? kTileBytes / 2 : 16];
  __shared__ float m_w[kWaves][kHeads], l_w[kWaves][kHeads];
  __shared__ __align__(16) int tok_ids[kTok ? kMaxSplit : 4];  // page size 1: the split's token slots

  // Workgroup id -> (split s, sequence b, kv head g).  Ids are dispatched in
  // order, round-robin over the 8 XCDs; units are split-major (every
  // sequence's split 0, then split 1, ...), so the splits a short sequence
  // leaves empty come last and the busy ones spread over all XCDs.
  const int unit = blockIdx.x;  // (s * B + b) * H_kv + g
  if (unit >= a.num_units) return;
  const int seq_heads = a.num_units / a.num_splits;  // B * H_kv
  const int s = unit / seq_heads;
  const int g = (unit - s * seq_heads) % a.num_kv_heads;
  const int b = (unit - s * seq_heads) / a.num_kv_heads;
  const int lane = __lane_id();
  // wave-uniform by construction; readfirstlane keeps it in a scalar register
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int Hkv = a.num_kv_heads;
  const int Hq = a.num_q_heads;
  const int nh = Hq / Hkv;            // heads of the group (<= 16); columns past it are idle
  const int h0 = g * nh;              // first query head of the group
  const int li = lane & 15, lg = lane >> 4;

  // Issued together, before the length is known: the page ids of split s as
  // it is when the sequence fills its capacity (page j of the split in lane
  // j % 64 of register j / 64; ids past the sequence's end are never used),
  // the length, and q.  Other lengths reload the page ids below.
  const int32_t* bt_row = a.block_table + (size_t)b * a.max_pages;
  auto load_pages = [&](int tok_first, int ntok, int (&pages)[kPageRegs]) {
    const int fp = tok_first / kPage;
    const int np = min(ntok / kPage, a.max_pages - fp);
#pragma unroll
    for (int r = 0; r < kPageRegs; ++r)
      pages[r] = lane + 64 * r < np ? bt_row[fp + lane + 64 * r] : 0;
  };
  int my_page[kPageRegs] = {0, 0};
  const int full_begin = s * a.tokens_per_split;  // < capacity, since s < num_splits
  if constexpr (!kTok) load_pages(full_begin, a.tokens_per_split, my_page);

  // q, the B operand of K Q^T: lane (li, lg) holds head li's dims of k-step k
  // -- bf16 pools: 32k + 8lg .. +7; e4m3 pools: k = 2m + e covers
  // 16(lg + 4m) + 8e .. +7, matching the 16-byte K pieces loaded there.
  bf16x8_t qf[8];
  {
    const uint16_t* qrow = a.q + ((size_t)b * Hq + (size_t)(h0 + min(li, nh - 1))) * kD;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int d0 = kFp8 ? 16 * (lg + 4 * (k >> 1)) + 8 * (k & 1) : 32 * k + 8 * lg;
      uint4 v = ldg16(qrow + d0);
      if (li >= nh) v = make_uint4(0, 0, 0, 0);
      qf[k] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // Lengths past the capacity and page ids outside the pool break the
  // documented preconditions; both are clamped so such input yields garbage
  // in its own row instead of an access outside the buffers.
  const int capacity = kTok ? a.max_pages : a.max_pages * kPage;
  long long first_index = 0;
  const int L = seq_length(a.seq_lens, a.kv_indptr, a.index_capacity, b, capacity, &first_index);
  // First visible token: the sliding window keeps the last `window` tokens.
  const int tok_lo = a.window > 0 ? max(0, L - a.window) : 0;
  const SplitRange sr = split_range(L, a.window, a.num_splits, a.tokens_per_split,
                                    a.split_units, a.split_target);
  if (s >= sr.count) return;  // empty split: stage 2 never reads its slot
  const int tok_begin = sr.base + s * sr.tokens;
  const int tok_end = min(L, tok_begin + sr.tokens);
  const int first_page = tok_begin / kPage;
  if constexpr (kTok) {
    // one slot per token: the split's slots go to LDS (at most kMaxSplit)
    const int32_t* ids = a.kv_indptr != nullptr ? a.kv_indices + first_index : bt_row;
    for (int i = threadIdx.x; i < sr.tokens; i += kWaves * 64) {
      const int tok = tok_begin + i;
      const int idv = tok < tok_end ? ids[tok] : 0;
      tok_ids[i] = (int)min((long long)max(idv, 0), a.num_pages - 1);
    }
    __syncthreads();
  } else {
    if (tok_begin != full_begin) load_pages(tok_begin, sr.tokens, my_page);
#pragma unroll
    for (int r = 0; r < kPageRegs; ++r)
      my_page[r] = (int)min((long long)max(my_page[r], 0), a.num_pages - 1);
  }

  constexpr int kElem = kFp8 ? 1 : 2;  // bytes per pool element
  const size_t row_bytes = (size_t)Hkv * kD * kElem;    // between tokens
  const size_t page_bytes = (size_t)kPage * row_bytes;  // between pages
  const size_t head_bytes = (size_t)g * kD * kElem;
  // this head's row of token (tile i, row r) in a pool
  auto row_ptr = [&](const char* pool, int i, int r) -> const char* {
    if constexpr (kTok) {
      return pool + (size_t)tok_ids[i * kPage + r] * row_bytes + head_bytes;
    } else {
      const int j = (tok_begin / kPage + i) - first_page;  // wave-uniform
      const int pg = j < 64 ? __builtin_amdgcn_readlane(my_page[0], j)
                            : __builtin_amdgcn_readlane(my_page[1], j - 64);
      return pool + (size_t)pg * page_bytes + (size_t)r * row_bytes + head_bytes;
    }
  };

  f32x4_t o[16];  // O[head 4lg + r][d = 16t + li]
#pragma unroll
  for (int t = 0; t < 16; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;  // reference max (log2 units) of head li
  float l_row = 0.f;        // this lane's share of head li's running sum

  const int n_tiles = (tok_end - tok_begin + kPage - 1) / kPage;
  const int vis_lo = max(tok_begin, tok_lo);  // first visible token of the split
  const int first_tile = (vis_lo - tok_begin) / kPage;

  // K of tile i.  bf16: key li, dims 32k + 8lg .. +7 for k-step k (8 x 16 B).
  // e4m3: 4 x 16 B, bytes 16(lg + 4m) .. +15 of key li (k-steps 2m, 2m + 1).
  struct KRaw {
    uint4 w[kFp8 ? 4 : 8];
  };
  auto load_k = [&](int i, KRaw& kr) {
    const char* p = row_ptr(a.k_pool, i, li);
#pragma unroll
    for (int k = 0; k < (kFp8 ? 4 : 8); ++k)
      kr.w[k] = ldg16_stream(p + (kFp8 ? 16 * (lg + 4 * k) : 64 * k + 16 * lg));
  };
  // Rows outside the visible range [lo, hi) of a tile copy the nearest
  // visible row instead (finite data whose probability is exactly 0), so the
  // V copies need no branches and the compiler's wait counts stay exact.
  auto visible_rows = [&](int i, int& lo, int& hi) {
    const int t0 = tok_begin + i * kPage;
    lo = max(vis_lo, t0) - t0;
    hi = min(tok_end, t0 + kPage) - t0;
  };
  // bf16 V tile i -> LDS: copy d fills rows 2d, 2d + 1 (lane l: row
  // 2d + l/32, physical chunk l%32 <- logical chunk (l%32) ^ 2(row & 7)).
  auto stage_v = [&](int i, char* buf) {
    int lo, hi;
    visible_rows(i, lo, hi);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const int r = 2 * d + (lane >> 5);
      const int rc = min(max(r, lo), hi - 1);
      const int p = lane & 31;
      const char* src = row_ptr(a.v_pool, i, rc) + 16 * (p ^ ((r & 7) << 1));
      __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(buf + 2 * d * 512), 16, 0, kNt);
    }
  };
  // e4m3 V tile i -> LDS raw (copy d: rows 4d .. 4d + 3, 16 lanes per row).
  auto stage_v8 = [&](int i, char* raw) {
    int lo, hi;
    visible_rows(i, lo, hi);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int r = 4 * d + (lane >> 4);
      const int rc = min(max(r, lo), hi - 1);
      const char* src = row_ptr(a.v_pool, i, rc) + 16 * (lane & 15);
      __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(raw + d * 1024), 16, 0, kNt);
    }
  };
  // raw e4m3 tile -> the swizzled bf16 tile: lane l converts bytes
  // 64(l%4) .. +63 of row l/4 (logical 16-byte chunks 8(l%4) .. +7)
  auto convert_v8 = [&](const char* raw, char* buf) {
    const int r = lane >> 2, q4 = lane & 3;
    uint4 w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = *reinterpret_cast<const uint4*>(raw + r * 256 + 64 * q4 + 16 * k);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t w4[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
      uint32_t bf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bf[2 * e] = e4m3x2_to_bf16x2<false>(w4[e]);
        bf[2 * e + 1] = e4m3x2_to_bf16x2<true>(w4[e]);
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int c = 8 * q4 + 2 * k + hh;
        *reinterpret_cast<uint4*>(buf + r * 512 + 16 * (c ^ ((r & 7) << 1))) =
            make_uint4(bf[4 * hh], bf[4 * hh + 1], bf[4 * hh + 2], bf[4 * hh + 3]);
      }
    }
  };
  // transpose-read offsets: source lane (li, lg) reads row 4lg + li/4, 8 bytes
  // at logical byte 32t + 8(li&3) of the bf16 row -> chunk pair t ^ (row & 7)
  const int vrow = 4 * lg + (li >> 2);
  int voff[8];
#pragma unroll
  for (int t8 = 0; t8 < 8; ++t8) voff[t8] = vrow * 512 + 32 * (t8 ^ (vrow & 7)) + 8 * (li & 3);

  // ---- S^T = K Q^T of one tile ----------------------------------------------
  auto scores = [&](const KRaw& kr) {
    bf16x8_t kf[8];
    if constexpr (kFp8) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t w4[4] = {kr.w[m].x, kr.w[m].y, kr.w[m].z, kr.w[m].w};
        uint32_t bf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bf[2 * e] = e4m3x2_to_bf16x2<false>(w4[e]);
          bf[2 * e + 1] = e4m3x2_to_bf16x2<true>(w4[e]);
        }
        kf[2 * m] = __builtin_bit_cast(bf16x8_t, make_uint4(bf[0], bf[1], bf[2], bf[3]));
        kf[2 * m + 1] = __builtin_bit_cast(bf16x8_t, make_uint4(bf[4], bf[5], bf[6], bf[7]));
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) kf[k] = __builtin_bit_cast(bf16x8_t, kr.w[k]);
    }
    f32x4_t st = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 8; ++k) st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[k], qf[k], st, 0, 0, 0);
    return st;
  };

  // ---- mask, lazy online softmax (head li), split P, O += P V ----------------
  auto softmax_pv = [&](int i, f32x4_t st, const char* vbuf) {
    const int t0 = tok_begin + i * kPage;
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[r] = st[r] * a.scale_log2;
    if (t0 + kPage > tok_end || t0 < tok_lo) {  // a tile the range ends or starts in
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 4 * lg + r;
        sv[r] = (t < tok_end && t >= tok_lo) ? sv[r] : -INFINITY;
      }
    }
    // Lazy rescaling: probabilities are taken relative to a reference max
    // m_ref that is only raised (with a rescale of l and O) when some score of
    // the tile exceeds it by more than kSlack (log2 units); any reference
    // gives the same O, and probabilities stay in [0, 2^kSlack].
    bool raise = false;
#pragma unroll
    for (int r = 0; r < 4; ++r) raise |= sv[r] > m_ref + kSlack;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {  // wave-uniform
      float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float m_new = fmaxf(m_ref, mx);
      // a head with no visible key so far keeps -inf; its factor is then 1
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      l_row *= alpha;
      m_ref = m_new;
      // O holds heads 4lg + r: fetch those heads' factors from lanes li = 4lg + r
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __int_as_float(
            __builtin_amdgcn_ds_bpermute((4 * lg + r) << 2, __float_as_int(alpha)));
#pragma unroll
        for (int t = 0; t < 16; ++t) o[t][r] *= ar;
      }
    }
    const float mref_safe = (m_ref == -INFINITY) ? 0.f : m_ref;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = __builtin_amdgcn_exp2f(sv[r] - mref_safe);
      l_row += p[r];
    }
    // p = hi + lo, both bf16; the row sum takes p itself
    const uint32_t h01 = pk_bf16(p[0], p[1]), h23 = pk_bf16(p[2], p[3]);
    const uint32_t l01 = pk_bf16(p[0] - bf16_lo(h01), p[1] - bf16_hi(h01));
    const uint32_t l23 = pk_bf16(p[2] - bf16_lo(h23), p[3] - bf16_hi(h23));
    const s16x4_t ph = __builtin_bit_cast(s16x4_t, make_uint2(h01, h23));
    const s16x4_t pl = __builtin_bit_cast(s16x4_t, make_uint2(l01, l23));
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      s16x4_t vf[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = 4 * tg + u;
        vf[u] = lds_tr_read(vbuf + voff[t & 7] + 256 * (t >> 3));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        o[4 * tg + u] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph, vf[u], o[4 * tg + u], 0, 0, 0);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        o[4 * tg + u] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl, vf[u], o[4 * tg + u], 0, 0, 0);
    }
  };

  // One K register set per tile in flight: the next tile's K is requested as
  // soon as this tile's score MFMAs have read its registers.  bf16 V tiles
  // alternate between two buffers filled by direct copies (two tiles in
  // flight); e4m3 tiles are half the bytes, so their loop keeps two K sets
  // and two raw V tiles in flight and converts each raw tile just before its
  // P V.  The loops are unrolled twice so every buffer is named statically.
  char* bufA = vA[wave];
  char* bufB = vB[wave];
  char* bufC = vC[wave];
  int i = first_tile + wave;
  if (i < n_tiles) {
    KRaw kr;
    load_k(i, kr);
    if constexpr (kFp8) {
      KRaw kr2;
      stage_v8(i, bufB);
      if (i + kWaves < n_tiles) {
        load_k(i + kWaves, kr2);
        stage_v8(i + kWaves, bufC);
      }
      for (;;) {
        f32x4_t st = scores(kr);
        convert_v8(bufB, bufA);
        __builtin_amdgcn_sched_barrier(0);
        if (i + 2 * kWaves < n_tiles) {
          load_k(i + 2 * kWaves, kr);
          stage_v8(i + 2 * kWaves, bufB);
        }
        softmax_pv(i, st, bufA);
        i += kWaves;
        if (i >= n_tiles) break;
        st = scores(kr2);
        convert_v8(bufC, bufA);
        __builtin_amdgcn_sched_barrier(0);
        if (i + 2 * kWaves < n_tiles) {
          load_k(i + 2 * kWaves, kr2);
          stage_v8(i + 2 * kWaves, bufC);
        }
        softmax_pv(i, st, bufA);
        i += kWaves;
        if (i >= n_tiles) break;
      }
    } else {
      stage_v(i, bufA);
      for (;;) {
        f32x4_t st = scores(kr);
        __builtin_amdgcn_sched_barrier(0);
        if (i + kWaves < n_tiles) {
          load_k(i + kWaves, kr);
          stage_v(i + kWaves, bufB);
        }
        softmax_pv(i, st, bufA);
        i += kWaves;
        if (i >= n_tiles) break;
        st = scores(kr);
        __builtin_amdgcn_sched_barrier(0);
        if (i + kWaves < n_tiles) {
          load_k(i + kWaves, kr);
          stage_v(i + kWaves, bufA);
        }
        softmax_pv(i, st, bufB);
        i += kWaves;
        if (i >= n_tiles) break;
      }
    }
  }

  // ---- merge the waves' states and write the split's partial ---------------
  // Each wave's O goes to its own LDS tiles as fp32 [head][256]: heads 0-7 in
  // vA, 8-15 in vB (bf16 pools) or 8-11 in vB and 12-15 in vC (e4m3 pools).
  auto o_row = [&](int w, int hh) -> float* {
    if (hh < 8) return reinterpret_cast<float*>(vA[w]) + hh * kD;
    if (!kFp8 || hh < 12) return reinterpret_cast<float*>(vB[w]) + (hh - 8) * kD;
    return reinterpret_cast<float*>(vC[w]) + (hh - 12) * kD;
  };
  l_row += shfl_xor(l_row, 16);  // the head's four lanes hold disjoint keys
  l_row += shfl_xor(l_row, 32);
  if (lg == 0) {
    m_w[wave][li] = m_ref;
    l_w[wave][li] = l_row;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float* dst = o_row(wave, 4 * lg + r);
#pragma unroll
    for (int t = 0; t < 16; ++t) dst[16 * t + li] = o[t][r];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < nh * (kD / 4); e += kWaves * 64) {
    const int h = e / (kD / 4);
    const int c = e - h * (kD / 4);  // 4 values each
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, m_w[w][h]);
    float lam = 0.f;
    float out[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wgt = __builtin_amdgcn_exp2f(m_w[w][h] - M);  // 0 for a wave without tokens
      lam += l_w[w][h] * wgt;
      const float4 x = *reinterpret_cast<const float4*>(o_row(w, h) + 4 * c);
      out[0] = fmaf(x.x, wgt, out[0]);
      out[1] = fmaf(x.y, wgt, out[1]);
      out[2] = fmaf(x.z, wgt, out[2]);
      out[3] = fmaf(x.w, wgt, out[3]);
    }
    const size_t row = ((size_t)b * Hq + (size_t)(h0 + h)) * a.num_splits + s;
    *reinterpret_cast<float4*>(a.part_acc + row * kD + c * 4) = make_float4(out[0], out[1], out[2], out[3]);
    if (c == 0) {
      a.part_ml[row * 2 + 0] = M;
      a.part_ml[row * 2 + 1] = lam;
    }
  }
}

__global__ __launch_bounds__(512, 1) void decode_stage1_kernel(Stage1Args a) {
  stage1_valu_body<false>(a);
}

__global__ __launch_bounds__(512, 1) void decode_stage1_tok_kernel(Stage1Args a) {
  stage1_valu_body<true>(a);
}

__global__ __launch_bounds__(512, 1) void decode_stage1_mma_kernel(Stage1Args a) {
  stage1_mma_body<false, false>(a);
}

__global__ __launch_bounds__(512, 1) void decode_stage1_mma_fp8_kernel(Stage1Args a) {
  stage1_mma_body<true, false>(a);
}

__global__ __launch_bounds__(512, 1) void decode_stage1_mma_tok_kernel(Stage1Args a) {
  stage1_mma_body<false, true>(a);
}

struct Stage2Args {
  const uint16_t* gate;
  const int32_t* seq_lens;
  const float* part_acc;
  const float* part_ml;
  const float* sinks;  // [H_q] sink logits (natural-log units) or null
  const int32_t* kv_indptr;  // CSR row pointers or null (then seq_lens)
  long long index_capacity;
  uint16_t* out;
  float* lse;          // [B][H_q] or null
  float v_descale;     // e4m3 pools: V = v_descale * code value (1 for bf16)
  int num_q_heads;
  int tokens_per_split;
  int num_splits;
  int batch;
  int capacity;  // max_pages * page size
  int window;
  int split_units;
  int split_target;
};

// One wave per (b, h); lane owns d = 4*lane .. 4*lane+3.  4 waves per block.
// The per-split (m, l) pairs are wave-uniform, so every lane folds them itself
// from scalar loads (no cross-lane reduction); the partial rows are read eight
// splits at a time so that their loads are in flight together.
__global__ __launch_bounds__(256) void decode_stage2_gate_kernel(Stage2Args a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // b * H_q + h
  if (row >= a.batch * a.num_q_heads) return;
  const int lane = __lane_id();
  const int b = row / a.num_q_heads;
  const float* ml = a.part_ml + (size_t)row * a.num_splits * 2;
  const float* pa = a.part_acc + (size_t)row * a.num_splits * kD + lane * 4;
  // Issued before the length is known: the gate, the length, and the first
  // eight splits' partials (only the valid ones are used below).
  const uint2 graw = *reinterpret_cast<const uint2*>(a.gate + (size_t)row * kD + lane * 4);
  const int n0 = min(a.num_splits, 8);
  float4 x0[8];
  float2 ml0[8];
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if (u < n0) {
      x0[u] = *reinterpret_cast<const float4*>(pa + (size_t)u * kD);
      ml0[u] = *reinterpret_cast<const float2*>(ml + 2 * u);
    }
  const int h = row - b * a.num_q_heads;
  // A sink joins the denominator as one more term exp(sink) (in log2 units
  // here, like the partials' maxima); it takes no part in the numerator.
  const float sink2 = a.sinks != nullptr ? a.sinks[h] * kLog2e : -INFINITY;
  long long first_index;
  const int L = seq_length(a.seq_lens, a.kv_indptr, a.index_capacity, b, a.capacity,
                           &first_index);  // as in stage 1
  uint16_t o16[4] = {0, 0, 0, 0};
  float lse = sink2 * kLn2;  // a dead row: ln(exp(sink)), or -inf
  if (L > 0) {  // L <= 0: padded slot, output +0
    const int ns = split_range(L, a.window, a.num_splits, a.tokens_per_split, a.split_units,
                               a.split_target).count;  // >= 1 here
    float M = sink2;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (u < ns) M = fmaxf(M, ml0[u].x);
    for (int s = 8; s < ns; ++s) M = fmaxf(M, ml[2 * s]);
    float lam = a.sinks != nullptr ? __builtin_amdgcn_exp2f(sink2 - M) : 0.f;
    float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (u < ns) {
        const float w = __builtin_amdgcn_exp2f(ml0[u].x - M);
        lam = fmaf(ml0[u].y, w, lam);
        o[0] = fmaf(x0[u].x, w, o[0]);
        o[1] = fmaf(x0[u].y, w, o[1]);
        o[2] = fmaf(x0[u].z, w, o[2]);
        o[3] = fmaf(x0[u].w, w, o[3]);
      }
    for (int s0 = 8; s0 < ns; s0 += 8) {
      float4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (s0 + u < ns) x[u] = *reinterpret_cast<const float4*>(pa + (size_t)(s0 + u) * kD);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (s0 + u < ns) {
          const float w = __builtin_amdgcn_exp2f(ml[2 * (s0 + u)] - M);
          lam = fmaf(ml[2 * (s0 + u) + 1], w, lam);
          o[0] = fmaf(x[u].x, w, o[0]);
          o[1] = fmaf(x[u].y, w, o[1]);
          o[2] = fmaf(x[u].z, w, o[2]);
          o[3] = fmaf(x[u].w, w, o[3]);
        }
      }
    }
    const uint16_t gt[4] = {(uint16_t)(graw.x & 0xffff), (uint16_t)(graw.x >> 16),
                            (uint16_t)(graw.y & 0xffff), (uint16_t)(graw.y >> 16)};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint16_t ob = bf16_rne_f32(o[e] * a.v_descale / lam);
      o16[e] = gate_output(ob, gt[e]);
    }
    lse = (M + log2f(lam)) * kLn2;
  }
  if (a.lse != nullptr && lane == 0) a.lse[row] = lse;
  uint2 w;
  w.x = (uint32_t)o16[0] | ((uint32_t)o16[1] << 16);
  w.y = (uint32_t)o16[2] | ((uint32_t)o16[3] << 16);
  *reinterpret_cast<uint2*>(a.out + (size_t)row * kD + lane * 4) = w;
}

// Which stage 1 runs.  The MFMA body serves e4m3 pools (its conversions cost
// a fraction of the VALU body's), groups of more than 8 heads (one workgroup
// reads the K/V once for all 16 MFMA columns), and short capacities (splits
// under 1,024 tokens: latency-bound, where its shorter per-tile chain wins).
// The VALU body streams long bf16 sequences of groups up to 8 about 3% faster
// (measured at B=64, L=4096 with inputs rotated so no call finds the previous
// one's rows in the Infinity Cache: 91.9 vs 95.1 us per call).
// The environment variable GATED_ATTN_DECODE_STAGE1 = "mma" or "valu" forces
// one body where both apply (tests run every case through each).
bool use_mma_stage1(const DecodeLaunch& d) {
  const int group = d.num_q_heads / d.num_kv_heads;
  if (d.kv_fp8 || group > kGroup) return true;  // the VALU body takes neither
  if (const char* e = std::getenv("GATED_ATTN_DECODE_STAGE1")) {
    if (std::strcmp(e, "mma") == 0) return true;
    if (std::strcmp(e, "valu") == 0) return false;
  }
  return d.tokens_per_split < 1024;
}

hipError_t launch_decode(const DecodeLaunch& d, hipStream_t stream) {
  Stage1Args a1;
  a1.q = d.q;
  a1.k_pool = static_cast<const char*>(d.k_pool);
  a1.v_pool = static_cast<const char*>(d.v_pool);
  a1.block_table = d.block_table;
  a1.seq_lens = d.seq_lens;
  a1.kv_indptr = d.kv_indptr;
  a1.kv_indices = d.kv_indices;
  a1.index_capacity = d.index_capacity;
  a1.part_acc = d.part_acc;
  a1.part_ml = d.part_ml;
  a1.scale_log2 = d.scale * d.k_descale * kLog2e;  // the K factor folds into the scores
  a1.num_q_heads = d.num_q_heads;
  a1.num_kv_heads = d.num_kv_heads;
  a1.max_pages = d.max_pages;
  a1.num_pages = d.num_pages;
  a1.tokens_per_split = d.tokens_per_split;
  a1.num_splits = d.num_splits;
  a1.window = d.window;
  a1.split_units = d.batch * d.num_kv_heads;
  a1.split_target = d.split_target;
  a1.num_units = d.batch * d.num_kv_heads * d.num_splits;
  dim3 grid1(a1.num_units);
  hipError_t err;
  if (d.stage1_start != nullptr) {
    err = hipEventRecord(d.stage1_start, stream);
    if (err != hipSuccess) return err;
  }
  const dim3 block(kWaves * 64);
  if (use_mma_stage1(d)) {
    if (d.kv_fp8)
      hipLaunchKernelGGL(decode_stage1_mma_fp8_kernel, grid1, block, 0, stream, a1);
    else if (d.page_size == 1)
      hipLaunchKernelGGL(decode_stage1_mma_tok_kernel, grid1, block, 0, stream, a1);
    else
      hipLaunchKernelGGL(decode_stage1_mma_kernel, grid1, block, 0, stream, a1);
  } else if (d.page_size == 1) {
    hipLaunchKernelGGL(decode_stage1_tok_kernel, grid1, block, 0, stream, a1);
  } else {
    hipLaunchKernelGGL(decode_stage1_kernel, grid1, block, 0, stream, a1);
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (d.stage1_stop != nullptr) {
    err = hipEventRecord(d.stage1_stop, stream);
    if (err != hipSuccess) return err;
  }

  Stage2Args a2;
  a2.gate = d.gate;
  a2.seq_lens = d.seq_lens;
  a2.kv_indptr = d.kv_indptr;
  a2.index_capacity = d.index_capacity;
  a2.part_acc = d.part_acc;
  a2.part_ml = d.part_ml;
  a2.sinks = d.sinks;
  a2.out = d.out;
  a2.lse = d.lse;
  a2.v_descale = d.v_descale;
  a2.window = d.window;
  a2.tokens_per_split = d.tokens_per_split;
  a2.split_units = a1.split_units;
  a2.split_target = d.split_target;
  a2.num_q_heads = d.num_q_heads;
  a2.num_splits = d.num_splits;
  a2.batch = d.batch;
  a2.capacity = d.max_pages * d.page_size;
  const int rows = d.batch * a2.num_q_heads;
  hipLaunchKernelGGL(decode_stage2_gate_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, a2);
  return hipGetLastError();
}

}  // namespace ga
