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
//   S^T (16 keys x 16 head columns) = K Q^T, 8 MFMAs 16x16x32.  A = K
//       fragments (lane (li, lg): key li, 8 dims per k-step), B = q (column =
//       head; idle columns are zero).  Each lane then holds head li's scores
//       of keys 4lg .. 4lg+3 -- already the A layout of P for P V.
//   online softmax per head in fp32 (lazy rescaling against a reference max);
//   P = Phi + Pmid + Plo, three bf16 terms holding the fp32 weight exactly;
//   O (16 heads x 256) += P V, 16 column tiles x 3 MFMAs 16x16x16.  V needs
//       keys along k while rows are stored dims-first: gfx950's transposing
//       LDS reads (ds_read_b64_tr_b16, ds_read_b64_tr_b8) deliver it.
// Both K and V reach LDS by direct copies that read whole rows (every copy
// instruction covers whole 128-byte pieces of rows; K fragments read straight
// from HBM would cover half pieces, which measured about 8% slower), through
// buffer descriptors: the compiler tracks a buffer-form copy as a plain
// vector-memory access, so its wait counts stay exact, whereas the
// global-address form counts as a possible flat access and every wait after
// it drains all outstanding requests.  bf16 tiles are single-buffered (the
// next tile's K is requested as soon as this tile's fragments are in
// registers, its V once P V has read this tile's); e4m3 tiles are half the
// size and double-buffered.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ga_device.h"
#include "ga_internal.h"

namespace ga {

namespace {

constexpr int kD = 256;          // head dim
constexpr int kHeads = 16;       // query-head columns of a stage-1 workgroup
constexpr int kPage = 16;        // tokens per page = keys per tile
constexpr int kWaves = 8;        // waves per stage-1 workgroup (one workgroup per CU)
constexpr int kPageRegs = 2;     // page ids per lane: a wave copies at most 128 tiles of a split
constexpr int kMaxTokSplit = 2048;  // tokens of the largest split at page size 1 (slots in LDS)
constexpr int kMinSplit = 64;    // tokens of the smallest split a sizing rule asks for
constexpr int kTileBytes = kPage * kD * 2;  // one bf16 K or V tile in LDS
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
  int split_shift;   // log2 of the workgroups the sizing rule aims for
  DivU32 by_splits;  // division by num_splits
  DivU32 by_units;   // division by B * H_kv
  DivU32 by_kv;      // division by H_kv
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef s16x4_t __attribute__((address_space(3))) lds_s16x4_t;
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef i32x2_t __attribute__((address_space(3))) lds_i32x2_t;
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// K/V rows are read exactly once per call: the copies carry the non-temporal
// cache policy (bit "nt"), which keeps them from displacing reusable lines in
// L2 and the Infinity Cache (MALL).
constexpr int kNt = 2;

// One 16-byte-per-lane copy from global memory into LDS (the destination is
// wave-uniform; lane l writes lds + 16 l).  kWide = false: through a buffer
// descriptor at `base` with a 32-bit lane offset (reads past `extent` bytes
// return zeros); true: the global-address form, for offsets that do not fit
// 32 bits (its waits drain every outstanding request, see the file comment).
template <bool kWide>
__device__ __forceinline__ void copy16(const char* base, uint32_t extent, size_t off, char* lds) {
  if constexpr (kWide) {
    __builtin_amdgcn_global_load_lds(base + off, (lds_void_t*)lds, 16, 0, kNt);
  } else {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, (int)extent, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)lds, 16, (uint32_t)off, 0, 0, kNt);
  }
}

// Wait until this wave's LDS reads have returned, before a copy overwrites
// the tile they read.
__device__ __forceinline__ void lds_reads_done() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

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

__device__ __forceinline__ SplitRange split_range(int L, int window, int max_tokens, int units,
                                                  int target_shift, DivU32 by_splits, bool uneven) {
  SplitRange r;
  const int tok_lo = window > 0 ? max(0, L - window) : 0;
  r.base = tok_lo & ~(kPage - 1);
  const int n = L - r.base;
  if (n <= 0) {
    r.tokens = 0;
    r.count = 0;
    return r;
  }
  // ceil(n units / target); the target is a power of two
  long long t = ((long long)n * units + ((1LL << target_shift) - 1)) >> target_shift;
  t = max(t, (long long)kMinSplit);
  t = max(t, (long long)divu32((uint32_t)(n - 1), by_splits) + 1);  // at most num_splits splits
  // unsigned 32-bit divisions from here on (every operand is positive)
  const uint32_t un = (uint32_t)n, ti = (uint32_t)min(t, (long long)max_tokens);
  const uint32_t count = (un + ti - 1) / ti;
  r.tokens = (int)((((un + count - 1) / count) + kPage - 1) & ~(uint32_t)(kPage - 1));
  r.count = (int)((un + (uint32_t)r.tokens - 1) / (uint32_t)r.tokens);
  // More workgroups than CUs (several rounds): of two splits, split 0 --
  // dispatched first, the grid being split-major -- takes about 11/16 of the
  // tokens (at most max_tokens), so the workgroups that start last are the
  // short ones and the rounds end closer together (B=224, L 4094..6142:
  // 367.4 -> 357.1 us per call).
  if (uneven && r.count == 2) {
    const uint32_t big = min(((un * 11u + 15u) / 16u + kPage - 1) & ~(uint32_t)(kPage - 1), ti);
    if (big > (uint32_t)r.tokens && big < un) r.tokens = (int)big;
  }
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

// The same in two steps, so that the loads go out first: len_load reads the
// two words the length comes from (for a block table the second is the first
// again), len_value interprets them.
struct LenWords {
  int w0, w1;
};
__device__ __forceinline__ LenWords len_load(const int32_t* seq_lens, const int32_t* indptr, int b) {
  const int32_t* p0 = indptr != nullptr ? indptr + b : seq_lens + b;
  const int32_t* p1 = indptr != nullptr ? indptr + b + 1 : p0;
  return LenWords{*p0, *p1};
}
__device__ __forceinline__ int len_value(LenWords w, bool csr, long long index_capacity,
                                         int capacity, long long* first_index) {
  if (csr) {
    const long long lo = min(max((long long)w.w0, 0LL), index_capacity);
    const long long hi = min(max((long long)w.w1, lo), index_capacity);
    *first_index = lo;
    return (int)min(hi - lo, (long long)capacity);
  }
  *first_index = 0;
  return min(w.w0, capacity);
}

// The stage-1 body: kFp8 = e4m3 pools; kTok = one token per page
// (block-table entries or CSR indices are token slots); kWide = a page-size-1
// pool whose byte offsets do not fit 32 bits.
template <bool kFp8, bool kTok, bool kWide, int kW = kWaves>
__device__ __forceinline__ void stage1_body(const Stage1Args& a) {
  static_assert(kW == 8 || kW == 4, "tiles go to waves by a shift");
  constexpr int kLog2W = kW == 8 ? 3 : 2;
  // Per-wave LDS tiles, separate objects so the compiler can tell a copy into
  // one from a read of another (its wait before a read then covers only the
  // copy that read needs).  bf16 pools: tA = the V tile, tB = the K tile.
  // e4m3 pools: tA / tB = V tiles and tC / tD = K tiles, used in turn.  After
  // the loop they hold the wave's O (16 heads x 256 fp32 = 16 KiB) for the
  // merge.
  constexpr int kTile = kFp8 ? kTileBytes / 2 : kTileBytes;
  __shared__ __align__(16) char tA[kW][kTile];
  __shared__ __align__(16) char tB[kW][kTile];
  __shared__ __align__(16) char tC[kW][kFp8 ? kTile : 16];
  __shared__ __align__(16) char tD[kW][kFp8 ? kTile : 16];
  __shared__ float m_w[kW][kHeads], l_w[kW][kHeads];
  __shared__ __align__(16) int tok_ids[kTok ? kMaxTokSplit : 4];  // page size 1: the split's token slots

  // Workgroup id -> (split s, sequence b, kv head g).  Ids are dispatched in
  // order, round-robin over the 8 XCDs; units are split-major (every
  // sequence's split 0, then split 1, ...), so the splits a short sequence
  // leaves empty come last and the busy ones spread over all XCDs.
  const int unit = blockIdx.x;  // (s * B + b) * H_kv + g; the grid has exactly num_units
  const int seq_heads = a.split_units;  // B * H_kv
  const int s = (int)divu32((uint32_t)unit, a.by_units);
  const int rem = unit - s * seq_heads;
  const int b = (int)divu32((uint32_t)rem, a.by_kv);
  const int g = rem - b * a.num_kv_heads;
  // the length's words first: the split's range, and so every copy, waits on them
  const LenWords len_words = len_load(a.seq_lens, a.kv_indptr, b);
  const int lane = __lane_id();
  // wave-uniform by construction; readfirstlane keeps it in a scalar register
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int Hkv = a.num_kv_heads;
  const int Hq = a.num_q_heads;
  const int nh = Hq / Hkv;            // heads of the group (<= 16); columns past it are idle
  const int h0 = g * nh;              // first query head of the group
  const int li = lane & 15, lg = lane >> 4;

  // Issued together, before the length is known: the page ids of the tiles
  // this wave copies when the sequence fills its capacity (its k-th tile,
  // tile wave + kW k of split s, in lane k % 64 of register k / 64; ids past
  // the sequence's end are never used), the length, and q.  Other lengths and
  // windows reload the page ids below.  load_pages(fp, np): the split's
  // tiles from page fp on, np of them.
  const int32_t* bt_row = a.block_table + (size_t)b * a.max_pages;
  auto load_pages = [&](int fp, int np, int (&pages)[kPageRegs]) {
#pragma unroll
    for (int r = 0; r < kPageRegs; ++r) {
      const int j = wave + kW * (lane + 64 * r);
      pages[r] = j < np ? bt_row[fp + j] : 0;
    }
  };
  int my_page[kPageRegs] = {0, 0};
  const int full_begin = s * a.tokens_per_split;  // < capacity, since s < num_splits
  if constexpr (!kTok)
    load_pages(full_begin / kPage, min(a.tokens_per_split / kPage, a.max_pages - full_begin / kPage),
               my_page);

  // q, the B operand of K Q^T: lane (li, lg) holds head li's dims of k-step k
  // -- bf16 pools: 32k + 8lg .. +7; e4m3 pools: k = 2m + e covers
  // 16(lg + 4m) + 8e .. +7, matching the 16-byte K pieces read there.
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
  const int L = len_value(len_words, a.kv_indptr != nullptr, a.index_capacity, capacity, &first_index);
  // First visible token: the sliding window keeps the last `window` tokens.
  const int tok_lo = a.window > 0 ? max(0, L - a.window) : 0;
  const SplitRange sr = split_range(L, a.window, a.tokens_per_split, a.split_units, a.split_shift,
                                    a.by_splits, a.split_units * a.num_splits > (1 << a.split_shift));
  if (s >= sr.count) return;  // empty split: stage 2 never reads its slot
  const int tok_begin = sr.base + s * sr.tokens;
  const int tok_end = min(L, tok_begin + sr.tokens);
  const int n_tiles = (tok_end - tok_begin + kPage - 1) / kPage;
  const int vis_lo = max(tok_begin, tok_lo);  // first visible token of the split
  const int first_tile = (vis_lo - tok_begin) / kPage;
  if constexpr (kTok) {
    // one slot per token: the split's slots go to LDS (at most kMaxTokSplit)
    const int32_t* ids = a.kv_indptr != nullptr ? a.kv_indices + first_index : bt_row;
    for (int i = threadIdx.x; i < sr.tokens; i += kW * 64) {
      const int tok = tok_begin + i;
      const int idv = tok < tok_end ? ids[tok] : 0;
      tok_ids[i] = (int)min((long long)max(idv, 0), a.num_pages - 1);
    }
    __syncthreads();
  } else {
    if (tok_begin != full_begin || first_tile != 0)
      load_pages(tok_begin / kPage + first_tile, n_tiles - first_tile, my_page);
#pragma unroll
    for (int r = 0; r < kPageRegs; ++r)
      my_page[r] = (int)min((long long)max(my_page[r], 0), a.num_pages - 1);
  }
  // this wave's last tile index k (its tiles are first_tile + wave + kW k)
  const int k_last = (n_tiles - 1 - first_tile - wave) >> kLog2W;

  constexpr int kElem = kFp8 ? 1 : 2;  // bytes per pool element
  constexpr int kRow = kD * kElem;     // bytes of one head's row
  const size_t row_bytes = (size_t)Hkv * kRow;          // between tokens
  const size_t page_bytes = (size_t)kPage * row_bytes;  // between pages
  const size_t head_bytes = (size_t)g * kRow;
  // Bytes a copy may read from its tile base: the rest of the page, or of
  // the pool at page size 1 (the launch picks kWide when that exceeds 32 bits).
  const uint32_t extent = kTok ? (uint32_t)min((size_t)a.num_pages * row_bytes - head_bytes,
                                               (size_t)0xffffffffu)
                               : (uint32_t)(page_bytes - head_bytes);
  // Tile i's rows in a pool (i is one of this wave's tiles, i < n_tiles: a
  // wave's last tile runs after its loop and requests no next tile).
  auto tile_base = [&](const char* pool, int i) -> const char* {
    if constexpr (kTok) {
      return pool + head_bytes;
    } else {
      const int k = min((i - first_tile - wave) >> kLog2W, k_last);  // wave-uniform, < 128 (clamp: a guard)
      const int pg = __builtin_amdgcn_readlane(k < 64 ? my_page[0] : my_page[1], k & 63);
      return pool + (size_t)pg * page_bytes + head_bytes;
    }
  };
  // byte offset of row r of tile i from tile_base
  auto row_off = [&](int i, int r) -> size_t {
    if constexpr (kTok) {
      return (size_t)tok_ids[i * kPage + r] * row_bytes;
    } else {
      return (size_t)r * row_bytes;
    }
  };
  // Rows outside the visible range [lo, hi) of a tile copy the nearest
  // visible row of V instead (finite data whose probability is exactly 0).
  // K rows need no such care: their scores are replaced by -inf.
  auto visible_rows = [&](int i, int& lo, int& hi) {
    const int t0 = tok_begin + i * kPage;
    lo = max(vis_lo, t0) - t0;
    hi = min(tok_end, t0 + kPage) - t0;
  };

  // ---- HBM -> LDS copies of one tile (kRow / 16 chunks of 16 bytes per row) --
  // K: copy d fills whole rows; chunk c of row r is stored at c ^ (r & 15), so
  // a fragment read of 16 rows at one chunk touches 16 different bank groups.
  auto stage_k = [&](int i, char* buf) {
    constexpr int kChunks = kRow / 16;       // 32 (bf16) or 16 (e4m3)
    constexpr int kRowsPerCopy = 64 / kChunks;
    const char* base = tile_base(a.k_pool, i);
#pragma unroll
    for (int d = 0; d < kPage / kRowsPerCopy; ++d) {
      const int r = kRowsPerCopy * d + lane / kChunks;
      const int p = lane % kChunks;
      copy16<kWide>(base, extent, row_off(i, r) + 16 * (p ^ (r & 15)), buf + d * 1024);
    }
  };
  // bf16 V: copy d fills rows 2d, 2d + 1; chunk c of row r is stored at
  // c ^ 2(r & 7), which keeps the transposing reads below conflict-free.
  auto stage_v = [&](int i, char* buf) {
    int lo, hi;
    visible_rows(i, lo, hi);
    const char* base = tile_base(a.v_pool, i);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const int r = 2 * d + (lane >> 5);
      const int rc = min(max(r, lo), hi - 1);
      const int p = lane & 31;
      copy16<kWide>(base, extent, row_off(i, rc) + 16 * (p ^ ((r & 7) << 1)), buf + d * 1024);
    }
  };
  // e4m3 V: 32-dim granule G of row r is stored at 2048(r / 8) + 256 G +
  // 32(r % 8).  Copy d fills rows 8(d / 2) .. +7, granules 4(d % 2) .. +3:
  // lane l takes 16 bytes of row 8(d / 2) + (l / 2) % 8 at byte
  // 128(d % 2) + 32(l / 16) + 16(l % 2) -- a whole 128-byte piece per row.
  auto stage_v8 = [&](int i, char* buf) {
    int lo, hi;
    visible_rows(i, lo, hi);
    const char* base = tile_base(a.v_pool, i);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int r = 8 * (d >> 1) + ((lane >> 1) & 7);
      const int rc = min(max(r, lo), hi - 1);
      copy16<kWide>(base, extent,
                    row_off(i, rc) + (128 * (d & 1) + 32 * (lane >> 4) + 16 * (lane & 1)),
                    buf + d * 1024);
    }
  };

  // ---- LDS -> registers ------------------------------------------------------
  // K fragments, 16 bytes per piece: bf16, k-step s <- key li, chunk 4s + lg
  // (dims 32s + 8lg .. +7); e4m3, piece m <- key li, chunk lg + 4m (the dims
  // of k-steps 2m and 2m + 1, as q is laid out above).
  struct KFrag {
    uint4 w[kFp8 ? 4 : 8];
  };
  auto read_k = [&](const char* buf, KFrag& kf) {
#pragma unroll
    for (int m = 0; m < (kFp8 ? 4 : 8); ++m) {
      const int c = kFp8 ? lg + 4 * m : 4 * m + lg;
      kf.w[m] = *reinterpret_cast<const uint4*>(buf + li * kRow + 16 * (c ^ li));
    }
  };
  // bf16 V through ds_read_b64_tr_b16 (within 16 lanes, lane i of the result
  // gets element i % 4 of source lane 4k + i / 4 in slot k).  Source lane
  // (li, lg) points at key 4lg + li / 4, dims 16t + 4(li % 4) .. +3: result
  // lane (li, lg) then holds keys 4lg .. 4lg+3 of dim 16t + li, the B operand
  // of column tile t.  Offsets of tiles t and t + 8 differ by 256 bytes.
  const int vrow = 4 * lg + (li >> 2);
  int voff[8];
#pragma unroll
  for (int t8 = 0; t8 < 8; ++t8) voff[t8] = vrow * 512 + 32 * (t8 ^ (vrow & 7)) + 8 * (li & 3);
  // e4m3 V through ds_read_b64_tr_b8 (within 16 lanes, lane i of the result
  // gets byte i % 8 of source lane 2k + i / 8 in byte k).  Source lane
  // (li, lg) points at key 4lg + (li / 2) % 4, 8 bytes at dims
  // 32p + 16(li / 8) + 8(li % 2): result lane (li, lg) then holds keys
  // 4lg .. 4lg+3 of dim 32p + li in bytes 0-3 (column tile 2p) and of dim
  // 32p + 16 + li in bytes 4-7 (tile 2p + 1).  With the staging layout the
  // eight 32-byte pieces a half wave reads fall in eight different bank
  // groups, and p only moves the address by 256 p.
  const int v8row = 4 * lg + ((li >> 1) & 3);
  const int v8base = 2048 * (v8row >> 3) + 32 * (v8row & 7) + 16 * (li >> 3) + 8 * (li & 1);

  f32x4_t o[16];  // O[head 4lg + r][d = 16t + li]
#pragma unroll
  for (int t = 0; t < 16; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;  // reference max (log2 units) of head li
  float l_row = 0.f;        // this lane's share of head li's running sum

  // ---- S^T = K Q^T of one tile ----------------------------------------------
  auto scores = [&](const KFrag& kr) {
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
    // p = hi + mid + lo, three bf16 terms that hold the fp32 weight exactly
    // (each remainder is exact in fp32 and the last one fits bf16's 8 bits;
    // checked for every weight above 2^-100 -- smaller ones lie below any
    // output's resolution); the row sum takes p itself
    const uint32_t h01 = pk_bf16(p[0], p[1]), h23 = pk_bf16(p[2], p[3]);
    const float r0 = p[0] - bf16_lo(h01), r1 = p[1] - bf16_hi(h01);
    const float r2 = p[2] - bf16_lo(h23), r3 = p[3] - bf16_hi(h23);
    const uint32_t m01 = pk_bf16(r0, r1), m23 = pk_bf16(r2, r3);
    const uint32_t l01 = pk_bf16(r0 - bf16_lo(m01), r1 - bf16_hi(m01));
    const uint32_t l23 = pk_bf16(r2 - bf16_lo(m23), r3 - bf16_hi(m23));
    const s16x4_t ph = __builtin_bit_cast(s16x4_t, make_uint2(h01, h23));
    const s16x4_t pm = __builtin_bit_cast(s16x4_t, make_uint2(m01, m23));
    const s16x4_t pl = __builtin_bit_cast(s16x4_t, make_uint2(l01, l23));
    if constexpr (kFp8) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint2 w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const i32x2_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (lds_i32x2_t*)(vbuf + v8base + 256 * (4 * half + u)));
          w[u] = make_uint2((uint32_t)r[0], (uint32_t)r[1]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int t = 2 * (4 * half + u);  // column tiles t, t + 1
          const s16x4_t v0 = __builtin_bit_cast(
              s16x4_t, make_uint2(e4m3x2_to_bf16x2<false>(w[u].x), e4m3x2_to_bf16x2<true>(w[u].x)));
          const s16x4_t v1 = __builtin_bit_cast(
              s16x4_t, make_uint2(e4m3x2_to_bf16x2<false>(w[u].y), e4m3x2_to_bf16x2<true>(w[u].y)));
          o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph, v0, o[t], 0, 0, 0);
          o[t + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph, v1, o[t + 1], 0, 0, 0);
          o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pm, v0, o[t], 0, 0, 0);
          o[t + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pm, v1, o[t + 1], 0, 0, 0);
          o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl, v0, o[t], 0, 0, 0);
          o[t + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl, v1, o[t + 1], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int tg = 0; tg < 4; ++tg) {
        s16x4_t vf[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int t = 4 * tg + u;
          vf[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4_t*)(vbuf + voff[t & 7] + 256 * (t >> 3)));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          o[4 * tg + u] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph, vf[u], o[4 * tg + u], 0, 0, 0);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          o[4 * tg + u] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pm, vf[u], o[4 * tg + u], 0, 0, 0);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          o[4 * tg + u] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl, vf[u], o[4 * tg + u], 0, 0, 0);
      }
    }
  };

  int i = first_tile + wave;
  if (i < n_tiles) {
    KFrag kf;
    if constexpr (kFp8) {
      // double-buffered: the next tile's K and V are requested before this
      // tile's K fragments are read; unrolled twice so every tile in the loop
      // is named statically.  The wave's last tile runs after the loop and
      // requests nothing, so the wave does not end waiting for a copy that
      // nothing reads.
      char* const kA = tC[wave];
      char* const kB = tD[wave];
      char* const vA = tA[wave];
      char* const vB = tB[wave];
      stage_k(i, kA);
      stage_v8(i, vA);
      bool last_in_b = false;  // which buffers hold the wave's last tile
      if (i + kW < n_tiles) {
        for (;;) {
          lds_reads_done();
          stage_k(i + kW, kB);
          stage_v8(i + kW, vB);
          read_k(kA, kf);
          const f32x4_t st = scores(kf);
          __builtin_amdgcn_sched_barrier(0);
          softmax_pv(i, st, vA);
          i += kW;
          if (i + kW >= n_tiles) {
            last_in_b = true;
            break;
          }
          lds_reads_done();
          stage_k(i + kW, kA);
          stage_v8(i + kW, vA);
          read_k(kB, kf);
          const f32x4_t st2 = scores(kf);
          __builtin_amdgcn_sched_barrier(0);
          softmax_pv(i, st2, vB);
          i += kW;
          if (i + kW >= n_tiles) break;
        }
      }
      // the wave's last tile: nothing more to request
      read_k(last_in_b ? kB : kA, kf);
      const f32x4_t st = scores(kf);
      __builtin_amdgcn_sched_barrier(0);
      softmax_pv(i, st, last_in_b ? vB : vA);
    } else {
      // single-buffered (two bf16 tiles per wave fill the LDS): the next K
      // is requested once this tile's fragments are in registers, the next V
      // once P V has read this tile's; the wave's last tile, after the loop,
      // requests nothing
      char* const kbuf = tB[wave];
      char* const vbuf = tA[wave];
      stage_k(i, kbuf);
      stage_v(i, vbuf);
      while (i + kW < n_tiles) {
        read_k(kbuf, kf);
        lds_reads_done();
        stage_k(i + kW, kbuf);
        const f32x4_t st = scores(kf);
        __builtin_amdgcn_sched_barrier(0);
        softmax_pv(i, st, vbuf);
        __builtin_amdgcn_sched_barrier(0);
        lds_reads_done();
        stage_v(i + kW, vbuf);
        i += kW;
      }
      // the wave's last tile: nothing more to request
      read_k(kbuf, kf);
      const f32x4_t st = scores(kf);
      __builtin_amdgcn_sched_barrier(0);
      softmax_pv(i, st, vbuf);
    }
    // nothing is in flight here (the last tile requested nothing); kept as a
    // guard before the merge reuses the tiles
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  // ---- merge the waves' states and write the split's partial ---------------
  // Each wave's O goes to its own LDS tiles as fp32 [head][256]: heads 0-7 in
  // tA and 8-15 in tB (bf16 pools), four heads in each of tA .. tD (e4m3).
  auto o_row = [&](int w, int hh) -> float* {
    if constexpr (kFp8) {
      char* const t[4] = {tA[w], tB[w], tC[w], tD[w]};
      return reinterpret_cast<float*>(t[hh >> 2]) + (hh & 3) * kD;
    }
    return reinterpret_cast<float*>(hh < 8 ? tA[w] : tB[w]) + (hh & 7) * kD;
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
  for (int e = threadIdx.x; e < nh * (kD / 4); e += kW * 64) {
    const int h = e / (kD / 4);
    const int c = e - h * (kD / 4);  // 4 values each
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kW; ++w) M = fmaxf(M, m_w[w][h]);
    float lam = 0.f;
    float out[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kW; ++w) {
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
  stage1_body<false, false, false>(a);
}

// Splits of at most 4 tiles (short sequences at small batch): 4 waves, one
// tile each, and a 4-way merge.
__global__ __launch_bounds__(256, 1) void decode_stage1_w4_kernel(Stage1Args a) {
  stage1_body<false, false, false, 4>(a);
}

__global__ __launch_bounds__(512, 1) void decode_stage1_fp8_kernel(Stage1Args a) {
  stage1_body<true, false, false>(a);
}

__global__ __launch_bounds__(512, 1) void decode_stage1_tok_kernel(Stage1Args a) {
  stage1_body<false, true, false>(a);
}

__global__ __launch_bounds__(512, 1) void decode_stage1_tok_wide_kernel(Stage1Args a) {
  stage1_body<false, true, true>(a);
}

__global__ __launch_bounds__(512, 1) void decode_stage1_fp8_tok_kernel(Stage1Args a) {
  stage1_body<true, true, false>(a);
}

__global__ __launch_bounds__(512, 1) void decode_stage1_fp8_tok_wide_kernel(Stage1Args a) {
  stage1_body<true, true, true>(a);
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
  int split_shift;
  DivU32 by_splits;
};

// One workgroup of one wave per (b, h); lane owns d = 4*lane .. 4*lane+3.
// The per-split (m, l) pairs are wave-uniform, so every lane folds them itself
// from scalar loads (no cross-lane reduction); the partial rows are read eight
// splits at a time so that their loads are in flight together.  (Workgroups of
// 4 and 16 waves, sharing one LDS table, measured slower at B = 1: 9.55 and
// 11.6 us per call against 9.31, with the same time at B = 64.)
__global__ __launch_bounds__(64) void decode_stage2_gate_kernel(Stage2Args a) {
  // The sigmoid table -> this wave's LDS by direct copies issued first, so the
  // copy runs alongside the partials' loads and the lookups below read LDS
  // instead of making a second trip to memory (8 copies of 1 KiB).
  __shared__ uint16_t sig_tab[4096];
  const int lane = __lane_id();
  {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(kSigmoidTable), 0, (int)sizeof(kSigmoidTable), 0x00020000);
#pragma unroll
    for (int c = 0; c < 8; ++c)  // 1 KiB chunk c
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(sig_tab + 512 * c),
                                               16, 16 * lane + 1024 * c, 0, 0, 0);
  }
  const int row = blockIdx.x;  // b * H_q + h; the grid is exactly the rows
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
  uint16_t ob[4] = {0, 0, 0, 0}, gq[4] = {0, 0, 0, 0};
  bool live = false;
  float lse = sink2 * kLn2;  // a dead row: ln(exp(sink)), or -inf
  if (L > 0) {  // L <= 0: padded slot, output +0
    const int ns = split_range(L, a.window, a.tokens_per_split, a.split_units, a.split_shift,
                               a.by_splits, a.split_units * a.num_splits > (1 << a.split_shift)).count;  // >= 1 here
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
      ob[e] = bf16_rne_f32(o[e] * a.v_descale / lam);
      gq[e] = gt[e];
    }
    live = true;
    lse = (M + log2f(lam)) * kLn2;
  }
  // the table copies have landed (this wave made all of them)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (live) {
    // The product of two bf16 values has at most 16 significant bits: fp32
    // (denormals kept) holds it exactly down to 2^-134, and below that its
    // fp32 rounding cannot carry it across 2^-134, half the smallest bf16
    // step.  So one rounding of the fp32 product to bf16 is the exact
    // product's rounding for every input.
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint16_t sb = sigmoid_from_entry(gq[e], sig_tab[sigmoid_table_slot(gq[e])]);
      o16[e] = bf16_rne_f32(bf16_to_f32(ob[e]) * bf16_to_f32(sb));
    }
  }
  if (a.lse != nullptr && lane == 0) a.lse[row] = lse;
  uint2 w;
  w.x = (uint32_t)o16[0] | ((uint32_t)o16[1] << 16);
  w.y = (uint32_t)o16[2] | ((uint32_t)o16[3] << 16);
  *reinterpret_cast<uint2*>(a.out + (size_t)row * kD + lane * 4) = w;
}

// Page size 1: the copies address a token's row by a 32-bit offset from the
// pool's start unless the pool's rows span more bytes than that; then the
// 64-bit address form is used.  The choice follows from the pool's size alone.
bool wide_offsets(const DecodeLaunch& d) {
  const unsigned long long bytes =
      (unsigned long long)d.num_pages * d.num_kv_heads * kD * (d.kv_fp8 ? 1 : 2);
  return bytes > 0xffffffffull;
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
  a1.split_shift = 0;
  while ((1 << a1.split_shift) < d.split_target) ++a1.split_shift;  // a power of two
  a1.by_splits = divu32_make((uint32_t)d.num_splits);
  a1.by_units = divu32_make((uint32_t)(a1.split_units > 0 ? a1.split_units : 1));
  a1.by_kv = divu32_make((uint32_t)d.num_kv_heads);
  a1.num_units = d.batch * d.num_kv_heads * d.num_splits;
  dim3 grid1(a1.num_units);
  hipError_t err;
  const dim3 block(kWaves * 64);
  if (d.kv_fp8 && d.page_size == 1 && wide_offsets(d))
    hipLaunchKernelGGL(decode_stage1_fp8_tok_wide_kernel, grid1, block, 0, stream, a1);
  else if (d.kv_fp8 && d.page_size == 1)
    hipLaunchKernelGGL(decode_stage1_fp8_tok_kernel, grid1, block, 0, stream, a1);
  else if (d.kv_fp8)
    hipLaunchKernelGGL(decode_stage1_fp8_kernel, grid1, block, 0, stream, a1);
  else if (d.page_size == 1 && wide_offsets(d))
    hipLaunchKernelGGL(decode_stage1_tok_wide_kernel, grid1, block, 0, stream, a1);
  else if (d.page_size == 1)
    hipLaunchKernelGGL(decode_stage1_tok_kernel, grid1, block, 0, stream, a1);
  else if (d.tokens_per_split <= 4 * kPage)
    hipLaunchKernelGGL(decode_stage1_w4_kernel, grid1, dim3(4 * 64), 0, stream, a1);
  else
    hipLaunchKernelGGL(decode_stage1_kernel, grid1, block, 0, stream, a1);
  err = hipGetLastError();
  if (err != hipSuccess) return err;

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
  a2.split_shift = a1.split_shift;
  a2.by_splits = a1.by_splits;
  a2.num_q_heads = d.num_q_heads;
  a2.num_splits = d.num_splits;
  a2.batch = d.batch;
  a2.capacity = d.max_pages * d.page_size;
  const int rows = d.batch * a2.num_q_heads;
  hipLaunchKernelGGL(decode_stage2_gate_kernel, dim3(rows), dim3(64), 0, stream, a2);
  return hipGetLastError();
}

}  // namespace ga
