// prefill.hip -- gated dense (optionally causal) attention for gfx950 with bf16
// MFMA products and fp32 online softmax, gate applied in the epilogue.
//
// cuDNN FE-OSS "Gated Attention Block (SM107)", Overview stage (4)
// O = softmax(Q K^T * scale + mask) V with GQA, stage (5) O * sigmoid(GATE);
// Forward, fuse_gate: the gate is applied inside the attention epilogue.  The
// bf16 rounding chain of the gate (bf16 O, bf16 sigmoid, rounded product) is
// the one of FreeToken PR #781, Summary.
//
// Workgroup = (16 query positions, kv head g, sequence b, head part); 8 waves,
// two per SIMD, wave w serving query head w of the part (up to 8 heads), so a
// 64-key K or V tile staged in LDS feeds the whole part.  The tiles reach LDS
// by direct copies (buffer loads into LDS, no registers), two buffers each for
// K and V: the copies of tile t + 1 are issued while the scores of tile t are
// computed, so they have the whole of tile t to land.  One barrier per tile;
// all waves are in the same phase (scores, softmax, P V) at about the same
// time, which keeps the LDS reading one kind of operand at a time.
//
// MFMA v_mfma_f32_16x16x32_bf16 operand layout (wave64): A row = lane % 16,
// k = 8*(lane/16) + 0..7; B column = lane % 16, same k; C row = 4*(lane/16) + r,
// column = lane % 16, r = 0..3.  Per tile, wave and head:
//   S^T (64 keys x 16 rows) = K Q^T : 4 key tiles x 8 k-steps.  Computing the
//        transpose leaves each lane 4 consecutive keys of one query row, which
//        is already the A-operand layout of P for the P V product (k-slot
//        order: keys 4*(lane/16)+0..3 of two neighbouring key tiles).
//   online softmax in fp32 on that layout (lazy rescaling, see decode.hip);
//   P = Phi + Plo, two bf16 values per fp32 probability (~16 significant bits);
//   O (16 rows x 256) += Phi V + Plo V : 16 column tiles x 2 k-steps x 2.  The
//        B operand (4 consecutive keys of one V column per lane and read) comes
//        from V in LDS through the gfx950 transpose read ds_read_b64_tr_b16:
//        within a 16-lane group, lane i of the result gets element (i % 4) of
//        the source lane 4k + i/4 in slot k, so source lane s points at
//        V[key0 + s/4][d0 + 4*(s % 4)] and result lane i receives
//        V[key0 + k][d0 + i], k = 0..3.
// LDS rows are 512 bytes with 16-byte chunks swizzled by row (K: chunk c of
// row r at c ^ (r & 15); V: at c ^ 2(r & 7)), so each 16-lane read touches
// every bank group once; each copy instruction fills two whole rows.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ga_device.h"
#include "ga_internal.h"

namespace ga {

namespace {

constexpr int kD = 256;
constexpr int kBM = 16;    // query positions per workgroup
constexpr int kBN = 64;    // keys per tile
constexpr int kH = 1;                // query heads per wave
constexpr int kWavesPf = kMaxHeadsPerPart / kH;
constexpr int kThreads = 64 * kWavesPf;
constexpr int kCopyRows = kBN / kWavesPf;     // tile rows each wave copies
constexpr int kCopies = kCopyRows / 2;        // copy instructions per wave per tile (K or V)
constexpr int kTileBytes = kBN * kD * 2;  // one K or V tile (32 KiB)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSlack = 8.f;  // lazy-rescale threshold, log2 units
static_assert(kH * kWavesPf == kMaxHeadsPerPart, "a workgroup serves a head part");
static_assert(kCopies == 4 || kCopies == 8, "copy instructions ride with the P V groups");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef s16x4 __attribute__((address_space(3))) lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* gate;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float scale_log2;
  int causal;
  int seq_len;
  int num_q_heads;
  int num_kv_heads;
  int parts;           // workgroups per (sequence, kv head, query tile): 1 or 2
  int heads_per_part;  // query heads of part 0: G, or ceil(G / 2) (<= 8); part 1 has the rest
  int batch;
  int num_m_tiles;
  // attention-spec options (null / 0: plain attention)
  const int32_t* kv_lens;  // [B] key lengths: keys j >= kv_lens[b] are masked
  const float* sinks;      // [H_q] sink logits (natural-log units)
  float* lse;              // [B][S][H_q] natural-log log-sum-exp
  int window;              // > 0: row i sees keys j > i - window
};

// Workgroup order.  Workgroups are dispatched round-robin over the 8 XCDs of
// an MI355X, each with its own L2.  Every query tile of one (sequence, kv
// head, head part) slice re-reads that slice's K/V, so the slices are pinned to XCDs
// (8 / slices XCDs per slice, or slices / 8 slices per XCD) to keep a slice's
// K/V in one L2, and within an XCD the heaviest causal tiles (latest query
// positions) go first.  Returns false for the few padding ids of the grid.
constexpr int kXcds = 8;

__device__ __forceinline__ bool map_workgroup(const PrefillArgs& a, int id, int& mt, int& gp, int& b) {
  const int slices = a.batch * a.num_kv_heads * a.parts;
  const int nm = a.num_m_tiles;
  int slice, slot;
  const int xcd = id % kXcds, k = id / kXcds;
  if (slices <= kXcds && kXcds % slices == 0) {
    const int per = kXcds / slices;  // XCDs per slice
    slice = xcd / per;
    slot = k * per + xcd % per;
  } else if (slices % kXcds == 0) {
    const int per = slices / kXcds;  // slices per XCD
    slice = xcd * per + k % per;
    slot = k / per;
  } else {  // no even split: heaviest first across all slices
    slice = id % slices;
    slot = id / slices;
  }
  if (slot >= nm) return false;
  mt = nm - 1 - slot;
  gp = slice % (a.num_kv_heads * a.parts);  // kv head * parts + part
  b = slice / (a.num_kv_heads * a.parts);
  return true;
}

// Grid size for map_workgroup: every (slice, m tile) pair gets an id.
__host__ __forceinline__ int grid_size(int slices, int nm) {
  if (slices <= kXcds && kXcds % slices == 0) {
    const int per = kXcds / slices;
    return kXcds * ((nm + per - 1) / per);
  }
  if (slices % kXcds == 0) return kXcds * (slices / kXcds) * nm;
  return slices * nm;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// p must point into LDS (8-byte aligned).
__device__ __forceinline__ uint2 tr_read(const char* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(uint2, r);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair (v_cvt_pk_bf16_f32, round to nearest even);
// used for the P operand only, whose precision the hi/lo split restores.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float x, float y) {
  const f32x2 v = {x, y};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

}  // namespace

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPf / 4, kWavesPf / 4)))
void prefill_gate_kernel(PrefillArgs a) {
  // K and V tiles, two of each, as separate objects: the compiler then tells
  // a direct copy into one tile from a read of another, and waits only for
  // the copies a read needs.
  __shared__ __align__(16) char k0[kTileBytes];
  __shared__ __align__(16) char k1[kTileBytes];
  __shared__ __align__(16) char v0[kTileBytes];
  __shared__ __align__(16) char v1[kTileBytes];

  int mt, gp, b;
  if (!map_workgroup(a, (int)blockIdx.x, mt, gp, b)) return;
  const int S = a.seq_len;
  const int Hkv = a.num_kv_heads;
  const int Hq = a.num_q_heads;
  const int g = gp / a.parts;  // kv head
  const int part = gp - g * a.parts;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = __lane_id();
  // Heads of this part; wave w serves part heads kH w .. kH w + kH - 1 (kH = 1:
  // head w).  A wave past the part's heads only helps copy K/V; with kH = 2 a
  // missing second head computes a copy of the first and is not stored.
  const int heads = part == 0 ? a.heads_per_part : Hq / Hkv - a.heads_per_part;  // >= 1
  const bool active = kH * wave < heads;
  const bool second = kH * wave + 1 < heads;  // (kH == 2) the wave's second head is real
  const int hbase = g * (Hq / Hkv) + part * a.heads_per_part;
  int hw[kH];
#pragma unroll
  for (int h = 0; h < kH; ++h) hw[h] = hbase + min(kH * wave + h, heads - 1);
  const int p0 = mt * kBM;

  const int li = lane & 15;  // query row of this lane's S^T column / MFMA column
  const int lg = lane >> 4;  // lane group: k-slot block / C row block
  const int qi = p0 + li;

  // Keys this query tile can see: [kv_lo, kv_end).  The key length masks keys
  // only; the causal mask ends at the tile's last row; the window starts at
  // the first row's window.
  const int len = a.kv_lens != nullptr ? min(max(a.kv_lens[b], 0), S) : S;
  const int kv_end = a.causal ? min(len, p0 + kBM) : len;
  const int kv_lo = a.window > 0 ? max(0, p0 - a.window + 1) : 0;
  const int kt_lo = kv_lo / kBN;
  const int n_tiles = (kv_end + kBN - 1) / kBN;  // key tiles kt_lo .. n_tiles - 1
  const int row_bytes = Hkv * kD * 2;            // between consecutive keys

  // ---- direct HBM/L2 -> LDS copies of one tile ---------------------------------
  // Wave w copies rows kCopyRows w .. + kCopyRows - 1 of the tile's K and of
  // its V (kCopies instructions each, two whole rows per instruction).  The
  // copies go through one buffer descriptor per tensor whose range is the
  // visible keys [kv_lo, kv_end): a row outside it reads as zeros (finite data
  // whose probability is exactly 0, or, for K, whose score is replaced by
  // -inf), so no offset needs clamping.  The per-lane part of every offset is
  // fixed; a tile adds one uniform term.
  const size_t key_lo = ((size_t)b * S * Hkv + (size_t)kv_lo * Hkv + g) * kD;  // elements
  const int vis_bytes = max(kv_end - kv_lo, 0) * row_bytes;  // the descriptors' range (0: no key)
  uint32_t lane_off[2][kCopies];                        // [K / V][instruction]
#pragma unroll
  for (int d = 0; d < kCopies; ++d) {
    const int r = kCopyRows * wave + 2 * d + (lane >> 5);  // tile row
    const int p = lane & 31;                               // 16-byte slot in the row
    lane_off[0][d] = (uint32_t)(r * row_bytes + 16 * (p ^ (r & 15)));         // K chunk stored there
    lane_off[1][d] = (uint32_t)(r * row_bytes + 16 * (p ^ ((r & 7) << 1)));  // V chunk
  }
  // copy_one(.., d): instruction d (0 .. kCopies - 1) of this wave's share of
  // tile kt of K (is_v false) or V
  auto copy_one = [&](const uint16_t* base, int kt, char* buf, bool is_v, int d) {
    // the descriptor from wave-uniform values, kept in scalar registers
    const uintptr_t addr = reinterpret_cast<uintptr_t>(base + key_lo);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(((uintptr_t)hi << 32) | lo), 0,
        __builtin_amdgcn_readfirstlane(vis_bytes), 0x00020000);
    // rows before kv_lo wrap to offsets far past the range (modulo 2^32)
    const uint32_t tile = (uint32_t)(kt * kBN - kv_lo) * (uint32_t)row_bytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(buf + (kCopyRows * wave + 2 * d) * 512), 16,
                                             lane_off[is_v][d] + tile, 0, 0, 0);
  };
  auto copy_tile = [&](const uint16_t* base, int kt, char* buf, bool is_v) {
#pragma unroll
    for (int d = 0; d < kCopies; ++d) copy_one(base, kt, buf, is_v, d);
  };

  // Q fragments (B operand of K Q^T) of the wave's heads: row p0 + li, d = 32*ks + 8*lg .. +7
  bf16x8 qf[kH][8];
  {
    const int pos = min(qi, S - 1);
#pragma unroll
    for (int h = 0; h < kH; ++h) {
      const uint16_t* qrow = a.q + (((size_t)b * S + pos) * Hq + hw[h]) * kD;
#pragma unroll
      for (int s = 0; s < 8; ++s)
        qf[h][s] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * lg));
    }
  }

  f32x4 o[kH][16];  // O[head][row 4*lg + r][d = 16*t + li]
#pragma unroll
  for (int h = 0; h < kH; ++h)
#pragma unroll
    for (int t = 0; t < 16; ++t) o[h][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref[kH], l_row[kH];  // reference max (log2 units) of row li; this lane's share of its sum
#pragma unroll
  for (int h = 0; h < kH; ++h) {
    m_ref[h] = -INFINITY;
    l_row[h] = 0.f;
  }

  // ---- S^T = K Q^T of one tile for the wave's heads -------------------------------
  // k-step outer, key tile inner: eight accumulators interleave.
  // hook(s) runs after the K reads of k-step s + 1 are issued: the next
  // tile's copies ride along with the MFMAs (issued early, so they have the
  // whole tile to land) instead of stalling on their own
  // LDS offsets of the lane's K fragment pieces, fixed for the whole loop: key
  // row 16 ct + li, chunk 4 s + lg stored at (4 s + lg) ^ li (ct: immediate)
  uint32_t k_lane[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) k_lane[s] = (uint32_t)(li * 512 + 16 * ((4 * s + lg) ^ li));
  auto scores = [&](const char* kb, f32x4 (&st)[kH][4], auto&& hook) {
#pragma unroll
    for (int h = 0; h < kH; ++h)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) st[h][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 kf[2][4];
    auto read_k = [&](int s, bf16x8 (&dst)[4]) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        dst[ct] = as_bf16x8(*reinterpret_cast<const uint4*>(kb + k_lane[s] + ct * 16 * 512));
    };
    read_k(0, kf[0]);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s + 1 < 8) read_k(s + 1, kf[(s + 1) & 1]);
      hook(s);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int h = 0; h < kH; ++h)
          st[h][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s & 1][ct], qf[h][s], st[h][ct], 0, 0, 0);
    }
    // issue order: the fragments of k-step s + 1 are read before the MFMAs of
    // k-step s, so each read has eight MFMAs to land
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s + 1 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, kCopies / 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * kH, 0);
    }
  };

  // ---- mask, lazy online softmax (row li), split P ----------------------------------
  // p = hi + lo, both bf16 (hardware round-to-nearest-even conversion); the row
  // sum takes p itself (hi + lo equals p to ~2^-18 relative).
  // The visible keys of row qi, less the lane's key offset 4 lg within a
  // 16-key group: j < kv_end, j <= qi when causal, j > qi - window with a window
  const int key_last = min(kv_end - 1, a.causal ? qi : INT_MAX) - 4 * lg;
  const int key_first = (a.window > 0 ? qi - a.window + 1 : 0) - 4 * lg;
  auto softmax = [&](int kt, f32x4 (&st)[kH][4], uint32_t (&phw)[kH][2][4], uint32_t (&plw)[kH][2][4]) {
    const int j0 = kt * kBN;
    // Only a tile that reaches past the first row of the query tile (causal),
    // past the last key, or before the window needs the mask; the test is uniform.
    const bool need_mask = (j0 + kBN > kv_end) || (a.causal && j0 + kBN - 1 > p0) ||
                           (a.window > 0 && j0 < p0 + kBM - a.window);
#pragma unroll
    for (int h = 0; h < kH; ++h) {
      // raw scores (the scale is applied inside the exponent below); masked
      // keys get -inf
      float sv[4][4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) sv[ct][r] = st[h][ct][r];
      if (need_mask) {
        // key j0 + 16 ct + 4 lg + r is visible iff 16 ct + r lies in
        // [key_first - j0, key_last - j0] (the lane's bounds, fixed per row)
        const int hi_c = key_last - j0, lo_c = key_first - j0;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) sv[ct][r] = 16 * ct + r <= hi_c ? sv[ct][r] : -INFINITY;
        if (a.window > 0) {
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) sv[ct][r] = 16 * ct + r >= lo_c ? sv[ct][r] : -INFINITY;
        }
      }
      // the lane's largest score, scaled (the scale is positive, so this is the
      // largest scaled score)
      float mx = sv[0][0];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sv[ct][r]);
      mx *= a.scale_log2;
      if (__builtin_amdgcn_ballot_w64(mx > m_ref[h] + kSlack) != 0) {  // wave-uniform, rare
        mx = fmaxf(mx, shfl_xor(mx, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        const float m_new = fmaxf(m_ref[h], mx);
        // a row with no visible key so far keeps -inf; its factor is then 1
        const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref[h] - m_new);
        l_row[h] *= alpha;
        m_ref[h] = m_new;
        // O holds rows 4*lg + r: fetch those rows' factors from lanes li = 4*lg + r
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ar = __int_as_float(
              __builtin_amdgcn_ds_bpermute((4 * lg + r) << 2, __float_as_int(alpha)));
#pragma unroll
          for (int t = 0; t < 16; ++t) o[h][t][r] *= ar;
        }
      }
      const float neg_m = (m_ref[h] == -INFINITY) ? 0.f : -m_ref[h];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
        for (int rp = 0; rp < 2; ++rp) {
          const float pa = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[ct][2 * rp], a.scale_log2, neg_m));
          const float pb = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[ct][2 * rp + 1], a.scale_log2, neg_m));
          l_row[h] += pa + pb;
          const uint32_t hi = cvt_pk_bf16(pa, pb);
          const uint32_t lo = cvt_pk_bf16(pa - bf16_lo(hi), pb - bf16_hi(hi));
          phw[h][ct >> 1][(ct & 1) * 2 + rp] = hi;
          plw[h][ct >> 1][(ct & 1) * 2 + rp] = lo;
        }
      }
    }
  };

  // ---- O += P V  (B operand through the LDS transpose read) ---------------------
  // V row r, dims 16t + 4(li % 4) .. +3 sit at r * 512 + 32 (t8 ^ (r & 7)) +
  // 256 (t / 8) + 8 (li % 4), t8 = t % 8; k-slots 0..3 of k-step ks are keys
  // 32ks + 4lg + 0..3 (rows 32ks + 4lg + li / 4 as sources), k-slots 4..7 the
  // same 16 keys later.
  // LDS offsets of the lane's transpose-read sources, fixed for the whole loop:
  // row vr = 4 lg + li / 4 of a 16-key group, dims 16 t + 4 (li % 4) .. +3 of
  // column tile t at 32 (t % 8 ^ (vr & 7)) + 256 (t / 8) + 8 (li % 4)
  // (as addresses in v0: inside the loop a read of v1 adds a constant, which
  // fits the read's immediate offset, so no tile adds a base; the last tile's
  // buffer is chosen at run time and adds one register offset)
  const int vr = 4 * lg + (li >> 2);
  const char* vsrc[8];
#pragma unroll
  for (int t8 = 0; t8 < 8; ++t8) vsrc[t8] = v0 + vr * 512 + 32 * (t8 ^ (vr & 7)) + 8 * (li & 3);
  auto pv = [&](const char* vb, const uint32_t (&phw)[kH][2][4], const uint32_t (&plw)[kH][2][4]) {
    bf16x8 ph[2][kH], pl[2][kH];  // [k-step][head]
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int h = 0; h < kH; ++h) {
        ph[ks][h] = as_bf16x8(make_uint4(phw[h][ks][0], phw[h][ks][1], phw[h][ks][2], phw[h][ks][3]));
        pl[ks][h] = as_bf16x8(make_uint4(plw[h][ks][0], plw[h][ks][1], plw[h][ks][2], plw[h][ks][3]));
      }
    // group gi = (k-step gi / 4, column tiles 4 (gi % 4) .. +3)
    auto read_v = [&](int gi, bf16x8 (&dst)[4]) {
      const int ks = (int)(vb - v0) + 32 * (gi >> 2) * 512;  // a constant inside the loop
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = 4 * (gi & 3) + u;
        const char* const src = vsrc[t & 7] + ks + 256 * (t >> 3);
        const uint2 x0 = tr_read(src);
        const uint2 x1 = tr_read(src + 16 * 512);
        dst[u] = as_bf16x8(make_uint4(x0.x, x0.y, x1.x, x1.y));
      }
    };
    bf16x8 vf[2][4];
    read_v(0, vf[0]);
#pragma unroll
    for (int gi = 0; gi < 8; ++gi) {
      if (gi + 1 < 8) read_v(gi + 1, vf[(gi + 1) & 1]);
      const int ks = gi >> 2, tg = gi & 3;
      // every head's P_hi terms, then the P_lo terms: each accumulator's two
      // MFMAs are 4 kH MFMAs apart
#pragma unroll
      for (int h = 0; h < kH; ++h)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          o[h][4 * tg + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph[ks][h], vf[gi & 1][u], o[h][4 * tg + u], 0, 0, 0);
#pragma unroll
      for (int h = 0; h < kH; ++h)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          o[h][4 * tg + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl[ks][h], vf[gi & 1][u], o[h][4 * tg + u], 0, 0, 0);
    }
    // issue order: the V fragments of group gi + 1 are read before the 16
    // MFMAs of group gi
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int gi = 0; gi < 8; ++gi) {
      if (gi + 1 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 8 * kH, 0);
    }
  };

  // ---- the tile loop ----------------------------------------------------------------
  // Iteration t (buffers named statically: the loop is unrolled twice):
  //   barrier -- K(t) and V(t) have landed; every wave is done with tile t - 1
  //   copies of K(t+1) and V(t+1) into the buffers tile t - 1 used
  //   S(t) = K(t) Q^T;  softmax -> P(t);  O += P(t) V(t)
  // and the last tile the same without copies, after the loop.
  //
  // The gate rows of the wave's heads, as 16-byte pieces of rows (piece j:
  // row 2j + lane / 32, dims 8 (lane % 32) .. +7), requested at the start of
  // the last tile so that their latency overlaps its work.
  const int pc = lane & 31;
  uint4 gt8[kH][8];
  auto load_gate = [&]() {
#pragma unroll
    for (int h = 0; h < kH; ++h)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int qr = min(p0 + 2 * j + (lane >> 5), S - 1);  // rows past S are not stored
        gt8[h][j] = *reinterpret_cast<const uint4*>(a.gate + (((size_t)b * S + qr) * Hq + hw[h]) * kD + 8 * pc);
      }
  };
  if (kt_lo < n_tiles) {
    copy_tile(a.k, kt_lo, k0, false);
    copy_tile(a.v, kt_lo, v0, true);
    f32x4 st[kH][4];
    uint32_t phw[kH][2][4], plw[kH][2][4];
    auto step = [&](int kt, char* kc, char* vc, char* kn, char* vn) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      // The next tile's copies (a step never runs the last tile), issued
      // among the score MFMAs.
      if (active) {
        // the K instructions with k-steps 0..3, the V ones with 4..7
        scores(kc, st, [&](int gi) {
#pragma unroll
          for (int e = 0; e < kCopies / 4; ++e)
            copy_one(gi < 4 ? a.k : a.v, kt + 1, gi < 4 ? kn : vn, gi >= 4,
                     (kCopies / 4) * (gi & 3) + e);
        });
        softmax(kt, st, phw, plw);
        pv(vc, phw, plw);
      } else {
        copy_tile(a.k, kt + 1, kn, false);
        copy_tile(a.v, kt + 1, vn, true);
      }
    };
    // The last tile: no copies to issue; the gate rows are requested first.
    // It runs after the loop, from the buffers its parity selects, so the gate
    // registers are live only from here on (a loop body that could be the
    // last tile would hold them through every tile).
    auto last_step = [&](int kt, char* kc, char* vc) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (active) {
        load_gate();
        scores(kc, st, [&](int) {});
        softmax(kt, st, phw, plw);
        pv(vc, phw, plw);
      }
    };
    int kt = kt_lo;
    if (kt + 1 < n_tiles) {
      for (;;) {
        step(kt, k0, v0, k1, v1);
        if (++kt + 1 >= n_tiles) break;
        step(kt, k1, v1, k0, v0);
        if (++kt + 1 >= n_tiles) break;
      }
    }
    const bool odd = ((kt - kt_lo) & 1) != 0;  // uniform: which buffers hold the last tile
    last_step(kt, odd ? k1 : k0, odd ? v1 : v0);
  } else if (active) {
    load_gate();  // no visible key: every row is dead, the values are not used
  }

  // ---- epilogue: O / l -> bf16, gate, store ------------------------------------
  // The gate rows are in flight since the last tile.  bf16(O) of the
  // wave's kH x 16 rows goes through LDS from the MFMA layout (lane: 4 rows x 16
  // strided columns) to whole 16-byte pieces of rows, so each lane issues 8 kH
  // gate loads and 8 kH output stores of 16 bytes instead of 64 kH of 2 bytes.
  __syncthreads();  // every wave is done with the tiles: their LDS is reused below
  // Regions: this wave's kH x 8 KiB of bf16(O) in the K tiles, and one sigmoid
  // table for the workgroup in the first V tile, extended so that it holds
  // every gate's result without range tests: index
  //   sign * 2304 + (exponent - 117) * 128 + mantissa
  // for the gate's magnitude bits (exponent, mantissa) clamped to the range
  // of buckets 117 .. 134, where bucket 117 stands for |g| < 2^-9 (result
  // 0.5), buckets 118 .. 133 are the correctly rounded table, and bucket 134
  // for |g| >= 128 (1, or +0 for negative g).  Only NaN gates need a test of
  // their own.  Two gates (one 32-bit word) are indexed at a time in 16-bit
  // lanes.
  constexpr int kRegion = kH * kBM * kD * 2;
  constexpr int kPerTile = kTileBytes / kRegion;  // regions per K tile buffer
  static_assert(kPerTile * 2 >= kWavesPf, "the epilogue regions fit the K tile buffers");
  static_assert(2 * 18 * 128 * 2 <= kTileBytes, "the extended table fits a V tile buffer");
  char* const lds = (wave < kPerTile ? k0 : k1) + (wave % kPerTile) * kRegion;
  uint16_t* const ob_lds = reinterpret_cast<uint16_t*>(lds);  // [head][16 rows][256]
  uint16_t* const sig_lds = reinterpret_cast<uint16_t*>(v0);
  {
    // the 4,096-entry table by direct copies: 512 pieces of 16 bytes, one per
    // lane of the 8 waves; piece c holds entries 8c .. 8c + 7 (sign c / 256)
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(kSigmoidTable), 0, (int)sizeof(kSigmoidTable), 0x00020000);
    static_assert(kWavesPf == 8, "one table piece per lane of 8 waves");
    const int sgn = wave >> 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (lds_void*)(sig_lds + sgn * 2304 + 128 + 512 * (wave & 3)), 16, 16 * lane + 1024 * wave, 0, 0,
        0);
    // the constant buckets: waves 0 / 1 write sign 0 / 1, lanes 0-31 bucket
    // 117 and lanes 32-63 bucket 134, four entries each
    if (wave < 2) {
      const uint32_t big = wave == 0 ? 0x3f803f80u : 0u;
      const uint32_t v = lane < 32 ? 0x3f003f00u : big;
      const int ent = wave * 2304 + (lane < 32 ? 0 : 2176) + 4 * (lane & 31);
      *reinterpret_cast<uint2*>(sig_lds + ent) = make_uint2(v, v);
    }
  }
  if (active) {
#pragma unroll
    for (int h = 0; h < kH; ++h) {
      const int hq = hw[h];
      float lr_own = l_row[h];
      lr_own += shfl_xor(lr_own, 16);  // the row's four lanes hold disjoint keys
      lr_own += shfl_xor(lr_own, 32);
      // A sink joins the denominator as one more term exp(sink) (log2 units
      // here, like m_ref); a row with no visible key (l = 0) is dead: out = +0.
      const float sink2 = a.sinks != nullptr ? a.sinks[hq] * kLog2e : -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * lg + r;
        const float lr = __int_as_float(__builtin_amdgcn_ds_bpermute(row << 2, __float_as_int(lr_own)));
        const float mr = __int_as_float(__builtin_amdgcn_ds_bpermute(row << 2, __float_as_int(m_ref[h])));
        const int qr = p0 + row;
        float mtot = mr, f = 1.f, den = lr;
        if (a.sinks != nullptr) {
          mtot = fmaxf(mr, sink2);
          f = __builtin_amdgcn_exp2f(mr - mtot);  // 0 for a dead row
          den = fmaf(lr, f, __builtin_amdgcn_exp2f(sink2 - mtot));
        }
        // O f / den as O times one factor per row (within about an fp32 ulp
        // of the quotient; it is rounded to bf16 next), rounded two at a time
        // by the hardware conversion (round to nearest even; denormals kept)
        const float gq = f / den;
#pragma unroll
        for (int t = 0; t < 16; t += 2) {
          const uint32_t pk = cvt_pk_bf16(o[h][t][r] * gq, o[h][t + 1][r] * gq);
          ob_lds[(h * kBM + row) * kD + 16 * t + li] = (uint16_t)pk;
          ob_lds[(h * kBM + row) * kD + 16 * (t + 1) + li] = (uint16_t)(pk >> 16);
        }
        if (a.lse != nullptr && li == 0 && qr < S && (h == 0 || second))
          a.lse[((size_t)b * S + qr) * Hq + hq] = (den > 0.f) ? (mtot + log2f(den)) * kLn2 : -INFINITY;
      }
    }
  }
  // the table copies and the gate rows have landed; the whole table and every
  // wave's bf16(O) are in LDS
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (!active) return;
  // The gate: bf16(O) times the sigmoid, in fp32, rounded once by the
  // conversion.  Both factors are bf16, so their product has at most 16
  // significant bits and fp32 holds it exactly down to 2^-134 (fp32
  // denormals are kept); below that the fp32 rounding cannot move it across
  // 2^-134, half the smallest bf16 step, so its bf16 rounding is the exact
  // product's in every case.
#pragma unroll
  for (int h = 0; h < kH; ++h) {
    if (h == 1 && !second) break;
    const int hq = hw[h];
    float lr_own = l_row[h];  // as above: row li's sum, for the dead-row test
    lr_own += shfl_xor(lr_own, 16);
    lr_own += shfl_xor(lr_own, 32);
    // this lane's 16 bytes of row p0 + lane / 32; piece j is 2j rows further
    uint16_t* const out_row = a.out + (((size_t)b * S + p0 + (lane >> 5)) * Hq + hq) * kD + 8 * pc;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 2 * j + (lane >> 5);
      const float lr = __int_as_float(__builtin_amdgcn_ds_bpermute(row << 2, __float_as_int(lr_own)));
      const bool dead = lr == 0.f;
      const uint4 ob8 = *reinterpret_cast<const uint4*>(&ob_lds[(h * kBM + row) * kD + 8 * pc]);
      const uint32_t ow[4] = {ob8.x, ob8.y, ob8.z, ob8.w};
      const uint32_t gw[4] = {gt8[h][j].x, gt8[h][j].y, gt8[h][j].z, gt8[h][j].w};
      uint32_t res[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        // both gates of the word at once (16-bit lanes): the magnitude clamped
        // to [bucket 117, mantissa 0 .. bucket 134, mantissa 127] indexes the
        // extended table directly, the sign adds one table of 2304 entries
        const u16x2 g2 = __builtin_bit_cast(u16x2, gw[e2]);
        const u16x2 mag = g2 & (u16x2)0x7fff;
        const u16x2 cl = __builtin_elementwise_min(__builtin_elementwise_max(mag, (u16x2)0x3a80),
                                                   (u16x2)0x437f);
        const u16x2 soff = __builtin_bit_cast(u16x2, __builtin_bit_cast(i16x2, g2) >> 15) & (u16x2)2304;
        const uint32_t ix = __builtin_bit_cast(uint32_t, soff + cl);
        const uint32_t t0 = sig_lds[(ix & 0xffffu) - 0x3a80u];
        const uint32_t t1 = sig_lds[(ix >> 16) - 0x3a80u];
        // NaN gates (magnitude above 0x7f80) give NaN: bit 15 of mag + 0x7f
        const uint32_t nan = __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2, mag + (u16x2)0x7f) >> 15);
        const uint32_t sw = ((t0 | (t1 << 16)) & ~nan) | (0x7fc07fc0u & nan);
        const float pr0 = bf16_lo(ow[e2]) * bf16_lo(sw);
        const float pr1 = bf16_hi(ow[e2]) * bf16_hi(sw);
        res[e2] = dead ? 0u : cvt_pk_bf16(pr0, pr1);
      }
      // rows past the sequence are not stored; the output is written with the
      // non-temporal hint (it is not read again by this kernel)
      if (p0 + row < S)
        __builtin_nontemporal_store(u32x4{res[0], res[1], res[2], res[3]},
                                    reinterpret_cast<u32x4*>(out_row + (size_t)j * (2 * Hq * kD)));
    }
  }
}

hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t stream) {
  PrefillArgs a;
  a.q = p.q;
  a.gate = p.gate;
  a.k = p.k;
  a.v = p.v;
  a.out = p.out;
  a.scale_log2 = p.scale * kLog2e;
  a.causal = p.causal;
  a.seq_len = p.seq_len;
  a.num_q_heads = p.num_q_heads;
  a.num_kv_heads = p.num_kv_heads;
  const int group = p.num_q_heads / p.num_kv_heads;
  a.parts = head_parts(group);
  a.heads_per_part = (group + a.parts - 1) / a.parts;
  a.batch = p.batch;
  a.num_m_tiles = (p.seq_len + kBM - 1) / kBM;
  a.kv_lens = p.kv_lens;
  a.sinks = p.sinks;
  a.lse = p.lse;
  a.window = p.window;
  dim3 grid(grid_size(p.batch * p.num_kv_heads * a.parts, a.num_m_tiles));
  hipLaunchKernelGGL(prefill_gate_kernel, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ga
