// prefill.hip -- gated dense (optionally causal) attention for gfx950 with bf16
// MFMA products and fp32 online softmax, gate applied in the epilogue.
//
// cuDNN FE-OSS "Gated Attention Block (SM107)", Overview stage (4)
// O = softmax(Q K^T * scale + mask) V with GQA, stage (5) O * sigmoid(GATE);
// Forward, fuse_gate: the gate is applied inside the attention epilogue.  The
// bf16 rounding chain of the gate (bf16 O, bf16 sigmoid, rounded product) is
// the one of FreeToken PR #781, Summary.
//
// Workgroup = (16 query positions, kv head g, sequence b); 8 waves, wave w is
// query head 8g + w, so every 64-key K/V tile staged in LDS feeds 8 heads x 16
// rows.  Tiles are double-buffered in LDS; the next tile's global loads are in
// flight (in registers) while the current one is computed.
//
// MFMA v_mfma_f32_16x16x32_bf16 operand layout (wave64): A row = lane % 16,
// k = 8*(lane/16) + 0..7; B column = lane % 16, same k; C row = 4*(lane/16) + r,
// column = lane % 16, r = 0..3.  Per tile and wave:
//   S^T (64 keys x 16 rows) = K Q^T : 4 key tiles x 8 k-steps.  Computing the
//        transpose leaves each lane 4 consecutive keys of one query row, which
//        is already the A-operand layout of P for the P V product (k-slot
//        order: keys 4*(lane/16)+0..3 of two neighbouring key tiles).
//   online softmax in fp32 on that layout (lazy rescaling, see decode.hip);
//   P = Phi + Plo, two bf16 values per fp32 probability (~16 significant bits);
//   O (16 rows x 256) += Phi V + Plo V : 16 column tiles x 2 k-steps x 2.  The
//        B operand (4 consecutive keys of one V column per lane and read) comes
//        straight from row-major V in LDS through the gfx950 transpose read
//        ds_read_b64_tr_b16: within a 16-lane group, lane i of the result gets
//        element (i % 4) of the source lane 4k + i/4 in slot k, so source lane
//        s points at V[key0 + s/4][d0 + 4*(s % 4)] and result lane i receives
//        V[key0 + k][d0 + i], k = 0..3.
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
// Row strides in LDS (bf16 elements).  32 bytes of padding per row spread a
// wave's K-fragment reads (16 rows x 64 B) and V transpose reads over all
// banks; measured on gfx950, 16 bytes of padding leaves K reads ~1.5x slower.
constexpr int kKRow = kD + 16;  // K row stride: +32 B
constexpr int kVRow = kD + 16;  // V row stride: +32 B
constexpr int kThreads = 512;
constexpr int kWavesPf = kThreads / 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSlack = 8.f;  // lazy-rescale threshold, log2 units

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef s16x4 __attribute__((address_space(3))) lds_s16x4;

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

struct alignas(16) TileBuf {
  uint16_t k[kBN * kKRow];
  uint16_t v[kBN * kVRow];
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// p must point into LDS (8-byte aligned).
__device__ __forceinline__ uint2 tr_read(const uint16_t* p) {
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

__global__ __launch_bounds__(kThreads) void prefill_gate_kernel(PrefillArgs a) {
  __shared__ TileBuf buf[2];

  int mt, gp, b;
  if (!map_workgroup(a, (int)blockIdx.x, mt, gp, b)) return;
  const int S = a.seq_len;
  const int Hkv = a.num_kv_heads;
  const int Hq = a.num_q_heads;
  const int g = gp / a.parts;  // kv head
  const int part = gp - g * a.parts;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = __lane_id();
  // Waves past the workgroup's head count only help stage K/V tiles.
  const int heads = part == 0 ? a.heads_per_part : Hq / Hkv - a.heads_per_part;  // >= 1
  const bool active = wave < heads;
  const int h = g * (Hq / Hkv) + part * a.heads_per_part + min(wave, heads - 1);
  const int p0 = mt * kBM;

  const int li = lane & 15;  // query row of this lane's S^T column / MFMA column
  const int lg = lane >> 4;  // lane group: k-slot block / C row block

  // Q fragments (B operand of K Q^T): row p0 + li, d = 32*ks + 8*lg .. +7
  bf16x8 qf[8];
  {
    const int pos = min(p0 + li, S - 1);
    const uint16_t* qrow = a.q + (((size_t)b * S + pos) * Hq + h) * kD;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qf[s] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * lg));
  }

  f32x4 o[16];  // O[row 4*lg + r][d = 16*t + li]
#pragma unroll
  for (int t = 0; t < 16; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;  // reference max (log2 units) of row li
  float l_row = 0.f;        // this lane's share of the sum of row li

  const int qi = p0 + li;
  // Keys this query tile can see: [kv_lo, kv_end).  The key length masks keys
  // only; the causal mask ends at the tile's last row; the window starts at
  // the first row's window.
  const int len = a.kv_lens != nullptr ? min(max(a.kv_lens[b], 0), S) : S;
  const int kv_end = a.causal ? min(len, p0 + kBM) : len;
  const int kv_lo = a.window > 0 ? max(0, p0 - a.window + 1) : 0;
  const int kt_lo = kv_lo / kBN;
  const int n_tiles = (kv_end + kBN - 1) / kBN;  // key tiles kt_lo .. n_tiles - 1
  const size_t kv_row_stride = (size_t)Hkv * kD;
  const uint16_t* kbase = a.k + ((size_t)b * S * Hkv + g) * kD;
  const uint16_t* vbase = a.v + ((size_t)b * S * Hkv + g) * kD;

  // staging: thread covers 16-byte pieces idx = it*512 + tid of each 64 x 256
  // tile: key it*16 + tid/32, column chunk tid%32 (offsets fixed per thread)
  const int st_key = threadIdx.x >> 5;
  const int st_c = threadIdx.x & 31;
  const unsigned g_off = (unsigned)(st_key * (int)kv_row_stride + st_c * 8);
  uint4 sk[4], sv[4];
  auto load_tile = [&](int kt) {
    const int j0 = kt * kBN;
    const uint16_t* kb = kbase + (size_t)j0 * kv_row_stride;
    const uint16_t* vb = vbase + (size_t)j0 * kv_row_stride;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const unsigned off = g_off + (unsigned)(it * 16 * (int)kv_row_stride);
      sk[it] = make_uint4(0, 0, 0, 0);
      sv[it] = make_uint4(0, 0, 0, 0);
      const int j = j0 + it * 16 + st_key;
      if (j < kv_end && j >= kv_lo) {  // keys no row of the tile sees stay zero
        sk[it] = *reinterpret_cast<const uint4*>(kb + off);
        sv[it] = *reinterpret_cast<const uint4*>(vb + off);
      }
    }
  };
  auto store_tile = [&](TileBuf& tb) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int key = it * 16 + st_key;
      *reinterpret_cast<uint4*>(&tb.k[key * kKRow + st_c * 8]) = sk[it];
      *reinterpret_cast<uint4*>(&tb.v[key * kVRow + st_c * 8]) = sv[it];
    }
  };

  if (kt_lo < n_tiles) {
    load_tile(kt_lo);
    store_tile(buf[0]);
    if (kt_lo + 1 < n_tiles) load_tile(kt_lo + 1);
  }
  __syncthreads();

  for (int kt = kt_lo; kt < n_tiles; ++kt) {
    const TileBuf& tb = buf[(kt - kt_lo) & 1];
    const int j0 = kt * kBN;

    if (active) {
      // ---- S^T = K Q^T ---------------------------------------------------------
      // k-step outer, key tile inner: the four accumulators interleave, so no
      // MFMA waits on the one just issued.
      f32x4 st[4];  // st[ct][r] = S[row li][key j0 + 16*ct + 4*lg + r]
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) st[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      {
        const uint16_t* krow = &tb.k[li * kKRow + 8 * lg];
        bf16x8 kf[2][4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
          kf[0][ct] = as_bf16x8(*reinterpret_cast<const uint4*>(krow + ct * 16 * kKRow));
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          if (s + 1 < 8) {
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
              kf[(s + 1) & 1][ct] =
                  as_bf16x8(*reinterpret_cast<const uint4*>(krow + ct * 16 * kKRow + 32 * (s + 1)));
          }
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
            st[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s & 1][ct], qf[s], st[ct], 0, 0, 0);
        }
      }

      // ---- mask, lazy online softmax (row li), split P ------------------------
      // Only a tile that reaches past the first row of the query tile (causal)
      // or past the last key needs the mask; the test is uniform.
      const bool need_mask = (j0 + kBN > kv_end) || (a.causal && j0 + kBN - 1 > p0) ||
                             (a.window > 0 && j0 < p0 + kBM - a.window);
      float sv_[4][4];
      bool raise = false;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) sv_[ct][r] = st[ct][r] * a.scale_log2;
      if (need_mask) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int kj = j0 + ct * 16 + 4 * lg + r;
            const bool ok = (kj < kv_end) && (!a.causal || kj <= qi) &&
                            (a.window <= 0 || kj > qi - a.window);
            sv_[ct][r] = ok ? sv_[ct][r] : -INFINITY;
          }
      }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) raise |= sv_[ct][r] > m_ref + kSlack;
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {  // wave-uniform, rare
        float mx = -INFINITY;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sv_[ct][r]);
        mx = fmaxf(mx, shfl_xor(mx, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        const float m_new = fmaxf(m_ref, mx);
        // a row with no visible key so far keeps -inf; its factor is then 1
        const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
        l_row *= alpha;
        m_ref = m_new;
        // O holds rows 4*lg + r: fetch those rows' factors from lanes li = 4*lg + r
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ar = __int_as_float(
              __builtin_amdgcn_ds_bpermute((4 * lg + r) << 2, __float_as_int(alpha)));
#pragma unroll
          for (int t = 0; t < 16; ++t) o[t][r] *= ar;
        }
      }
      // p = hi + lo, both bf16 (hardware round-to-nearest-even conversion); the
      // row sum takes p itself (hi + lo equals p to ~2^-18 relative).
      const float mref_safe = (m_ref == -INFINITY) ? 0.f : m_ref;
      uint32_t phw[2][4], plw[2][4];  // packed bf16 A operands, k-step ks = ct / 2
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
        for (int rp = 0; rp < 2; ++rp) {
          const float pa = __builtin_amdgcn_exp2f(sv_[ct][2 * rp] - mref_safe);
          const float pb = __builtin_amdgcn_exp2f(sv_[ct][2 * rp + 1] - mref_safe);
          l_row += pa + pb;
          const uint32_t hi = cvt_pk_bf16(pa, pb);
          const uint32_t lo = cvt_pk_bf16(pa - bf16_lo(hi), pb - bf16_hi(hi));
          phw[ct >> 1][(ct & 1) * 2 + rp] = hi;
          plw[ct >> 1][(ct & 1) * 2 + rp] = lo;
        }
      }

      // ---- O += P V  (B operand through the LDS transpose read) ---------------
      // The V fragments of the next group of four column tiles are requested
      // before the current group's MFMAs are issued.
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 ph = as_bf16x8(make_uint4(phw[ks][0], phw[ks][1], phw[ks][2], phw[ks][3]));
        const bf16x8 pl = as_bf16x8(make_uint4(plw[ks][0], plw[ks][1], plw[ks][2], plw[ks][3]));
        // k-slots 0..3: keys 32ks + 4lg + 0..3; k-slots 4..7: keys 32ks + 16 + 4lg + 0..3
        const uint16_t* v0 = &tb.v[(32 * ks + 4 * lg + (li >> 2)) * kVRow + 4 * (li & 3)];
        const uint16_t* v1 = v0 + 16 * kVRow;
        bf16x8 vf[2][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint2 a0 = tr_read(v0 + 16 * u);
          const uint2 a1 = tr_read(v1 + 16 * u);
          vf[0][u] = as_bf16x8(make_uint4(a0.x, a0.y, a1.x, a1.y));
        }
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) {
          if (tg + 1 < 4) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int t = 4 * (tg + 1) + u;
              const uint2 a0 = tr_read(v0 + 16 * t);
              const uint2 a1 = tr_read(v1 + 16 * t);
              vf[(tg + 1) & 1][u] = as_bf16x8(make_uint4(a0.x, a0.y, a1.x, a1.y));
            }
          }
#pragma unroll
          for (int u = 0; u < 4; ++u)
            o[4 * tg + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vf[tg & 1][u], o[4 * tg + u], 0, 0, 0);
#pragma unroll
          for (int u = 0; u < 4; ++u)
            o[4 * tg + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vf[tg & 1][u], o[4 * tg + u], 0, 0, 0);
        }
      }
    }

    // ---- next tile: staged registers -> the other buffer ---------------------
    if (kt + 1 < n_tiles) {
      store_tile(buf[(kt + 1 - kt_lo) & 1]);
      if (kt + 2 < n_tiles) load_tile(kt + 2);
    }
    __syncthreads();
  }

  // ---- epilogue: O / l -> bf16, gate, store ------------------------------------
  // bf16(O) of the wave's 16 rows goes through LDS (the loop ended with a
  // barrier, so the tile buffers are free) from the MFMA layout (lane: 4 rows x
  // 16 strided columns) to whole 16-byte pieces of rows, so each lane issues 8
  // gate loads and 8 output stores of 16 bytes instead of 64 of 2 bytes, and
  // waits for memory once.
  if (!active) return;
  l_row += shfl_xor(l_row, 16);  // the row's four lanes hold disjoint keys
  l_row += shfl_xor(l_row, 32);
  // LDS (139,264 B): 8 x 8 KiB of bf16(O), 8 x 64 B of row flags, then a copy
  // of the sigmoid table per wave (8 x 8 KiB): 131,584 B in all
  char* const lds = reinterpret_cast<char*>(&buf[0]);
  uint16_t* const ob_lds = reinterpret_cast<uint16_t*>(lds) + wave * (kBM * kD);  // [16 rows][256]
  uint32_t* const row_flags =
      reinterpret_cast<uint32_t*>(lds + kWavesPf * kBM * kD * 2) + wave * kBM;  // bit 0 live, bit 1 dead
  uint16_t* const sig_lds =
      reinterpret_cast<uint16_t*>(lds + kWavesPf * kBM * (kD * 2 + 4)) + wave * 4096;
  {  // the table -> this wave's copy by direct copies (no registers), 1 KiB each
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(kSigmoidTable), 0, (int)sizeof(kSigmoidTable), 0x00020000);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(sig_lds + 512 * k),
                                               16, 16 * lane + 1024 * k, 0, 0, 0);
  }
  // A sink joins the denominator as one more term exp(sink) (log2 units here,
  // like m_ref); a row with no visible key (l = 0) is dead: out = +0.
  const float sink2 = a.sinks != nullptr ? a.sinks[h] * kLog2e : -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * lg + r;
    const float lr = __int_as_float(__builtin_amdgcn_ds_bpermute(row << 2, __float_as_int(l_row)));
    const float mr = __int_as_float(__builtin_amdgcn_ds_bpermute(row << 2, __float_as_int(m_ref)));
    const int qr = p0 + row;
    const bool dead = lr == 0.f;
    float mtot = mr, f = 1.f, den = lr;
    if (a.sinks != nullptr) {
      mtot = fmaxf(mr, sink2);
      f = __builtin_amdgcn_exp2f(mr - mtot);  // 0 for a dead row
      den = fmaf(lr, f, __builtin_amdgcn_exp2f(sink2 - mtot));
    }
    // O f / den through one reciprocal per row and a correction step (the
    // quotient to within about an fp32 ulp; it is rounded to bf16 next)
    const float inv = 1.f / den;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const float x = o[t][r] * f;
      const float q0 = x * inv;
      const float q = __builtin_fmaf(__builtin_fmaf(-q0, den, x), inv, q0);
      ob_lds[row * kD + 16 * t + li] = bf16_rne_f32(q);
    }
    if (li == 0) row_flags[row] = (qr < S ? 1u : 0u) | (dead ? 2u : 0u);
    if (a.lse != nullptr && li == 0 && qr < S)
      a.lse[((size_t)b * S + qr) * Hq + h] =
          (den > 0.f) ? (mtot + log2f(den)) * kLn2 : -INFINITY;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the table copies have landed
  // the wave's LDS writes above before its reads of other lanes' values below
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // piece j of this lane: row 2j + lane / 32, dims 8 (lane % 32) .. +7
  const int pc = lane & 31;
  uint4 ob8[8], gt8[8];
  uint32_t flg[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = 2 * j + (lane >> 5);
    flg[j] = row_flags[row];
    ob8[j] = *reinterpret_cast<const uint4*>(&ob_lds[row * kD + 8 * pc]);
    const int qr = min(p0 + row, S - 1);  // rows past S are not stored
    gt8[j] = *reinterpret_cast<const uint4*>(a.gate + (((size_t)b * S + qr) * Hq + h) * kD + 8 * pc);
  }
  // The gate: the sigmoid from the wave's table copy and the product in fp32
  // for all 64 elements (no branches) and the stores, then the fp64 product
  // for the rare ones whose fp32 product is not exact (zero, subnormal),
  // stored over the first result.
  uint64_t slow = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t ow[4] = {ob8[j].x, ob8[j].y, ob8[j].z, ob8[j].w};
    const uint32_t gw[4] = {gt8[j].x, gt8[j].y, gt8[j].z, gt8[j].w};
    const bool dead = (flg[j] & 2u) != 0;
    const bool live = (flg[j] & 1u) != 0;  // row inside the sequence
    uint32_t res[4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint16_t obe = (uint16_t)(ow[e >> 1] >> (16 * (e & 1)));
      const uint16_t ge = (uint16_t)(gw[e >> 1] >> (16 * (e & 1)));
      const uint16_t sb = sigmoid_from_entry(ge, sig_lds[sigmoid_table_slot(ge)]);
      uint16_t r;
      if (!gate_product_fast(obe, sb, r) && live && !dead) slow |= 1ull << (8 * j + e);
      const uint32_t rv = dead ? 0u : (uint32_t)r;
      if (e & 1) res[e >> 1] |= rv << 16; else res[e >> 1] = rv;
    }
    const int row = 2 * j + (lane >> 5);
    if (live)
      *reinterpret_cast<uint4*>(a.out + (((size_t)b * S + p0 + row) * Hq + h) * kD + 8 * pc) =
          make_uint4(res[0], res[1], res[2], res[3]);
  }
  if (slow != 0) {  // rare: re-read the element's bf16(O) and gate
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 2 * j + (lane >> 5);
      const size_t off = (((size_t)b * S + p0 + row) * Hq + h) * kD + 8 * pc;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if ((slow >> (8 * j + e)) & 1ull)
          a.out[off + e] = gate_output(ob_lds[row * kD + 8 * pc + e], a.gate[off + e]);
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
