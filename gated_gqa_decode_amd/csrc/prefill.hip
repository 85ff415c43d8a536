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
// query head 8g + w, so every K/V tile staged in LDS feeds 8 heads x 16 rows.
// Per 64-key tile and wave:
//   S (16x64)  = Q K^T   : 4 column tiles x 8 k-steps of v_mfma_f32_16x16x32_bf16
//   online softmax in fp32 on the accumulator layout
//   P = Phi + Plo, two bf16 values per fp32 probability (~16 significant bits)
//              -> per-wave LDS tiles, re-read in the MFMA A-operand layout
//   O (16x256) += Phi V + Plo V : 16 column tiles x 2 k-steps x 2; V is stored transposed
//                          in LDS so each lane's 8 keys of one column are
//                          contiguous.
// MFMA 16x16x32 operand layout (wave64): A row i = lane % 16, k = 8*(lane/16)
// + 0..7; B column j = lane % 16, same k; C row = 4*(lane/16) + r, column =
// lane % 16, r = 0..3.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ga_device.h"
#include "ga_internal.h"

namespace ga {

namespace {

constexpr int kD = 256;
constexpr int kGroup = 8;
constexpr int kBM = 16;    // query positions per workgroup
constexpr int kBN = 64;    // keys per tile
constexpr int kKRow = kD + 8;     // K row stride in LDS (bf16): +16 B breaks bank aliasing
constexpr int kVRow = kBN + 8;    // V^T row stride in LDS (bf16)
constexpr int kPRow = kBN + 8;    // P row stride in LDS (bf16)
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* gate;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float scale_log2;
  int causal;
  int seq_len;
  int num_kv_heads;
  int num_m_tiles;
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ float rowmax16(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  v = fmaxf(v, dpp<kDppMirror>(v));
  return v;
}

}  // namespace

__global__ __launch_bounds__(512) void prefill_gate_kernel(PrefillArgs a) {
  __shared__ uint16_t ks[kBN * kKRow];          // K tile  [key][d]
  __shared__ uint16_t vts[kD * kVRow];          // V tile transposed [d][key]
  __shared__ uint16_t ps[kGroup][2][kBM * kPRow];  // per-wave P hi/lo [row][key]

  // heaviest (latest) query tiles first under the causal mask
  const int mt = a.num_m_tiles - 1 - (int)blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int S = a.seq_len;
  const int Hkv = a.num_kv_heads;
  const int Hq = Hkv * kGroup;
  const int wave = threadIdx.x >> 6;
  const int lane = __lane_id();
  const int h = g * kGroup + wave;
  const int p0 = mt * kBM;

  const int li = lane & 15;   // A row / B column / C column
  const int lk = lane >> 4;   // k group (8 values) / C row group (4 rows)

  // Q fragments: row p0 + li, d = 32*kstep + 8*lk .. +7
  bf16x8 qf[8];
  {
    const int pos = min(p0 + li, S - 1);
    const uint16_t* qrow = a.q + (((size_t)b * S + pos) * Hq + h) * kD;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * lk));
  }

  f32x4 o[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[4], l_run[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
  }

  const int kv_end = a.causal ? min(S, p0 + kBM) : S;
  const int n_tiles = (kv_end + kBN - 1) / kBN;
  const size_t kv_row_stride = (size_t)Hkv * kD;
  const uint16_t* kbase = a.k + ((size_t)b * S * Hkv + g) * kD;
  const uint16_t* vbase = a.v + ((size_t)b * S * Hkv + g) * kD;

  for (int kt = 0; kt < n_tiles; ++kt) {
    const int j0 = kt * kBN;
    __syncthreads();  // previous tile fully consumed
    // ---- stage K (row-major) and V (transposed) for keys j0 .. j0+63 -------
    // K: a wave reads two whole 512-byte rows per instruction.
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = it * 512 + threadIdx.x;  // 2048 16-byte pieces per tile
      const int key = idx >> 5;
      const int c = idx & 31;
      uint4 kv4 = make_uint4(0, 0, 0, 0);
      if (j0 + key < kv_end)
        kv4 = *reinterpret_cast<const uint4*>(kbase + (size_t)(j0 + key) * kv_row_stride + c * 8);
      *reinterpret_cast<uint4*>(&ks[key * kKRow + c * 8]) = kv4;
    }
    // V: consecutive lanes take consecutive keys of one 16-byte column chunk, so
    // the transposed 2-byte LDS writes of a wave land in consecutive addresses.
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = it * 512 + threadIdx.x;
      const int key = idx & 63;
      const int c = idx >> 6;
      uint4 vv4 = make_uint4(0, 0, 0, 0);
      if (j0 + key < kv_end)
        vv4 = *reinterpret_cast<const uint4*>(vbase + (size_t)(j0 + key) * kv_row_stride + c * 8);
      const uint32_t w[4] = {vv4.x, vv4.y, vv4.z, vv4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vts[(c * 8 + 2 * e) * kVRow + key] = (uint16_t)(w[e] & 0xffff);
        vts[(c * 8 + 2 * e + 1) * kVRow + key] = (uint16_t)(w[e] >> 16);
      }
    }
    __syncthreads();

    // ---- S = Q K^T -----------------------------------------------------------
    f32x4 sacc[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      sacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* krow = &ks[(ct * 16 + li) * kKRow + 8 * lk];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 kf = as_bf16x8(*reinterpret_cast<const uint4*>(krow + 32 * s));
        sacc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[s], kf, sacc[ct], 0, 0, 0);
      }
    }
    // ---- mask + online softmax (rows 4*lk + r, columns 16*ct + li) ----------
    float pv[4][4];
    uint16_t phi[4][4], plo[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int qi = p0 + 4 * lk + r;
      float mx = -INFINITY;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int kj = j0 + ct * 16 + li;
        const bool ok = (kj < kv_end) && (!a.causal || kj <= qi);
        const float sv = ok ? sacc[ct][r] * a.scale_log2 : -INFINITY;
        pv[r][ct] = sv;
        mx = fmaxf(mx, sv);
      }
      mx = rowmax16(mx);
      const float m_new = fmaxf(m_run[r], mx);
      // a row whose keys so far are all masked keeps m = -inf; use 0 as the
      // reference so exp2 sees -inf - 0 (never -inf - -inf).
      const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[r] - m_ref);
      float rs = 0.f;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        pv[r][ct] = __builtin_amdgcn_exp2f(pv[r][ct] - m_ref);
        // split p = hi + lo into two bf16 values (together ~16 significant
        // bits), so the bf16 MFMA products keep the fp32 softmax's precision
        const uint16_t hi = bf16_rne_f32(pv[r][ct]);
        const uint16_t lo = bf16_rne_f32(pv[r][ct] - bf16_to_f32(hi));
        phi[r][ct] = hi;
        plo[r][ct] = lo;
        rs += bf16_to_f32(hi) + bf16_to_f32(lo);
      }
      rs += dpp<kDppXor1>(rs);
      rs += dpp<kDppXor2>(rs);
      rs += dpp<kDppHalfMirror>(rs);
      rs += dpp<kDppMirror>(rs);
      l_run[r] = l_run[r] * alpha + rs;
      m_run[r] = m_new;
#pragma unroll
      for (int t = 0; t < 16; ++t) o[t][r] *= alpha;
    }
    // ---- P (bf16 hi/lo) to LDS: accumulator layout -> A-operand layout ------
    uint16_t* pwh = ps[wave][0];
    uint16_t* pwl = ps[wave][1];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        pwh[(4 * lk + r) * kPRow + ct * 16 + li] = phi[r][ct];
        pwl[(4 * lk + r) * kPRow + ct * 16 + li] = plo[r][ct];
      }
    wave_lds_sync();
    bf16x8 pfh[2], pfl[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      pfh[s] = as_bf16x8(*reinterpret_cast<const uint4*>(&pwh[li * kPRow + 32 * s + 8 * lk]));
      pfl[s] = as_bf16x8(*reinterpret_cast<const uint4*>(&pwl[li * kPRow + 32 * s + 8 * lk]));
    }
    // ---- O += P V --------------------------------------------------------------
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const uint16_t* vrow = &vts[(t * 16 + li) * kVRow + 8 * lk];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 vf = as_bf16x8(*reinterpret_cast<const uint4*>(vrow + 32 * s));
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pfh[s], vf, o[t], 0, 0, 0);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pfl[s], vf, o[t], 0, 0, 0);
      }
    }
    wave_lds_sync();
  }

  // ---- epilogue: O / l -> bf16, gate, store -----------------------------------
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int qi = p0 + 4 * lk + r;
    if (qi >= S) continue;
    const size_t rowoff = (((size_t)b * S + qi) * Hq + h) * kD;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int d = t * 16 + li;
      const uint16_t ob = bf16_rne_f32(o[t][r] / l_run[r]);
      a.out[rowoff + d] = gate_output(ob, a.gate[rowoff + d]);
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
  a.num_kv_heads = p.num_kv_heads;
  a.num_m_tiles = (p.seq_len + kBM - 1) / kBM;
  dim3 grid(a.num_m_tiles, p.num_kv_heads, p.batch);
  hipLaunchKernelGGL(prefill_gate_kernel, grid, dim3(512), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ga
