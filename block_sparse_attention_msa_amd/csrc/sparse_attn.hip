// sparse_attn.hip - exact GQA attention over the selected blocks.
//
// Method ("MSA basics", vLLM MiniMax-M3.1-Flash post: the main attention runs
// exactly, but only over the kept blocks; "Prefill execution" step 4 and
// "Decode sparse GQA" of the MiniMax M3 x vLLM post: the result equals dense
// attention restricted to the selected set, computed with an online softmax
// over split work whose partial outputs are merged).
//
// Work split: (row, group) has 16 kept blocks; workgroup `split` takes 4 of
// them, one per wave, and writes an unnormalised partial (o, m, l) for the
// group's 4 query heads; a combine kernel merges the 4 partials by
// log-sum-exp.  Full K/V is read only for the kept blocks, straight from the
// paged pool (no dense staging copy).
//
// Per wave and block (NVFP4 K/V):
//  * QK: lane = (token slot, 16-dim chunk); each wave-load reads 8 tokens x
//    64 B of packed E2M1 (512 B contiguous).  E2M1 -> bf16 with
//    v_cvt_scalef32_pk_bf16_fp4 (exact), dot with the bf16 query slice on
//    v_dot2c_f32_bf16, and the chunk's E4M3 scale applied once per 16-element
//    partial dot (not once per element); K's tensor scale and sm_scale fold
//    into the exp2 argument.  Same 4-DPP-add reduction as the index scan.
//  * softmax: block max per head, p = exp2(z - m) stored to LDS per token.
//  * PV: same lane layout over V; E2M1 -> f32 pairs, the E4M3 scale folded into
//    p, fp32 FMAs into 4 heads x 16 dims per lane, reduced over the 8 token
//    slots once per block.
#include "msa_device.hpp"
#include "msa_kernels.hpp"

namespace msa {
namespace {

template <bool FP4>
struct AttnGeom {
  static constexpr int kLanesPerToken = FP4 ? 8 : 16;
  static constexpr int kLog2Lpt = FP4 ? 3 : 4;
  static constexpr int kTokensPerIter = kWave / kLanesPerToken;  // 8 or 4
  static constexpr int kIters = kBlock / kTokensPerIter;         // 16 or 32
  static constexpr int kDimsPerLane = FP4 ? 16 : 8;
  static constexpr int kPairs = kDimsPerLane / 2;
  static constexpr int kRowBytes = FP4 ? kDim / 2 : kDim * 2;    // bytes per (token, head) row
  static constexpr int kLaneBytes = FP4 ? kDimsPerLane / 2 : kDimsPerLane * 2;
};

constexpr int kDppRowRor8 = 0x128;  // lane i reads lane (i+8) mod 16 of its row (= xor 8)

template <bool FP4>
__global__ __launch_bounds__(256) void attn_partial_kernel(
    const uint8_t* __restrict__ kpool, const uint8_t* __restrict__ vpool, const uint8_t* __restrict__ k_sf,
    const uint8_t* __restrict__ v_sf, const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    const uint16_t* __restrict__ q, const int32_t* __restrict__ sel, float* __restrict__ partials, int q_len,
    int mbps, float qk_scale_log2) {
  using Geo = AttnGeom<FP4>;
  constexpr int DPL = Geo::kDimsPerLane;
  __shared__ float lds_p[4][kBlock][4];      // [wave][token][head]
  __shared__ float lds_o[4][4][kDim];        // [wave][head][dim]
  __shared__ float lds_ml[4][4][2];          // [wave][head][m, l]

  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int row = blockIdx.z;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int b = row / q_len;
  const int L = seq_lens[b];
  const int pos = L - q_len + row % q_len;
  int j = L > 0 ? sel[((size_t)row * kGroups + g) * kTopK + split * 4 + wave] : -1;
  // ids outside the row's visible blocks or the table contribute nothing
  if (j >= mbps || j * kBlock > pos) j = -1;

  const int chunk = lane & (Geo::kLanesPerToken - 1);
  const int slot = lane / Geo::kLanesPerToken;
  const bool owner = chunk < 4;        // holds a full (token, head) logit after the reduction
  const int hh = lane_group(lane);     // that head, within the group

  float m_w = -INFINITY;
  float l_lane = 0.f;
  float acc[4][DPL];
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int d = 0; d < DPL; ++d) acc[h][d] = 0.f;

  if (j >= 0) {  // wave-uniform
    const int64_t page = block_table[(size_t)b * mbps + j];
    const int64_t row0 = (page * kGroups + g) * kBlock;  // first (token, head) row of this page/head
    const int visible = pos - j * kBlock + 1;             // tokens 0..visible-1 are keys (>= 1)

    uint32_t qr[4][Geo::kPairs];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(
          q + ((size_t)row * (kGroups * kHeadsPerGroup) + g * kHeadsPerGroup + permuted_group(lane, k)) * kDim +
          chunk * DPL);
#pragma unroll
      for (int p = 0; p < Geo::kPairs; ++p) qr[k][p] = src[p];
    }

    // ---- QK
    float z[Geo::kIters];
#pragma unroll
    for (int it = 0; it < Geo::kIters; ++it) {
      const int tok = slot + it * Geo::kTokensPerIter;
      const uint8_t* kp = kpool + (row0 + tok) * Geo::kRowBytes + chunk * Geo::kLaneBytes;
      float a[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (FP4) {
        const uint2 w = *reinterpret_cast<const uint2*>(kp);
        const uint32_t ws[2] = {w.x, w.y};
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const bf16x2 e0 = e2m1x2_to_bf16x2<0>(ws[d]);
          const bf16x2 e1 = e2m1x2_to_bf16x2<1>(ws[d]);
          const bf16x2 e2 = e2m1x2_to_bf16x2<2>(ws[d]);
          const bf16x2 e3 = e2m1x2_to_bf16x2<3>(ws[d]);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            a[k] = dot2(e0, as_bf16x2(qr[k][4 * d + 0]), a[k]);
            a[k] = dot2(e1, as_bf16x2(qr[k][4 * d + 1]), a[k]);
            a[k] = dot2(e2, as_bf16x2(qr[k][4 * d + 2]), a[k]);
            a[k] = dot2(e3, as_bf16x2(qr[k][4 * d + 3]), a[k]);
          }
        }
        const float sc = e4m3_to_f32(k_sf[(row0 + tok) * (kDim / 16) + chunk]);
#pragma unroll
        for (int k = 0; k < 4; ++k) a[k] *= sc;
      } else {
        const uint4 w = *reinterpret_cast<const uint4*>(kp);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int k = 0; k < 4; ++k) a[k] = dot2(as_bf16x2(ws[d]), as_bf16x2(qr[k][d]), a[k]);
      }
      const float s = reduce4_permuted<Geo::kLog2Lpt>(a[0], a[1], a[2], a[3]);
      z[it] = tok < visible ? s * qk_scale_log2 : -INFINITY;
    }

    // ---- block softmax (per head, on the owner lanes)
    float mx = z[0];
#pragma unroll
    for (int it = 1; it < Geo::kIters; ++it) mx = fmaxf(mx, z[it]);
    m_w = wave_max_xor(mx, Geo::kLanesPerToken);
#pragma unroll
    for (int it = 0; it < Geo::kIters; ++it) {
      const float p = exp2f(z[it] - m_w);
      l_lane += p;
      if (owner) lds_p[wave][slot + it * Geo::kTokensPerIter][hh] = p;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- PV
#pragma unroll 4
    for (int it = 0; it < Geo::kIters; ++it) {
      const int tok = slot + it * Geo::kTokensPerIter;
      const float4 p4 = *reinterpret_cast<const float4*>(&lds_p[wave][tok][0]);
      const uint8_t* vp = vpool + (row0 + tok) * Geo::kRowBytes + chunk * Geo::kLaneBytes;
      float vv[DPL];
      float ph[4] = {p4.x, p4.y, p4.z, p4.w};
      if constexpr (FP4) {
        const uint2 w = *reinterpret_cast<const uint2*>(vp);
        const uint32_t ws[2] = {w.x, w.y};
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const f32x2 e0 = e2m1x2_to_f32x2<0>(ws[d]);
          const f32x2 e1 = e2m1x2_to_f32x2<1>(ws[d]);
          const f32x2 e2 = e2m1x2_to_f32x2<2>(ws[d]);
          const f32x2 e3 = e2m1x2_to_f32x2<3>(ws[d]);
          vv[8 * d + 0] = e0.x; vv[8 * d + 1] = e0.y;
          vv[8 * d + 2] = e1.x; vv[8 * d + 3] = e1.y;
          vv[8 * d + 4] = e2.x; vv[8 * d + 5] = e2.y;
          vv[8 * d + 6] = e3.x; vv[8 * d + 7] = e3.y;
        }
        const float vs = e4m3_to_f32(v_sf[(row0 + tok) * (kDim / 16) + chunk]);
#pragma unroll
        for (int h = 0; h < 4; ++h) ph[h] *= vs;
      } else {
        const uint4 w = *reinterpret_cast<const uint4*>(vp);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          vv[2 * d] = bf16lo_to_f32(ws[d]);
          vv[2 * d + 1] = bf16hi_to_f32(ws[d]);
        }
      }
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int d = 0; d < DPL; ++d) acc[h][d] = fmaf(ph[h], vv[d], acc[h][d]);
    }

    // ---- reduce over token slots
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int d = 0; d < DPL; ++d) {
        float x = acc[h][d];
        if constexpr (FP4) x += dpp<kDppRowRor8>(x);
        for (int off = 16; off < kWave; off <<= 1) x += __shfl_xor(x, off);
        acc[h][d] = x;
      }
    for (int off = Geo::kLanesPerToken; off < kWave; off <<= 1) l_lane += __shfl_xor(l_lane, off);
  }

  // ---- merge the 4 waves of this workgroup
  if (slot == 0) {
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int d = 0; d < DPL; ++d) lds_o[wave][h][chunk * DPL + d] = acc[h][d];
    if (owner) {
      lds_ml[wave][hh][0] = m_w;
      lds_ml[wave][hh][1] = l_lane;
    }
  }
  __syncthreads();
  {
    const int h = threadIdx.x >> 6;
    const int d0 = (threadIdx.x & 63) * 2;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, lds_ml[w][h][0]);
    float o0 = 0.f, o1 = 0.f, l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mw = lds_ml[w][h][0];
        if (mw == -INFINITY) continue;
        const float f = exp2f(mw - M);
        o0 = fmaf(f, lds_o[w][h][d0], o0);
        o1 = fmaf(f, lds_o[w][h][d0 + 1], o1);
        l = fmaf(f, lds_ml[w][h][1], l);
      }
    }
    float* part = partials + (((size_t)row * kGroups + g) * kAttnSplits + split) * kPartialFloats + h * (kDim + 2);
    part[d0] = o0;
    part[d0 + 1] = o1;
    if (d0 == 0) {
      part[kDim] = M;
      part[kDim + 1] = l;
    }
  }
}

// Merge the kAttnSplits partials of each (row, group) by log-sum-exp and
// normalise; rows with no keys (padded rows) get zeros.
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ partials, float* __restrict__ out,
                                                           float v_scale) {
  const int g = blockIdx.x;
  const int row = blockIdx.y;
  const int h = threadIdx.x >> 6;
  const int d0 = (threadIdx.x & 63) * 2;
  const float* base = partials + ((size_t)row * kGroups + g) * kAttnSplits * kPartialFloats + h * (kDim + 2);
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kAttnSplits; ++s) M = fmaxf(M, base[s * kPartialFloats + kDim]);
  float o0 = 0.f, o1 = 0.f, l = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int s = 0; s < kAttnSplits; ++s) {
      const float* p = base + s * kPartialFloats;
      const float ms = p[kDim];
      if (ms == -INFINITY) continue;
      const float f = exp2f(ms - M);
      o0 = fmaf(f, p[d0], o0);
      o1 = fmaf(f, p[d0 + 1], o1);
      l = fmaf(f, p[kDim + 1], l);
    }
  }
  float* o = out + ((size_t)row * (kGroups * kHeadsPerGroup) + g * kHeadsPerGroup + h) * kDim + d0;
  const float inv = l > 0.f ? v_scale / l : 0.f;
  o[0] = o0 * inv;
  o[1] = o1 * inv;
}

}  // namespace

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t stream) {
  dim3 grid(kAttnSplits, kGroups, a.rows);
  if (a.kv_nvfp4)
    attn_partial_kernel<true><<<grid, 256, 0, stream>>>(
        static_cast<const uint8_t*>(a.k), static_cast<const uint8_t*>(a.v), a.k_sf, a.v_sf, a.block_table, a.seq_lens,
        a.q, a.sel, a.partials, a.q_len, a.mbps, a.qk_scale_log2);
  else
    attn_partial_kernel<false><<<grid, 256, 0, stream>>>(
        static_cast<const uint8_t*>(a.k), static_cast<const uint8_t*>(a.v), a.k_sf, a.v_sf, a.block_table, a.seq_lens,
        a.q, a.sel, a.partials, a.q_len, a.mbps, a.qk_scale_log2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  attn_combine_kernel<<<dim3(kGroups, a.rows), 256, 0, stream>>>(a.partials, a.out, a.v_scale);
  return hipGetLastError();
}

}  // namespace msa
