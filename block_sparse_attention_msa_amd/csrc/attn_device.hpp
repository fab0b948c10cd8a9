// attn_device.hpp - one workgroup of the exact GQA attention over the kept
// blocks of one (query row, group, head pair), optionally preceded by the
// exact block selection of that (row, group).
//
// Method ("MSA basics", vLLM MiniMax-M3.1-Flash post: the main attention runs
// exactly, but only over the kept blocks, and every query head of a GQA group
// attends over its group's blocks; "Prefill execution" step 4 and "Decode
// sparse GQA" of the MiniMax M3 x vLLM post: the result equals dense attention
// restricted to the selected set, computed with an online softmax over split
// work whose partial outputs are merged).
//
// One 1024-thread workgroup per (row, group, head pair).  Each of the 16 waves
// takes one of the 16 kept blocks, and the waves' partial (o, m, l) are merged
// by log-sum-exp in LDS, so every head's softmax completes inside one
// workgroup and the output is written directly (no cross-workgroup merge).
// Full K/V is read only for the kept blocks, straight from the paged pool.
//
// Per wave and block (NVFP4 K/V):
//  * QK: lane = (token slot, 16-dim chunk); all 16 wave-loads of the block's K
//    (8 tokens x 64 B of packed E2M1 each, 512 B contiguous) are issued before
//    use, and the block's 1 KB of E4M3 scales is transposed through LDS.
//    E2M1 -> bf16 with v_cvt_scalef32_pk_bf16_fp4 (exact), dot with the bf16
//    query slices of the 2 heads on v_dot2c_f32_bf16, the chunk's E4M3 scale
//    applied once per 16-element partial dot; K's tensor scale and sm_scale
//    fold into the exp2 argument.  The 8-lane reduction of the 2 head partials
//    costs 3 DPP adds (lane-dependent head order).
//  * softmax over the wave's block, p = exp2(z - m) stored to LDS;
//  * PV: V loads issued before the softmax; E2M1 -> f32 pairs, the E4M3 scale
//    folded into p, fp32 FMAs into 2 heads x 16 dims per lane; token-slot pairs
//    summed with one DPP add, the rest through LDS with the waves'
//    exp2(m_w - M) weights.
#pragma once

#include <type_traits>

#include "msa_device.hpp"
#include "select_device.hpp"

namespace msa {

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
  using Vec = typename std::conditional<FP4, uint2, uint4>::type;  // one lane's bytes of one token
  static constexpr int kChunk = FP4 ? 16 : 8;                        // loads issued together
  static constexpr int kScaleBytes = FP4 ? kBlock * (kDim / 16) : 16;
};

// LDS written by some lanes of a wave and read by others of the same wave.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int kAttnThreads = 1024;
constexpr int kAttnWaves = kAttnThreads / kWave;  // 16
constexpr int kAttnHeads = 2;                         // query heads per workgroup
constexpr int kAttnBlocksPerWave = kTopK / kAttnWaves;    // 1
static_assert(kAttnBlocksPerWave == 1, "one kept block per wave");
constexpr int kAttnHeadPairs = kHeadsPerGroup / kAttnHeads;
constexpr int kAttnSlotGroups = 4;                    // token-slot groups left after the in-register step
constexpr int kDppRowRor8 = 0x128;                // lane i reads lane (i+8) mod 16 of its row (= xor 8)

struct MergeSmem {
  float o[kAttnWaves][kAttnSlotGroups][kAttnHeads][kDim];     // 64 KB
};

// Linear workgroup id -> (row, group, head pair).  Workgroups are dispatched
// round-robin over the 8 XCDs (id % 8); the two head-pair workgroups of one
// (row, group) get ids 8 apart so they share an XCD and its L2, and the second
// read of the group's K/V blocks hits there.
__device__ __forceinline__ void attn_decode_wg(int id, int& row, int& g, int& hp) {
  const int x = id & 7;
  hp = (id >> 3) & 1;
  const int pair = (id >> 4) * 8 + x;
  row = pair / kGroups;
  g = pair % kGroups;
}

// 2 per-lane partial dots a0, a1 belong to heads (0 ^ (lane&1)) and (1 ^ (lane&1));
// after the reduction over 2^LOG2 lanes, lanes whose bits 1..LOG2-1 are zero
// hold the full dot of head (lane & 1).
template <int LOG2>
__device__ __forceinline__ float reduce2_permuted(float a0, float a1) {
  a0 += dpp<kDppXor1>(a1);
  a0 += dpp<kDppXor2>(a0);
  a0 += dpp<kDppRowShl4>(a0);
  if constexpr (LOG2 == 4) a0 += dpp<kDppRowShl8>(a0);
  return a0;
}

template <bool FP4>
struct AttnSmem {
  union {
    SelectSmem<kAttnThreads> sel;
    MergeSmem merge;
  } u;
  float p[kAttnWaves][kBlock][kAttnHeads];                   // 16 KB
  uint8_t sc[kAttnWaves][AttnGeom<FP4>::kScaleBytes];     // 16 KB (NVFP4 scales)
  float ml[kAttnWaves][kAttnHeads][2];
  int32_t sel[kTopK];
};

// Selection (SELECT: from the block scores) and attention of (row, g, head pair hp).  Every thread of the
// workgroup must call it.
template <bool FP4, bool SELECT>
__device__ __forceinline__ void attn_workgroup(
    const uint8_t* __restrict__ kpool, const uint8_t* __restrict__ vpool, const uint8_t* __restrict__ k_sf,
    const uint8_t* __restrict__ v_sf, const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    const uint16_t* __restrict__ q, const float* __restrict__ block_scores, const int32_t* __restrict__ sel_in,
    int32_t* __restrict__ sel_out, float* __restrict__ out, int q_len, int mbps, float qk_scale_log2, float v_scale,
    int row, int g, int hp, AttnSmem<FP4>& sm) {
  using Geo = AttnGeom<FP4>;
  constexpr int DPL = Geo::kDimsPerLane;
  constexpr int ITERS = Geo::kIters;
  auto& U = sm.u;
  auto& lds_p = sm.p;
  auto& lds_sc = sm.sc;
  auto& lds_ml = sm.ml;
  auto& lds_sel = sm.sel;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int b = row / q_len;
  const int L = seq_lens[b];
  const int head0 = g * kHeadsPerGroup + hp * kAttnHeads;   // first query head of this workgroup
  float* out_row = out + ((size_t)row * (kGroups * kHeadsPerGroup) + head0) * kDim;

  if (L <= 0) {  // padded row
    if (tid < kAttnHeads * kDim) out_row[tid] = 0.f;
    if (SELECT && sel_out && hp == 0 && tid < kTopK) sel_out[((size_t)row * kGroups + g) * kTopK + tid] = -1;
    return;
  }
  const int pos = L - q_len + row % q_len;
  if constexpr (SELECT) {
    const int r = min(pos / kBlock, mbps - 1);
    select_blocks<kAttnThreads>(block_scores + ((size_t)row * kGroups + g) * mbps, r, U.sel, lds_sel);
    if (sel_out && hp == 0 && tid < kTopK) sel_out[((size_t)row * kGroups + g) * kTopK + tid] = lds_sel[tid];
  } else {
    if (tid < kTopK) lds_sel[tid] = sel_in[((size_t)row * kGroups + g) * kTopK + tid];
    __syncthreads();
  }

  const int chunk = lane & (Geo::kLanesPerToken - 1);
  const int slot = lane / Geo::kLanesPerToken;
  const bool owner = chunk < kAttnHeads;   // holds a full (token, head) logit after the reduction
  const int hh = lane & 1;             // that head, within the pair

  int j = lds_sel[wave];
  // ids outside the row's visible blocks or the table contribute nothing
  if (j >= mbps || j * kBlock > pos) j = -1;

  float m_w = -INFINITY;
  float l_lane = 0.f;
  if (j >= 0) {  // wave-uniform
    using Vec = typename Geo::Vec;
    constexpr int CHUNK = Geo::kChunk;
    const int64_t page = block_table[(size_t)b * mbps + j];
    const int64_t row0 = (page * kGroups + g) * kBlock;  // first (token, head) row of this page/head
    const int visible = pos - j * kBlock + 1;             // tokens 0..visible-1 are keys (>= 1)
    const uint8_t* kbase = kpool + row0 * Geo::kRowBytes + slot * Geo::kRowBytes + chunk * Geo::kLaneBytes;
    const uint8_t* vbase = vpool + row0 * Geo::kRowBytes + slot * Geo::kRowBytes + chunk * Geo::kLaneBytes;
    constexpr int kIterStride = Geo::kTokensPerIter * Geo::kRowBytes;  // bytes between iterations

    // ---- issue every K load of the first chunk (all of them for NVFP4) before any use
    Vec kb[CHUNK];
#pragma unroll
    for (int i = 0; i < CHUNK; ++i) kb[i] = *reinterpret_cast<const Vec*>(kbase + i * kIterStride);
    uint4 sc16 = make_uint4(0, 0, 0, 0);
    if constexpr (FP4) sc16 = *reinterpret_cast<const uint4*>(k_sf + row0 * (kDim / 16) + lane * 16);

    uint32_t qr[kAttnHeads][Geo::kPairs];
#pragma unroll
    for (int k = 0; k < kAttnHeads; ++k) {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(
          q + ((size_t)row * (kGroups * kHeadsPerGroup) + head0 + (k ^ hh)) * kDim + chunk * DPL);
#pragma unroll
      for (int p = 0; p < Geo::kPairs; ++p) qr[k][p] = src[p];
    }
    // the block's 1 KB of E4M3 scales, transposed through LDS: the scale of
    // (token slot + 8 it, chunk) is byte 64 it + lane
    if constexpr (FP4) {
      *reinterpret_cast<uint4*>(&lds_sc[wave][lane * 16]) = sc16;
      wave_sync();
    }

    // ---- QK
    float z[ITERS];
#pragma unroll
    for (int c0 = 0; c0 < ITERS; c0 += CHUNK) {
      if (c0 > 0) {
#pragma unroll
        for (int i = 0; i < CHUNK; ++i) kb[i] = *reinterpret_cast<const Vec*>(kbase + (c0 + i) * kIterStride);
      }
#pragma unroll
      for (int i = 0; i < CHUNK; ++i) {
        const int it = c0 + i;
        float a0 = 0.f, a1 = 0.f;
        if constexpr (FP4) {
          const uint32_t ws[2] = {kb[i].x, kb[i].y};
#pragma unroll
          for (int d = 0; d < 2; ++d) {
            const bf16x2 e0 = e2m1x2_to_bf16x2<0>(ws[d]);
            const bf16x2 e1 = e2m1x2_to_bf16x2<1>(ws[d]);
            const bf16x2 e2 = e2m1x2_to_bf16x2<2>(ws[d]);
            const bf16x2 e3 = e2m1x2_to_bf16x2<3>(ws[d]);
            a0 = dot2(e0, as_bf16x2(qr[0][4 * d + 0]), a0);
            a1 = dot2(e0, as_bf16x2(qr[1][4 * d + 0]), a1);
            a0 = dot2(e1, as_bf16x2(qr[0][4 * d + 1]), a0);
            a1 = dot2(e1, as_bf16x2(qr[1][4 * d + 1]), a1);
            a0 = dot2(e2, as_bf16x2(qr[0][4 * d + 2]), a0);
            a1 = dot2(e2, as_bf16x2(qr[1][4 * d + 2]), a1);
            a0 = dot2(e3, as_bf16x2(qr[0][4 * d + 3]), a0);
            a1 = dot2(e3, as_bf16x2(qr[1][4 * d + 3]), a1);
          }
          const float sc = e4m3_to_f32(lds_sc[wave][it * kWave + lane]);
          a0 *= sc;
          a1 *= sc;
        } else {
          const uint32_t ws[4] = {kb[i].x, kb[i].y, kb[i].z, kb[i].w};
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            a0 = dot2(as_bf16x2(ws[d]), as_bf16x2(qr[0][d]), a0);
            a1 = dot2(as_bf16x2(ws[d]), as_bf16x2(qr[1][d]), a1);
          }
        }
        const float s = reduce2_permuted<Geo::kLog2Lpt>(a0, a1);
        const int tok = slot + it * Geo::kTokensPerIter;
        z[it] = tok < visible ? s * qk_scale_log2 : -INFINITY;
      }
    }

    // ---- issue the first chunk of V loads, then the softmax while they fly
    Vec vb[CHUNK];
#pragma unroll
    for (int i = 0; i < CHUNK; ++i) vb[i] = *reinterpret_cast<const Vec*>(vbase + i * kIterStride);
    if constexpr (FP4) sc16 = *reinterpret_cast<const uint4*>(v_sf + row0 * (kDim / 16) + lane * 16);

    float mx = -INFINITY;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) mx = fmaxf(mx, z[it]);
    m_w = wave_max_xor(mx, Geo::kLanesPerToken);
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const float p = exp2_nonpos(z[it] - m_w);
      l_lane += p;
      if (owner) lds_p[wave][slot + it * Geo::kTokensPerIter][hh] = p;
    }
    if constexpr (FP4) *reinterpret_cast<uint4*>(&lds_sc[wave][lane * 16]) = sc16;
    wave_sync();

    // ---- PV
    float acc[kAttnHeads][DPL];
#pragma unroll
    for (int h = 0; h < kAttnHeads; ++h)
#pragma unroll
      for (int d = 0; d < DPL; ++d) acc[h][d] = 0.f;
#pragma unroll
    for (int c0 = 0; c0 < ITERS; c0 += CHUNK) {
      if (c0 > 0) {
#pragma unroll
        for (int i = 0; i < CHUNK; ++i) vb[i] = *reinterpret_cast<const Vec*>(vbase + (c0 + i) * kIterStride);
      }
#pragma unroll
      for (int i = 0; i < CHUNK; ++i) {
        const int it = c0 + i;
        const int tok = slot + it * Geo::kTokensPerIter;
        const float2 p2 = *reinterpret_cast<const float2*>(&lds_p[wave][tok][0]);
        float vv[DPL];
        float ph[kAttnHeads] = {p2.x, p2.y};
        if constexpr (FP4) {
          const uint32_t ws[2] = {vb[i].x, vb[i].y};
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
          const float vs = e4m3_to_f32(lds_sc[wave][it * kWave + lane]);
          ph[0] *= vs;
          ph[1] *= vs;
        } else {
          const uint32_t ws[4] = {vb[i].x, vb[i].y, vb[i].z, vb[i].w};
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            vv[2 * d] = bf16lo_to_f32(ws[d]);
            vv[2 * d + 1] = bf16hi_to_f32(ws[d]);
          }
        }
#pragma unroll
        for (int h = 0; h < kAttnHeads; ++h)
#pragma unroll
          for (int d = 0; d < DPL; ++d) acc[h][d] = fmaf(ph[h], vv[d], acc[h][d]);
      }
    }

    // ---- token slots -> 4 slot groups (FP4: pair slots s and s^1 with one DPP add)
    if constexpr (FP4) {
#pragma unroll
      for (int h = 0; h < kAttnHeads; ++h)
#pragma unroll
        for (int d = 0; d < DPL; ++d) acc[h][d] += dpp<kDppRowRor8>(acc[h][d]);
    }
    const bool writer = FP4 ? (lane & 8) == 0 : true;
    const int sg = lane >> 4;   // slot group 0..3
    if (writer) {
#pragma unroll
      for (int h = 0; h < kAttnHeads; ++h)
#pragma unroll
        for (int d = 0; d < DPL; d += 4)
          *reinterpret_cast<float4*>(&U.merge.o[wave][sg][h][chunk * DPL + d]) =
              make_float4(acc[h][d], acc[h][d + 1], acc[h][d + 2], acc[h][d + 3]);
    }
    for (int off = Geo::kLanesPerToken; off < kWave; off <<= 1) l_lane += __shfl_xor(l_lane, off);
  }
  if (lane < kAttnHeads) {  // owner lanes of slot 0: one per head
    lds_ml[wave][hh][0] = m_w;
    lds_ml[wave][hh][1] = l_lane;
  }
  __syncthreads();

  // ---- merge the waves and slot groups: thread -> (head, dim)
  if (tid < kAttnHeads * kDim) {
    const int h = tid / kDim;
    const int d = tid % kDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, lds_ml[w][h][0]);
    float o = 0.f, l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        const float mw = lds_ml[w][h][0];
        if (mw == -INFINITY) continue;
        const float f = exp2_nonpos(mw - M);
        float s = 0.f;
#pragma unroll
        for (int sgi = 0; sgi < kAttnSlotGroups; ++sgi) s += U.merge.o[w][sgi][h][d];
        o = fmaf(f, s, o);
        l = fmaf(f, lds_ml[w][h][1], l);
      }
    }
    out_row[h * kDim + d] = l > 0.f ? o * (v_scale / l) : 0.f;
  }
}

}  // namespace msa
