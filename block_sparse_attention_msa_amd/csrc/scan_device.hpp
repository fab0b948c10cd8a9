// scan_device.hpp - one wave of the decode index scan fused with the block
// max-pool (method: "MSA basics", vLLM MiniMax-M3.1-Flash post: every visible
// token scored against one index query per GQA group with a single shared
// index-key head, max-pooled to one score per 128-token block).
//
// gfx950 design (HBM-bound, VALU work kept well under the byte budget):
//  * one wave walks whole 128-token pages; every global load is a contiguous
//    1 KB wave-load (16 B per lane), 8 tokens x 128 FP8 bytes, all 16 loads of
//    a page issued before use, nontemporal (streamed once);
//  * lane = (token slot, 16-byte dim chunk); each lane holds its 16-dim slice
//    of all four index queries in 32 VGPRs (bf16 pairs), loaded once;
//  * FP8 -> bf16 with v_cvt_scalef32_pk_bf16_fp8 (2 values / instruction,
//    exact), products on v_dot2c_f32_bf16 (exact products, fp32 sums);
//  * the 8-lane token reduction for 4 groups costs 4 DPP adds: each lane keeps
//    its four group partials in a lane-dependent order so that after two
//    butterfly steps each lane owns one group;
//  * the block max is a running per-lane max plus 3 cross-slot steps, written
//    once per block and group.  Token scores never reach memory.
#pragma once

#include "msa_device.hpp"

namespace msa {

template <bool FP8>
struct ScanGeom {
  static constexpr int kLanesPerToken = FP8 ? 8 : 16;    // 128 dims x (1 or 2) B / 16 B
  static constexpr int kLog2Lpt = FP8 ? 3 : 4;
  static constexpr int kTokensPerLoad = kWave / kLanesPerToken;
  static constexpr int kLoadsPerBlock = kBlock / kTokensPerLoad;  // 16 or 32
  static constexpr int kPairsPerLane = FP8 ? 8 : 4;                // bf16 pairs per 16 B
  static constexpr size_t kPageBytes = (size_t)kBlock * kDim * (FP8 ? 1 : 2);
};

// Block scores of blocks [jbeg, jend) of one sequence (one query row):
//   bs_row[g * mbps + j] = idx_scale * max over visible tokens of block j of
//   sum_d iq_row[g][d] * ik[t][d]   (-inf for blocks past the last token).
// CHUNK: page loads issued together per wave (16: the whole FP8 page).
template <bool FP8, int CHUNK = 16>
__device__ __forceinline__ void scan_wave(const uint8_t* __restrict__ idx_pool, const int32_t* __restrict__ bt_row,
                                          int L, const uint16_t* __restrict__ iq_row, float* __restrict__ bs_row,
                                          int mbps, int jbeg, int jend, float idx_scale, int lane) {
  using Geo = ScanGeom<FP8>;
  const int nbv = L > 0 ? ((L - 1) / kBlock) + 1 : 0;
  const int my_group = lane_group(lane);

  // This lane's slice of the four index queries, group order permuted by lane.
  const int chunk = lane & (Geo::kLanesPerToken - 1);
  const int slot = lane / Geo::kLanesPerToken;
  uint32_t qr[4][Geo::kPairsPerLane];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t* src =
        reinterpret_cast<const uint32_t*>(iq_row + permuted_group(lane, k) * kDim + chunk * (2 * Geo::kPairsPerLane));
#pragma unroll
    for (int p = 0; p < Geo::kPairsPerLane; ++p) qr[k][p] = src[p];
  }

  for (int j = jbeg; j < jend; ++j) {
    if (j >= nbv) {
      if (lane < 4) bs_row[my_group * mbps + j] = -INFINITY;
      continue;
    }
    const int64_t page = bt_row[j];
    const uint8_t* base = idx_pool + page * Geo::kPageBytes + lane * 16;
    const int visible = L - j * kBlock;  // tokens of this block at or before the query
    float m = -INFINITY;
#pragma unroll
    for (int i0 = 0; i0 < Geo::kLoadsPerBlock; i0 += CHUNK) {
      u32x4 buf[CHUNK];
#pragma unroll
      for (int i = 0; i < CHUNK; ++i)
        buf[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + (size_t)(i0 + i) * 1024));
#pragma unroll
      for (int i = 0; i < CHUNK; ++i) {
        const uint32_t w[4] = {buf[i].x, buf[i].y, buf[i].z, buf[i].w};
        float a[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (FP8) {
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const bf16x2 lo = e4m3x2_to_bf16x2<false>(w[d]);
            const bf16x2 hi = e4m3x2_to_bf16x2<true>(w[d]);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              a[k] = dot2(lo, as_bf16x2(qr[k][2 * d]), a[k]);
              a[k] = dot2(hi, as_bf16x2(qr[k][2 * d + 1]), a[k]);
            }
          }
        } else {
#pragma unroll
          for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int k = 0; k < 4; ++k) a[k] = dot2(as_bf16x2(w[d]), as_bf16x2(qr[k][d]), a[k]);
        }
        const float s = reduce4_permuted<Geo::kLog2Lpt>(a[0], a[1], a[2], a[3]);
        const int tok = slot + (i0 + i) * Geo::kTokensPerLoad;
        m = fmaxf(m, tok < visible ? s : -INFINITY);
      }
    }
    m = wave_max_xor(m, Geo::kLanesPerToken);
    if (lane < 4) bs_row[my_group * mbps + j] = m * idx_scale;
  }
}

}  // namespace msa
