// attn_device.hpp - one workgroup of the exact GQA attention over the kept
// blocks of one (query row, group), all four query heads of the group,
// optionally preceded by the exact block selection of that (row, group).
//
// Method ("MSA basics", vLLM MiniMax-M3.1-Flash post: the main attention runs
// exactly, but only over the kept blocks, and every query head of a GQA group
// attends over its group's blocks; "Prefill execution" step 4 and "Decode
// sparse GQA" of the MiniMax M3 x vLLM post: the result equals dense attention
// restricted to the selected set, computed with an online softmax over split
// work whose partial outputs are merged).
//
// One workgroup per (row, group): 16 waves with one kept block each, or 8
// waves with two (online softmax across the pair); the waves' partial
// (o, m, l) are merged by log-sum-exp in LDS, so each head's softmax completes
// inside the workgroup and the output is written directly.  K/V are read only for the kept blocks,
// straight from the paged pool, and dequantised once for all four heads.
//
// gfx950 design, per wave and 128-token block (NVFP4 K/V):
//  * QK on v_mfma_f32_16x16x32_bf16, 16 tokens per tile: A = K codes
//    (E2M1 -> bf16 exact, one 16-byte load = 32 dims per lane), B = the bf16
//    queries placed so that MFMA column (j, h) only sums the dims of scale
//    group 2j (K steps 0-1) or 2j+1 (K steps 2-3) for head h.  The E4M3 group
//    scales are then applied once per 16-dim partial dot (fp32), and the four
//    group slots summed with two DPP adds: every product stays exact and the
//    MFMA runs with all 16 columns in use.
//  * softmax in registers (the block max per head is exact, so one block per
//    wave needs no rescaling); p is stored to LDS as f16 (for bf16 K/V as a
//    bf16 hi + lo pair, two MFMAs: a single bf16 p would carry 2^-9 relative
//    error into outputs that cancel);
//  * PV on v_mfma_f32_16x16x32_f16: A = p (rows = the 4 heads), B = V with
//    the tokens on the contraction axis.  NVFP4 V is stored by dim (row d of
//    the page's head slab: dim d of its 128 tokens, token 2i in the low nibble
//    of byte i), so one 4-byte load gives a lane 8 consecutive tokens of one
//    dim; each byte converts to a token pair (E2M1 -> f16 exact) and takes both
//    tokens' E4M3 scales with one packed f16 multiply (code x scale has <= 6
//    significant bits: exact in f16).  K's and V's tensor scales and sm_scale
//    are applied in fp32 outside the MFMAs.
#pragma once

#include "msa_device.hpp"
#include "select_device.hpp"

namespace msa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kQkTiles = kBlock / 16;   // 16-token MFMA tiles per block
constexpr int kPRow = kBlock + 16;      // LDS row of softmax weights (halves), padded
constexpr int kPvSteps = kBlock / 32;   // 32-token MFMA contraction steps per block

// Workgroup shapes: NT = 1024 (16 waves, one kept block each) or NT = 512
// (8 waves, two kept blocks each, online softmax across the pair; rows of at
// most 8,192 blocks).  The 512-thread form needs about half the LDS, so two
// workgroups share a CU and hide each other's load and selection latency.
// With the kept blocks split over SPLIT workgroups, each takes 16 / SPLIT
// slots, one per wave, or, with the tokens of each block split over TS waves
// (bf16 K/V), one per TS waves (NT = 1024 / SPLIT x TS).
template <int NT, int SPLIT = 1, int TS = 1>
struct AttnShape {
  static constexpr int kWaves = NT / kWave;
  static constexpr int kSlots = kTopK / SPLIT;  // kept-block slots of one workgroup
  static constexpr int kBlocksPerWave = kSlots * TS / kWaves;
  static_assert(kWaves * kBlocksPerWave * SPLIT == kTopK * TS, "kept blocks split evenly over the waves");
};

template <int NT>
struct MergeSmem {
  float o[NT / kWave][kHeadsPerGroup][kDim];
  float m[NT / kWave][kHeadsPerGroup];
  float l[NT / kWave][kHeadsPerGroup];
  float f[NT / kWave][kHeadsPerGroup];  // exp2(m_w - M_h): the wave's rescale factor per head
  float inv[kHeadsPerGroup];             // v_scale / sum_w f l_w per head (0 without keys)
};

template <int NT>
struct AttnSmem {
  static constexpr int kWaves = NT / kWave;
  union {
    SelectSmem<NT> sel;
    MergeSmem<NT> merge;
  } u;
  // softmax weights per wave: f16 (or the bf16 hi part) and the bf16 lo part
  // (bf16 K/V only).  Rows padded to 288 B: the 4 head rows' token writes fall
  // on distinct banks and the PV reads of the 4 heads on distinct 16-B slots.
  uint16_t p[kWaves][kHeadsPerGroup][kPRow];
  uint16_t plo[kWaves][kHeadsPerGroup][kPRow];
  uint8_t ksc[kWaves][kBlock * 8];               // 1 KB per wave: K scales [token][group]
  uint8_t vsc[kWaves][kBlock * 8];               // 1 KB per wave: V scales [token pair][group][2]
  int32_t sel[kTopK];
  int32_t page[kTopK];  // page ids of the kept blocks (fused selection)
};

// 16-dim group scales of 2 tokens (16 bytes: token a's 8, then token b's) ->
// [group][a, b] byte pairs, tokens past the visible end zeroed (so their V
// rows, whatever the bytes, contribute 0 x finite).
__device__ __forceinline__ uint4 pair_scales(uint4 w, bool a_vis, bool b_vis) {
  const uint32_t a0 = a_vis ? w.x : 0u, a1 = a_vis ? w.y : 0u;
  const uint32_t b0 = b_vis ? w.z : 0u, b1 = b_vis ? w.w : 0u;
  uint4 r;
  r.x = __builtin_amdgcn_perm(b0, a0, 0x05010400u);  // groups 0, 1
  r.y = __builtin_amdgcn_perm(b0, a0, 0x07030602u);  // groups 2, 3
  r.z = __builtin_amdgcn_perm(b1, a1, 0x05010400u);  // groups 4, 5
  r.w = __builtin_amdgcn_perm(b1, a1, 0x07030602u);  // groups 6, 7
  return r;
}

// The two E2M1 nibbles of byte k of w -> two f16 (exact), k a constant after unrolling.
__device__ __forceinline__ f16x2 e2m1x2_to_f16x2(uint32_t w, int k) {
  switch (k) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  }
}

template <bool FP4>
struct PvType;
template <>
struct PvType<true> {  // NVFP4 V: exact in f16
  using Vec8 = f16x8;
  static __device__ __forceinline__ uint16_t pack(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
  static __device__ __forceinline__ float unpack(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
  static __device__ __forceinline__ f32x4 mfma(Vec8 a, Vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <>
struct PvType<false> {  // bf16 V
  using Vec8 = bf16x8;
  static __device__ __forceinline__ uint16_t pack(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
  static __device__ __forceinline__ float unpack(uint16_t h) { return __builtin_bit_cast(float, (uint32_t)h << 16); }
  static __device__ __forceinline__ f32x4 mfma(Vec8 a, Vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

// Stores of a split part's partial: device-coherent when another workgroup
// of the same launch merges them (agent-scope relaxed atomic stores, which
// write through to the device's coherence point), plain otherwise.
template <bool COHERENT>
__device__ __forceinline__ void store_f32x2(float* p, float a, float b) {
  if constexpr (COHERENT) {
    const uint64_t u = (uint64_t)__builtin_bit_cast(uint32_t, a) | ((uint64_t)__builtin_bit_cast(uint32_t, b) << 32);
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p), u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    *reinterpret_cast<float2*>(p) = make_float2(a, b);
  }
}
template <bool COHERENT>
__device__ __forceinline__ void store_f32(float* p, float a) {
  if constexpr (COHERENT)
    __hip_atomic_store(p, a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = a;
}

// Selection (SELECT: from the block scores) and attention of (row, g) for
// output dims [part * 128 / DSPLIT, (part + 1) * 128 / DSPLIT).  The DSPLIT
// workgroups of one (row, g) repeat the selection and the softmax (identical,
// deterministic) and split the PV work; part 0 writes the selected ids.
// With SPLIT > 1 (DSPLIT = 1) the workgroups instead split the kept blocks:
// part p takes slots [16 p / SPLIT, 16 (p + 1) / SPLIT) and writes, instead of
// the output, its partial per head: po[pair][p][h][128] = sum over its keys of
// 2^(z - M) v (K/V tensor scales aside) and pml[pair][p][h] = (M, sum 2^(z - M)),
// M its largest logit (-inf, with zeros, for a part without keys); a merge
// launch, or the last part to finish, combines the parts (COHERENT: the
// partials are stored device-coherent for the latter).  Padded rows write
// nothing but -1 ids.
// TS > 1 (bf16 K/V, kept blocks split): each block's tokens are split over TS
// waves, wave q of a block taking tokens [q 128 / TS, (q + 1) 128 / TS) (its
// QK tiles and its PV steps); the waves' partials merge like those of
// different blocks.
// With SELECT, mbps must not exceed sel_max_blocks<NT>().  Every thread of the
// workgroup must call it.
template <bool FP4, bool SELECT, int DSPLIT, int NT, int SPLIT = 1, bool COHERENT = false, int TS = 1>
__device__ __forceinline__ void attn_workgroup(
    const uint8_t* __restrict__ kpool, const uint8_t* __restrict__ vpool, const uint8_t* __restrict__ k_sf,
    const uint8_t* __restrict__ v_sf, const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    const uint16_t* __restrict__ q, const float* __restrict__ block_scores, const int32_t* __restrict__ sel_in,
    int32_t* __restrict__ sel_out, float* __restrict__ out, int q_len, int mbps, float qk_scale_log2, float v_scale,
    int row, int g, int part, AttnSmem<NT>& sm, float* __restrict__ po = nullptr, float2* __restrict__ pml = nullptr) {
  static_assert(DSPLIT == 1 || DSPLIT == 2 || DSPLIT == 4, "output split");
  static_assert(SPLIT == 1 || DSPLIT == 1, "split either the output dims or the kept blocks");
  static_assert(TS == 1 || (!FP4 && SPLIT > 1 && kPvSteps % TS == 0), "token split: bf16 K/V, kept blocks split");
  constexpr int kWaves = AttnShape<NT, SPLIT, TS>::kWaves;
  constexpr int kBpw = AttnShape<NT, SPLIT, TS>::kBlocksPerWave;
  constexpr int kSlot0Step = AttnShape<NT, SPLIT, TS>::kSlots;  // first slot of part p: p * kSlots
  constexpr int kTilesPerWave = kQkTiles / TS;  // QK tiles of one wave per block
  constexpr int kStepsPerWave = kPvSteps / TS;  // PV steps of one wave per block
  // With the kept blocks split (one block per wave, at most 2 waves per SIMD)
  // the V loads go out with the K loads: registers are plentiful and the
  // wave's chain of round trips is what takes the time.
  constexpr bool kVEarly = SPLIT > 1;
  using PV = PvType<FP4>;
  constexpr int kRowBytes = FP4 ? kDim / 2 : kDim * 2;  // bytes per (token, head) row
  constexpr int kDims = kDim / DSPLIT;                  // output dims of this workgroup
  constexpr int kTiles = kDims / 16;                    // 16-column PV output tiles (8, 4, 2)
  constexpr int kLaneDims = kTiles;                     // consecutive dims per lane (one scale group)
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int b = row / q_len;
  const int L = seq_lens[b];
  [[maybe_unused]] SelLoads ld;  // the selection's loads, issued before the row length arrives
  if constexpr (SELECT)
    select_load<NT, true>(block_scores + ((size_t)row * kGroups + g) * mbps, block_table + (size_t)b * mbps, mbps, ld);
  const int head0 = g * kHeadsPerGroup;
  const int dbase = SPLIT > 1 ? 0 : part * kDims;
  float* out_row = out + ((size_t)row * (kGroups * kHeadsPerGroup) + head0) * kDim;
  int32_t* sel_row = (sel_out && part == 0) ? sel_out + ((size_t)row * kGroups + g) * kTopK : nullptr;

  if (L <= 0) {  // padded row
    if (SPLIT == 1)
      for (int i = tid; i < kHeadsPerGroup * kDims; i += NT) out_row[(i / kDims) * kDim + dbase + i % kDims] = 0.f;
    if (SELECT && sel_row && tid < kTopK) sel_row[tid] = -1;
    return;
  }
  const int pos = L - q_len + row % q_len;
  if constexpr (SELECT) {
    const int r = min(pos / kBlock, mbps - 1);
    select_blocks<NT, true>(ld, block_table + (size_t)b * mbps, r, mbps, sm.u.sel, sm.sel, sm.page);
    if (sel_row && tid < kTopK) sel_row[tid] = sm.sel[tid];
  } else {
    if (tid < kTopK) sm.sel[tid] = sel_in[((size_t)row * kGroups + g) * kTopK + tid];
    __syncthreads();
  }

  // MFMA lane roles: quarter c = lane / 16, column n = lane % 16.  QK column
  // n = (head hq, group slot jj); the 4 slots of a head sit in one DPP quad.
  const int c = lane >> 4;
  const int n = lane & 15;
  const int hq = n >> 2;
  const int jj = n & 3;
  const int d0 = dbase + kLaneDims * n;  // PV: this lane's first output dim

  float m_w = -INFINITY, l_w = 0.f;  // head hq
  f32x4 acc[kTiles];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // B operands: column (hq, jj) takes head hq's dims 32c + 8s + e when jj == c
  bf16x8 qb[4];
  {
    const uint16_t* qh = q + ((size_t)row * (kGroups * kHeadsPerGroup) + head0 + hq) * kDim + 32 * c;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 w = jj == c ? *reinterpret_cast<const uint4*>(qh + 8 * s) : make_uint4(0, 0, 0, 0);
      qb[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const int tq = wave % TS;  // this wave's token part of its blocks
  for (int kb = 0; kb < kBpw; ++kb) {
    const int slot = (SPLIT > 1 ? part * kSlot0Step : 0) + wave / TS + (kWaves / TS) * kb;
    const int j = sm.sel[slot];
    // ids outside the row's visible blocks or the table contribute nothing
    if (j < 0 || j >= mbps || j * kBlock > pos) continue;  // wave-uniform
    const int64_t page = SELECT ? sm.page[slot] : block_table[(size_t)b * mbps + j];
    const int64_t row0 = (page * kGroups + g) * kBlock;  // first (token, head) row of this page/head
    const int nvis = min(pos - j * kBlock + 1, kBlock);   // keys: tokens 0..nvis-1 (>= 1)
    if (tq * (kBlock / TS) >= nvis) continue;  // wave-uniform: no key in this wave's tokens
    const uint8_t* kbase = kpool + row0 * kRowBytes;
    const uint8_t* vbase = vpool + row0 * kRowBytes;

    [[maybe_unused]] uint32_t vw[kPvSteps][8];
    [[maybe_unused]] uint4 vq[FP4 ? kLaneDims : 1];  // NVFP4 V: dim d0 + t, tokens 32c .. 32c + 31
    [[maybe_unused]] uint4 vb[FP4 ? 1 : 8];
    [[maybe_unused]] uint4 vbe[(!FP4 && kVEarly) ? kStepsPerWave : 1][8];  // bf16 V, loaded early
    auto load_v = [&]() {
      if constexpr (!FP4 && kVEarly) {
#pragma unroll
        for (int u = 0; u < kStepsPerWave; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            vbe[u][e] = *reinterpret_cast<const uint4*>(
                vbase + (size_t)(32 * (tq * kStepsPerWave + u) + 8 * c + e) * kRowBytes + 2 * d0);
      } else if constexpr (!FP4 && kLaneDims == 2) {  // bf16 V, 2 dims per lane: all 4 steps' words fit 32 VGPRs
#pragma unroll
        for (int s = 0; s < kPvSteps; ++s)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            vw[s][e] = *reinterpret_cast<const uint32_t*>(vbase + (size_t)(32 * s + 8 * c + e) * kRowBytes + 2 * d0);
      }
      if constexpr (FP4) {
        // V by dim: row d0 + t holds dim d0 + t of the 128 tokens; this lane's
        // tokens 32c .. 32c + 31 (all four PV steps) are its 16 bytes at 16c
#pragma unroll
        for (int t = 0; t < kLaneDims; ++t)
          vq[t] = *reinterpret_cast<const uint4*>(vbase + (size_t)(d0 + t) * (kBlock / 2) + 16 * c);
      }
    };

    // ---- issue the K loads (NVFP4: the whole block, 16 B per lane and tile)
    [[maybe_unused]] uint4 kv[kQkTiles];
    if constexpr (FP4) {
#pragma unroll
      for (int T = 0; T < kQkTiles; ++T)
        kv[T] = *reinterpret_cast<const uint4*>(kbase + (size_t)(16 * T + n) * kRowBytes + 16 * c);
    }
    uint4 ks16 = make_uint4(0, 0, 0, 0), vs16 = make_uint4(0, 0, 0, 0);
    if constexpr (FP4) {
      ks16 = *reinterpret_cast<const uint4*>(k_sf + row0 * 8 + lane * 16);
      vs16 = *reinterpret_cast<const uint4*>(v_sf + row0 * 8 + lane * 16);
    }
    if constexpr (kVEarly) load_v();
    if constexpr (FP4) {
      *reinterpret_cast<uint4*>(&sm.ksc[wave][lane * 16]) = ks16;
      *reinterpret_cast<uint4*>(&sm.vsc[wave][lane * 16]) = pair_scales(vs16, 2 * lane < nvis, 2 * lane + 1 < nvis);
      wave_sync_lds();
    }

    // ---- QK: z[t] = logit (log2 domain) of token 16T + 4c + jj, head hq, T = tq kTilesPerWave + t
    float z[kTilesPerWave];
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
      const int T = tq * kTilesPerWave + t;
      f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
      if constexpr (FP4) {
        const uint32_t w[4] = {kv[T].x, kv[T].y, kv[T].z, kv[T].w};
        bf16x8 ka[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x2 e0 = e2m1x2_to_bf16x2<0>(w[s]);
          const bf16x2 e1 = e2m1x2_to_bf16x2<1>(w[s]);
          const bf16x2 e2 = e2m1x2_to_bf16x2<2>(w[s]);
          const bf16x2 e3 = e2m1x2_to_bf16x2<3>(w[s]);
          ka[s] = bf16x8{e0.x, e0.y, e1.x, e1.y, e2.x, e2.y, e3.x, e3.y};
        }
        a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[0], qb[0], a0, 0, 0, 0);
        a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[1], qb[1], a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[2], qb[2], a1, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[3], qb[3], a1, 0, 0, 0);
      } else {
        const uint8_t* kr = kbase + (size_t)(16 * T + n) * kRowBytes + 64 * c;
        uint4 w[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) w[s] = *reinterpret_cast<const uint4*>(kr + 16 * s);
        a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w[0]), qb[0], a0, 0, 0, 0);
        a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w[1]), qb[1], a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w[2]), qb[2], a1, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w[3]), qb[3], a1, 0, 0, 0);
      }
      // slot jj's partial of token 16T + 4c + i: groups 2jj (a0) and 2jj+1 (a1)
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (FP4) {
          const int tok = 16 * T + 4 * c + i;
          const uint32_t sw = *reinterpret_cast<const uint16_t*>(&sm.ksc[wave][tok * 8 + 2 * jj]);
          const f32x2 sc = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sw, 1.0f, false);
          v[i] = fmaf(sc.x, a0[i], sc.y * a1[i]);
        } else {
          v[i] = a0[i] + a1[i];
        }
      }
      // reduce-scatter over the quad: lane jj ends with the full dot of token i = jj
      const bool b1 = (jj & 2) != 0, b0 = (jj & 1) != 0;
      float y0 = b1 ? v[2] : v[0], y1 = b1 ? v[3] : v[1];
      const float x0 = b1 ? v[0] : v[2], x1 = b1 ? v[1] : v[3];
      y0 += dpp<kDppXor2>(x0);
      y1 += dpp<kDppXor2>(x1);
      const float keep = b0 ? y1 : y0, send = b0 ? y0 : y1;
      const float dot = keep + dpp<kDppXor1>(send);
      z[t] = 16 * T + 4 * c + jj < nvis ? dot * qk_scale_log2 : -INFINITY;
    }

    // ---- issue the V loads (here, or with the K loads): lane (c, n) takes
    //      dims d0 .. d0 + kLaneDims - 1 of tokens 32s + 8c + e
    if constexpr (!kVEarly) load_v();

    // ---- softmax over the block; with two blocks per wave, online across them
    float mx = z[0];
#pragma unroll
    for (int t = 1; t < kTilesPerWave; ++t) mx = fmaxf(mx, z[t]);
    mx = fmaxf(mx, dpp<kDppXor1>(mx));
    mx = fmaxf(mx, dpp<kDppXor2>(mx));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    mx = fmaxf(mx, m_w);  // >= one visible token, so finite
    if constexpr (kBpw > 1) {
      const float alpha = exp2_nonpos(m_w - mx);  // 0 on the wave's first block
      l_w *= alpha;
      // acc row i is head i; lane 4i holds head i's factor
#pragma unroll
      for (int i = 0; i < kHeadsPerGroup; ++i) {
        const float ai = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), 4 * i));
#pragma unroll
        for (int t = 0; t < kTiles; ++t) acc[t][i] *= ai;
      }
    }
    m_w = mx;
    float ls = 0.f;
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
      const int T = tq * kTilesPerWave + t;
      const float p = exp2_nonpos(z[t] - mx);
      ls += p;
      const uint16_t ph = PV::pack(p);
      sm.p[wave][hq][16 * T + 4 * c + jj] = ph;
      if constexpr (!FP4) sm.plo[wave][hq][16 * T + 4 * c + jj] = PV::pack(p - PV::unpack(ph));
    }
    ls += dpp<kDppXor1>(ls);
    ls += dpp<kDppXor2>(ls);
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    l_w += ls;
    wave_sync_lds();

    // ---- PV
#pragma unroll
    for (int u = 0; u < kStepsPerWave; ++u) {
      const int s = tq * kStepsPerWave + u;
      // A: p of head n (rows 4..15 zero); the contraction's K index 8c + e is
      // token 32c + 8s + e with NVFP4 V (a lane's V bytes of one dim are then
      // one 16-B run), token 32s + 8c + e with bf16 V
      const int tok0 = FP4 ? 32 * c + 8 * s : 32 * s + 8 * c;
      [[maybe_unused]] typename PV::Vec8 pa, pl;
      {
        const bool head = n < kHeadsPerGroup;
        const uint4 w = head ? *reinterpret_cast<const uint4*>(&sm.p[wave][n][tok0]) : make_uint4(0, 0, 0, 0);
        pa = __builtin_bit_cast(typename PV::Vec8, w);
        if constexpr (!FP4) {
          const uint4 wl = head ? *reinterpret_cast<const uint4*>(&sm.plo[wave][n][tok0]) : make_uint4(0, 0, 0, 0);
          pl = __builtin_bit_cast(typename PV::Vec8, wl);
        }
      }
      if constexpr (FP4) {
        // the E4M3 scales of token pairs tok0 + 2p, + 1 of this lane's group
        f16x2 sc[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int pair = (tok0 >> 1) + p;
          const uint32_t sw = *reinterpret_cast<const uint16_t*>(&sm.vsc[wave][pair * 16 + 2 * (d0 >> 4)]);
          sc[p] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false);
        }
        // output tile t holds dim d0 + t; word s of its run = tokens tok0 .. + 7,
        // byte p = tokens tok0 + 2p, + 1
#pragma unroll
        for (int t = 0; t < kLaneDims; ++t) {
          const uint32_t w = s == 0 ? vq[t].x : s == 1 ? vq[t].y : s == 2 ? vq[t].z : vq[t].w;
          f16x2 bt[4];
#pragma unroll
          for (int p = 0; p < 4; ++p) bt[p] = e2m1x2_to_f16x2(w, p) * sc[p];
          const f16x8 b = {bt[0].x, bt[0].y, bt[1].x, bt[1].y, bt[2].x, bt[2].y, bt[3].x, bt[3].y};
          acc[t] = PV::mfma(pa, b, acc[t]);
        }
      } else {
        // bf16 V: 8 tokens x kLaneDims dims; tokens past the end zeroed
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int tok = 32 * s + 8 * c + e;
          [[maybe_unused]] const uint8_t* src = vbase + (size_t)tok * kRowBytes + 2 * d0;
          if constexpr (kVEarly) {
            vb[e] = vbe[u][e];
          } else if constexpr (kLaneDims == 8) {
            vb[e] = *reinterpret_cast<const uint4*>(src);
          } else if constexpr (kLaneDims == 4) {
            const uint2 t2 = *reinterpret_cast<const uint2*>(src);
            vb[e] = make_uint4(t2.x, t2.y, 0, 0);
          } else {
            vb[e] = make_uint4(vw[s][e], 0, 0, 0);  // issued before the softmax
          }
          if (tok >= nvis) vb[e] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < kLaneDims / 2; ++k) {
          uint32_t bl[4], bh[4];
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint32_t xa[4] = {vb[2 * p].x, vb[2 * p].y, vb[2 * p].z, vb[2 * p].w};
            const uint32_t ya[4] = {vb[2 * p + 1].x, vb[2 * p + 1].y, vb[2 * p + 1].z, vb[2 * p + 1].w};
            bl[p] = __builtin_amdgcn_perm(ya[k], xa[k], 0x05040100u);  // dim d0 + 2k of both tokens
            bh[p] = __builtin_amdgcn_perm(ya[k], xa[k], 0x07060302u);  // dim d0 + 2k + 1
          }
          const uint4 w0 = make_uint4(bl[0], bl[1], bl[2], bl[3]);
          const uint4 w1 = make_uint4(bh[0], bh[1], bh[2], bh[3]);
          acc[2 * k] = PV::mfma(pa, __builtin_bit_cast(bf16x8, w0), acc[2 * k]);
          acc[2 * k] = PV::mfma(pl, __builtin_bit_cast(bf16x8, w0), acc[2 * k]);
          acc[2 * k + 1] = PV::mfma(pa, __builtin_bit_cast(bf16x8, w1), acc[2 * k + 1]);
          acc[2 * k + 1] = PV::mfma(pl, __builtin_bit_cast(bf16x8, w1), acc[2 * k + 1]);
        }
      }
    }
    wave_sync_lds();  // the next block rewrites this wave's LDS
  }
  __syncthreads();  // selection LDS is dead: the merge area reuses it

  // ---- per-wave partials to LDS: lanes 0..15 hold heads 0..3 (acc rows) x dims d0 + t
  if (c == 0) {
#pragma unroll
    for (int i = 0; i < kHeadsPerGroup; ++i) {
      float* dst = &sm.u.merge.o[wave][i][d0];
#pragma unroll
      for (int t = 0; t < kTiles; t += 2) *reinterpret_cast<float2*>(dst + t) = make_float2(acc[t][i], acc[t + 1][i]);
    }
  }
  if (c == 0 && jj == 0) {  // one lane per head hq
    sm.u.merge.m[wave][hq] = m_w;
    sm.u.merge.l[wave][hq] = l_w;
  }
  __syncthreads();

  // ---- merge the waves: first the per (wave, head) factors f = exp2(m_w - M_h)
  //      (0 for a wave without keys) and per head v_scale / sum_w f l_w, by one
  //      wave (lane = 4 w + h); then each thread (head, dim) sums f o_w
  if (wave == 0) {
    const int w = lane >> 2, h = lane & 3;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) M = fmaxf(M, sm.u.merge.m[k][h]);
    const float mw = w < kWaves ? sm.u.merge.m[w][h] : -INFINITY;
    const float f = mw == -INFINITY ? 0.f : exp2_nonpos(mw - M);
    float fl = w < kWaves ? f * sm.u.merge.l[w][h] : 0.f;
    fl += __shfl_xor(fl, 4);
    fl += __shfl_xor(fl, 8);
    fl += __shfl_xor(fl, 16);
    fl += __shfl_xor(fl, 32);
    if (w < kWaves) sm.u.merge.f[w][h] = f;
    if (w == 0) sm.u.merge.inv[h] = SPLIT > 1 ? 1.f : (fl > 0.f ? v_scale / fl : 0.f);
    if (SPLIT > 1 && w == 0) {
      float2* ml_dst = pml + ((size_t)(row * kGroups + g) * SPLIT + part) * kHeadsPerGroup + h;
      store_f32x2<COHERENT>(reinterpret_cast<float*>(ml_dst), M, fl);
    }
  }
  __syncthreads();
  float* dst = SPLIT > 1 ? po + ((size_t)(row * kGroups + g) * SPLIT + part) * kHeadsPerGroup * kDim : out_row;
  for (int i = tid; i < kHeadsPerGroup * kDims; i += NT) {
    const int h = i / kDims;
    const int d = dbase + i % kDims;
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) o = fmaf(sm.u.merge.f[w][h], sm.u.merge.o[w][h][d], o);
    store_f32<COHERENT>(dst + h * kDim + d, o * sm.u.merge.inv[h]);
  }
}

}  // namespace msa
