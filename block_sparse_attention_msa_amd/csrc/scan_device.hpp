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

// Wave-loads [i0, i0 + N) of one page (base: the page plus 16 B per lane): the
// running per-lane maximum m of the scores of their visible tokens (tokens
// before `visible`), each lane for group lane_group(lane) after the permuted
// reduction; the caller reduces over the token slots (wave_max_xor).
template <bool FP8, int N>
__device__ __forceinline__ float scan_loads(const uint8_t* __restrict__ base,
                                            const uint32_t (&qr)[4][ScanGeom<FP8>::kPairsPerLane], int visible,
                                            int i0, int lane, float m) {
  using Geo = ScanGeom<FP8>;
  const int slot = lane / Geo::kLanesPerToken;
  u32x4 buf[N];
#pragma unroll
  for (int i = 0; i < N; ++i)
    buf[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + (size_t)(i0 + i) * 1024));
#pragma unroll
  for (int i = 0; i < N; ++i) {
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
  return m;
}

// This lane's slice of the four index queries of one row, group order
// permuted by lane (lane = (token slot, 16-byte dim chunk)).
template <bool FP8>
__device__ __forceinline__ void scan_query_slice(const uint16_t* __restrict__ iq_row, int lane,
                                                 uint32_t (&qr)[4][ScanGeom<FP8>::kPairsPerLane]) {
  using Geo = ScanGeom<FP8>;
  const int chunk = lane & (Geo::kLanesPerToken - 1);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t* src =
        reinterpret_cast<const uint32_t*>(iq_row + permuted_group(lane, k) * kDim + chunk * (2 * Geo::kPairsPerLane));
#pragma unroll
    for (int p = 0; p < Geo::kPairsPerLane; ++p) qr[k][p] = src[p];
  }
}

// Block scores of blocks [jbeg, jend) of one sequence (one query row):
//   bs_row[g * mbps + j] = idx_scale * max over visible tokens of block j of
//   sum_d iq_row[g][d] * ik[t][d]   (-inf for blocks past the last token).
// CHUNK: page loads issued together per wave (16: the whole FP8 page).
template <bool FP8, int CHUNK = 16>
__device__ __forceinline__ void scan_wave(const uint8_t* __restrict__ idx_pool, const int32_t* __restrict__ bt_row,
                                          int L, const uint16_t* __restrict__ iq_row, float* __restrict__ bs_row,
                                          int mbps, int jbeg, int jend, float idx_scale, int lane) {
  using Geo = ScanGeom<FP8>;
  // block-table entries are read one page ahead of their use, before the
  // visibility test (entries of the row: jbeg < jend <= mbps); an invisible
  // block's entry is never followed
  int32_t pg = bt_row[jbeg];
  const int nbv = L > 0 ? ((L - 1) / kBlock) + 1 : 0;
  const int my_group = lane_group(lane);

  uint32_t qr[4][Geo::kPairsPerLane];
  scan_query_slice<FP8>(iq_row, lane, qr);

  for (int j = jbeg; j < jend; ++j) {
    const int32_t pg_j = pg;
    if (j + 1 < jend) pg = bt_row[j + 1];
    if (j >= nbv) {
      if (lane < 4) bs_row[my_group * mbps + j] = -INFINITY;
      continue;
    }
    const int64_t page = pg_j;
    const uint8_t* base = idx_pool + page * Geo::kPageBytes + lane * 16;
    const int visible = L - j * kBlock;  // tokens of this block at or before the query
    float m = -INFINITY;
#pragma unroll
    for (int i0 = 0; i0 < Geo::kLoadsPerBlock; i0 += CHUNK) m = scan_loads<FP8, CHUNK>(base, qr, visible, i0, lane, m);
    m = wave_max_xor(m, Geo::kLanesPerToken);
    if (lane < 4) bs_row[my_group * mbps + j] = m * idx_scale;
  }
}

}  // namespace msa

namespace msa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// NVFP4 index keys (E2M1 codes [P][128][64] + E4M3 scales [P][128][8]): block
// scores of blocks [jbeg, jend) of one sequence, one wave per block.
//
// With 64 B of codes per token a wave-load holds 16 whole tokens, so the scan
// takes the attention's exact QK tile: v_mfma_f32_16x16x32_bf16 with A = the
// codes of 16 tokens (E2M1 -> bf16, exact, one 16-B load = 32 dims per lane)
// and B = the four index queries, MFMA column (group hq, slot jj) holding
// group hq's dims of scale groups 2jj (K steps 0-1, accumulator a0) and 2jj+1
// (K steps 2-3, a1).  Each 16-dim partial dot is scaled once by its token's
// E4M3 group scale in fp32, and a reduce-scatter over the quad leaves lane
// (c, hq, jj) with the full score of token 16T + 4c + jj for group hq.
// Products are exact in fp32 (E2M1 x bf16 and the scale products), sums fp32.
// VALU per token: 4 conversions, 2 scale products and the reductions, about
// a third of the FP8 scan's per-byte work at 72 B per token.
__device__ __forceinline__ void scan_wave_nvfp4(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                const int32_t* __restrict__ bt_row, int L,
                                                const uint16_t* __restrict__ iq_row, float* __restrict__ bs_row,
                                                int mbps, int jbeg, int jend, float idx_scale, uint8_t* lds_sc,
                                                int lane) {
  const int nbv = L > 0 ? ((L - 1) / kBlock) + 1 : 0;
  const int c = lane >> 4;
  const int n = lane & 15;
  const int hq = n >> 2;   // index query (group) of this MFMA column
  const int jj = n & 3;    // scale-group slot of this column

  // B operands: column (hq, jj) takes group hq's dims 32c + 8s + e when jj == c
  bf16x8 qb[4];
  {
    const uint16_t* qh = iq_row + hq * kDim + 32 * c;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 w = jj == c ? *reinterpret_cast<const uint4*>(qh + 8 * s) : make_uint4(0, 0, 0, 0);
      qb[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // block-table entries are read one page ahead of their use, before the
  // visibility test (entries of the row: jbeg < jend <= mbps); an invisible
  // block's entry is never followed
  int32_t pg = bt_row[jbeg];
  for (int j = jbeg; j < jend; ++j) {
    const int32_t pg_j = pg;
    if (j + 1 < jend) pg = bt_row[j + 1];
    if (j >= nbv) {
      if (lane < 4) bs_row[lane * mbps + j] = -INFINITY;
      continue;
    }
    const int64_t page = pg_j;
    const uint8_t* kbase = codes + page * (kBlock * kDim / 2);
    u32x4 kv[8];
#pragma unroll
    for (int T = 0; T < 8; ++T)
      kv[T] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + (size_t)(16 * T + n) * 64 + 16 * c));
    const u32x4 sc16 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(scales + page * (kBlock * 8) + lane * 16));
    *reinterpret_cast<u32x4*>(lds_sc + lane * 16) = sc16;  // [token][group], this wave's 1 KB
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int visible = L - j * kBlock;  // tokens of this block at or before the query
    float m = -INFINITY;
#pragma unroll
    for (int T = 0; T < 8; ++T) {
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
      f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
      a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[0], qb[0], a0, 0, 0, 0);
      a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[1], qb[1], a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[2], qb[2], a1, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[3], qb[3], a1, 0, 0, 0);
      // slot jj's partial of token 16T + 4c + i: groups 2jj (a0) and 2jj+1 (a1)
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 16 * T + 4 * c + i;
        const uint32_t sw = *reinterpret_cast<const uint16_t*>(lds_sc + tok * 8 + 2 * jj);
        const f32x2 sc = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sw, 1.0f, false);
        v[i] = fmaf(sc.x, a0[i], sc.y * a1[i]);
      }
      // reduce-scatter over the quad: lane jj ends with the full score of token i = jj
      const bool b1 = (jj & 2) != 0, b0 = (jj & 1) != 0;
      float y0 = b1 ? v[2] : v[0], y1 = b1 ? v[3] : v[1];
      const float x0 = b1 ? v[0] : v[2], x1 = b1 ? v[1] : v[3];
      y0 += dpp<kDppXor2>(x0);
      y1 += dpp<kDppXor2>(x1);
      const float keep = b0 ? y1 : y0, send = b0 ? y0 : y1;
      const float dot = keep + dpp<kDppXor1>(send);
      m = fmaxf(m, 16 * T + 4 * c + jj < visible ? dot : -INFINITY);
    }
    // max over the 16 lanes of group hq: c (lane bits 4, 5) and jj (bits 0, 1)
    m = fmaxf(m, dpp<kDppXor1>(m));
    m = fmaxf(m, dpp<kDppXor2>(m));
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    if (c == 0 && jj == 0) bs_row[hq * mbps + j] = m * idx_scale;
    __builtin_amdgcn_wave_barrier();  // the next block rewrites this wave's scales
  }
}

}  // namespace msa

namespace msa {

// FP8 index keys, short multi-query batches: block scores of blocks
// [jbeg, jend) of one sequence for its q_len x 4 (query, group) columns,
// 16 x NT of them at most, one wave per block.
//
// The dense form of the scan, S[t][col] = sum_d ik[t][d] * iq[col][d], on
// v_mfma_f32_16x16x32_bf16: A = 16 tokens (E4M3 -> bf16, exact), B = 16
// columns, column col = 4 i + g of the sequence (query i, group g) exactly as
// the block-score rows are laid out.
//  * The page streams in as 16 contiguous 1 KB wave-loads (lane l: token
//    8i + l/8, 16-B chunk l%8), all issued before use, as in the decode scan.
//  * Per 16-token tile the wave moves its 2 KB through LDS into the MFMA
//    layout: chunk k of tile token t is stored at t*128 + 16 (k ^ (t % 8)), so
//    both the row writes and the column reads touch 8 distinct 16-B slots per
//    8 lanes (conflict-free).  Lane (c, n) = (lane / 16, lane % 16) reads
//    chunks 4h + c of token n (h = 0, 1): MFMA step s = 2h + u takes dims
//    64h + 16c + 8u + e at K index 8c + e, for A and B alike.
//  * The result holds tokens 4c + i of column n: a running max per lane with
//    the causal limit of the lane's column (query i sees tokens at or before
//    position seq_len - q_len + i), then 2 cross-lane steps per block.
// Products are exact in fp32, sums fp32 (the MFMA's accumulation).
//
// Which index query each column holds, where its block scores go and which
// tokens it sees come from a column map:
//   ncols            columns in use
//   pos0             smallest query position over the columns
//   nbv              blocks j >= nbv hold no visible token (scores -inf)
//   iq(col), bs(col) the column's index query and block-score row
//   last_pos(col)    the column's query position (tokens at or before it count)
struct SeqCols {  // one sequence's q_len x 4 (query, group) columns: col = 4 i + g
  const uint16_t* iq_seq;  // [q_len][4][128]
  float* bs_seq;           // [q_len][4][mbps]
  int mbps, ncols, pos0, nbv;
  __device__ const uint16_t* iq(int col) const { return iq_seq + (size_t)col * kDim; }
  __device__ float* bs(int col) const { return bs_seq + (size_t)col * mbps; }
  __device__ int brow(int col) const { return col; }  // the column's block-score row, relative to at()
  __device__ float* at(int brow, int j) const { return bs_seq + (size_t)brow * mbps + j; }
  __device__ int last_pos(int col) const { return pos0 + col / kGroups; }
};
struct ShareCols {  // a sharing group's members x q_len x 4 columns: col = (k q_len + i) 4 + g
  const int32_t* members;  // the group's sequence ids (-1 padded)
  const int32_t* seq_lens;
  const uint16_t* iq_all;  // [num_seqs * q_len][4][128]
  float* bs_all;           // [num_seqs * q_len][4][mbps]
  int mbps, ncols, pos0, nbv, q_len;
  // (query row, group) of column col: member k, query i, group g
  __device__ size_t row(int col) const {
    const int per = kGroups * q_len;
    return (size_t)members[col / per] * per + col % per;
  }
  __device__ const uint16_t* iq(int col) const { return iq_all + row(col) * kDim; }
  __device__ float* bs(int col) const { return bs_all + row(col) * mbps; }
  __device__ int brow(int col) const { return (int)row(col); }
  __device__ float* at(int brow, int j) const { return bs_all + (size_t)brow * mbps + j; }
  __device__ int last_pos(int col) const {
    const int per = kGroups * q_len;
    return seq_lens[members[col / per]] - q_len + (col % per) / kGroups;
  }
};

template <int NT, class Cols>
__device__ __forceinline__ void scan_wave_fp8_mfma(const uint8_t* __restrict__ idx_pool,
                                                   const int32_t* __restrict__ bt_row, const Cols& cm, int jbeg,
                                                   int jend, float idx_scale, uint8_t* lds, int lane) {
  // block-table entries are read one page ahead of their use, before the
  // visibility test (entries of the row: jbeg < jend <= mbps); an invisible
  // block's entry is never followed
  int32_t pg = bt_row[jbeg];
  const int nbv = cm.nbv;
  const int c = lane >> 4;
  const int n = lane & 15;
  const int ncols = cm.ncols;
  const int pos0 = cm.pos0;  // smallest query position of the columns
  // this lane's columns 16t + n: block-score rows and query positions
  int brow[NT];
  int lastp[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int col = 16 * t + n;
    brow[t] = col < ncols ? cm.brow(col) : 0;
    lastp[t] = col < ncols ? cm.last_pos(col) : 0;
  }
  // LDS offsets of this lane's tile writes (token 8hh + lane/8, chunk lane%8)
  // and column reads (token n, chunk 4h + c)
  const int wr = (lane >> 3) * 128 + (((lane & 7) ^ (lane >> 3)) << 4);
  const int rd0 = n * 128 + ((c ^ (n & 7)) << 4);
  const int rd1 = n * 128 + (((4 + c) ^ (n & 7)) << 4);

  // B operands: column 16t + n, dims 64h + 16c + 8u for step s = 2h + u
  bf16x8 qb[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int col = 16 * t + n;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int d = 64 * (s >> 1) + 16 * c + 8 * (s & 1);
      const uint4 w = col < ncols ? *reinterpret_cast<const uint4*>(cm.iq(col) + d) : make_uint4(0, 0, 0, 0);
      qb[t][s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  for (int j = jbeg; j < jend; ++j) {
    const int32_t pg_j = pg;
    if (j + 1 < jend) pg = bt_row[j + 1];
    if (j >= nbv) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
        if (c == 0 && 16 * t + n < ncols) *cm.at(brow[t], j) = -INFINITY;
      continue;
    }
    const int64_t page = pg_j;
    const uint8_t* base = idx_pool + page * (kBlock * kDim) + lane * 16;
    u32x4 kv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) kv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + 1024 * i));
    // every column sees the whole block: no mask (wave-uniform)
    const bool full = (j + 1) * kBlock - 1 <= pos0;
    int vis[NT];  // tokens of the block visible to this lane's column
#pragma unroll
    for (int t = 0; t < NT; ++t) vis[t] = lastp[t] + 1 - j * kBlock;
    float m[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) m[t] = -INFINITY;
#pragma unroll
    for (int T = 0; T < 8; ++T) {
      uint8_t* buf = lds + (T & 1) * 2048;
      *reinterpret_cast<u32x4*>(buf + wr) = kv[2 * T];
      *reinterpret_cast<u32x4*>(buf + 1024 + wr) = kv[2 * T + 1];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const u32x4 r[2] = {*reinterpret_cast<const u32x4*>(buf + rd0), *reinterpret_cast<const u32x4*>(buf + rd1)};
      bf16x8 ka[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t d[4] = {r[h].x, r[h].y, r[h].z, r[h].w};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const bf16x2 p0 = e4m3x2_to_bf16x2<false>(d[2 * u]);
          const bf16x2 p1 = e4m3x2_to_bf16x2<true>(d[2 * u]);
          const bf16x2 p2 = e4m3x2_to_bf16x2<false>(d[2 * u + 1]);
          const bf16x2 p3 = e4m3x2_to_bf16x2<true>(d[2 * u + 1]);
          ka[2 * h + u] = bf16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s], qb[t][s], acc, 0, 0, 0);
        if (full) {
          m[t] = fmaxf(m[t], fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3])));
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) m[t] = fmaxf(m[t], 16 * T + 4 * c + i < vis[t] ? acc[i] : -INFINITY);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float x = fmaxf(m[t], __shfl_xor(m[t], 16));
      x = fmaxf(x, __shfl_xor(x, 32));
      if (c == 0 && 16 * t + n < ncols) *cm.at(brow[t], j) = x * idx_scale;
    }
    __builtin_amdgcn_wave_barrier();  // the next block rewrites this wave's tiles
  }
}

}  // namespace msa

namespace msa {

// NVFP4 index keys, short multi-query batches (2 <= q_len <= 8): block scores
// of blocks [jbeg, jend) of one sequence for its q_len x 4 (query, group)
// columns, 16 x NT of them at most, one wave per block.
//
// The score contraction runs in f16 on v_mfma_f32_16x16x32_f16 (NVFP4 keys
// converted straight to FP16 for the indexer's score MMA: "NVIDIA
// Rubin-optimised MSA" of the vLLM MiniMax-M3.1-Flash post):
//  * keys: an E2M1 code times its 16-dim group's E4M3 scale has at most 6
//    significant bits within [2^-10, 2688], so the f16 key is exact: one
//    conversion and one packed f16 multiply per pair of values;
//  * queries: each column is scaled by a power of two 2^k so that its largest
//    |iq| lies in [2^14, 2^15) and converted to f16 (nearest-even).  Every
//    element within 2^-28 of the column's largest is exact; smaller ones
//    round to f16 subnormals (absolute error at most 2^-25 x 2^-k).  The
//    block maximum is multiplied back by 2^-k (exact);
//  * products are exact in fp32, sums fp32.
// With 64 B of codes per token one 16-B load per lane holds 16 whole tokens,
// so lane (c, n) = (lane / 16, lane % 16) loads token n's dims 32c .. 32c + 31
// (scale groups 2c, 2c + 1) in contiguous 1 KB wave-loads with no transpose;
// MFMA step s takes dims 32c + 8s + e at K index 8c + e, for A and B alike.
// The page's 1 KB of scales arrives with one 16-B load per lane into a
// per-wave LDS copy, from which each lane reads the two bytes of (token,
// 2c .. 2c + 1) per tile.  Columns, causal limits and the max-pool are those
// of the FP8 form.
template <int NT>
__device__ __forceinline__ void scan_wave_nvfp4_cols(const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ scales,
                                                     const int32_t* __restrict__ bt_row, int L, int q_len,
                                                     const uint16_t* __restrict__ iq_seq, float* __restrict__ bs_seq,
                                                     int mbps, int jbeg, int jend, float idx_scale,
                                                     uint8_t* lds_sc, int lane) {
  // block-table entries are read one page ahead of their use, before the
  // visibility test (entries of the row: jbeg < jend <= mbps); an invisible
  // block's entry is never followed
  int32_t pg = bt_row[jbeg];
  const int nbv = L > 0 ? ((L - 1) / kBlock) + 1 : 0;
  const int c = lane >> 4;
  const int n = lane & 15;
  const int ncols = q_len * kGroups;
  const int pos0 = L - q_len;  // position of query 0

  // B operands: column 16t + n, dims 32c + 8s .. + 7 for step s, times 2^k
  f16x8 qh[NT][4];
  float unscale[NT];  // 2^-k of the lane's column, times idx_scale
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int col = 16 * t + n;
    uint32_t w[4][4];
    float mx = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 v = col < ncols ? *reinterpret_cast<const uint4*>(iq_seq + (size_t)col * kDim + 32 * c + 8 * s)
                                  : make_uint4(0, 0, 0, 0);
      w[s][0] = v.x, w[s][1] = v.y, w[s][2] = v.z, w[s][3] = v.w;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        mx = fmaxf(mx, fmaxf(__builtin_fabsf(bf16lo_to_f32(w[s][k])), __builtin_fabsf(bf16hi_to_f32(w[s][k]))));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // mx in [2^(e-1), 2^e): scale by 2^(15 - e), kept within the normal fp32 range
    const int e = mx > 0.f ? __builtin_amdgcn_frexp_expf(mx) : 15;
    const int k = max(-126, min(126, 15 - e));
    const float up = __builtin_ldexpf(1.0f, k);
    unscale[t] = __builtin_ldexpf(1.0f, -k) * idx_scale;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        qh[t][s][2 * q] = (_Float16)(bf16lo_to_f32(w[s][q]) * up);
        qh[t][s][2 * q + 1] = (_Float16)(bf16hi_to_f32(w[s][q]) * up);
      }
  }

  for (int j = jbeg; j < jend; ++j) {
    const int32_t pg_j = pg;
    if (j + 1 < jend) pg = bt_row[j + 1];
    if (j >= nbv) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
        if (c == 0 && 16 * t + n < ncols) bs_seq[(size_t)(16 * t + n) * mbps + j] = -INFINITY;
      continue;
    }
    const int64_t page = pg_j;
    const uint8_t* kbase = codes + page * (kBlock * kDim / 2) + n * (kDim / 2) + 16 * c;
    u32x4 kv[8];
#pragma unroll
    for (int T = 0; T < 8; ++T)
      kv[T] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + (size_t)T * 1024));
    // the page's scales [token][group] (1 KB) through this wave's LDS copy
    const u32x4 sc16 =
        __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(scales + page * (kBlock * 8) + lane * 16));
    *reinterpret_cast<u32x4*>(lds_sc + lane * 16) = sc16;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    uint32_t sw[8];
#pragma unroll
    for (int T = 0; T < 8; ++T) sw[T] = *reinterpret_cast<const uint16_t*>(lds_sc + (16 * T + n) * 8 + 2 * c);
    const bool full = (j + 1) * kBlock - 1 <= pos0;  // wave-uniform: no mask
    int vis[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) vis[t] = pos0 + (16 * t + n) / kGroups + 1 - j * kBlock;
    float m[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) m[t] = -INFINITY;
#pragma unroll
    for (int T = 0; T < 8; ++T) {
      const uint32_t w[4] = {kv[T].x, kv[T].y, kv[T].z, kv[T].w};
      const f16x2 sf = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw[T], 1.0f, false);  // groups 2c, 2c + 1
      const f16x2 g0 = {sf.x, sf.x}, g1 = {sf.y, sf.y};
      f16x8 kh[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const f16x2 g = s < 2 ? g0 : g1;
        const f16x2 e0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[s], 1.0f, 0) * g;
        const f16x2 e1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[s], 1.0f, 1) * g;
        const f16x2 e2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[s], 1.0f, 2) * g;
        const f16x2 e3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[s], 1.0f, 3) * g;
        kh[s] = f16x8{e0.x, e0.y, e1.x, e1.y, e2.x, e2.y, e3.x, e3.y};
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kh[s], qh[t][s], acc, 0, 0, 0);
        if (full) {
          m[t] = fmaxf(m[t], fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3])));
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) m[t] = fmaxf(m[t], 16 * T + 4 * c + i < vis[t] ? acc[i] : -INFINITY);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float x = fmaxf(m[t], __shfl_xor(m[t], 16));
      x = fmaxf(x, __shfl_xor(x, 32));
      if (c == 0 && 16 * t + n < ncols) bs_seq[(size_t)(16 * t + n) * mbps + j] = x * unscale[t];
    }
    __builtin_amdgcn_wave_barrier();  // the next page rewrites this wave's scales
  }
}

}  // namespace msa

namespace msa {

// NVFP4 index keys with the columns of a column map (the members of a
// prefix-sharing group, at most 32 columns): the page's codes arrive as in
// scan_wave_nvfp4_cols, but each code x E4M3 group scale is converted exactly
// to bf16 (E2M1 -> f32, times the scale in f32, -> bf16: at most 6
// significant bits, so every step is exact) and the scores run on bf16 MFMAs
// against the bf16 index queries as they are: exact products, fp32 sums, no
// query rounding.  The conversion (4 VALU operations per 2 values) is paid
// once per page for all the columns.
template <int NT, class Cols>
__device__ __forceinline__ void scan_wave_nvfp4_exact_cols(const uint8_t* __restrict__ codes,
                                                           const uint8_t* __restrict__ scales,
                                                           const int32_t* __restrict__ bt_row, const Cols& cm,
                                                           int jbeg, int jend, float idx_scale, uint8_t* lds_sc,
                                                           int lane) {
  // block-table entries are read one page ahead of their use, before the
  // visibility test (entries of the row: jbeg < jend <= mbps); an invisible
  // block's entry is never followed
  int32_t pg = bt_row[jbeg];
  const int nbv = cm.nbv;
  const int c = lane >> 4;
  const int n = lane & 15;
  const int ncols = cm.ncols;
  const int pos0 = cm.pos0;  // smallest query position of the columns
  int brow[NT];
  int lastp[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int col = 16 * t + n;
    brow[t] = col < ncols ? cm.brow(col) : 0;
    lastp[t] = col < ncols ? cm.last_pos(col) : 0;
  }
  // B operands: column 16t + n, dims 32c + 8s .. + 7 for step s (the A side's
  // K order: dims 32c + 8s + e at K index 8c + e)
  bf16x8 qb[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int col = 16 * t + n;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 w = col < ncols ? *reinterpret_cast<const uint4*>(cm.iq(col) + 32 * c + 8 * s) : make_uint4(0, 0, 0, 0);
      qb[t][s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  for (int j = jbeg; j < jend; ++j) {
    const int32_t pg_j = pg;
    if (j + 1 < jend) pg = bt_row[j + 1];
    if (j >= nbv) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
        if (c == 0 && 16 * t + n < ncols) *cm.at(brow[t], j) = -INFINITY;
      continue;
    }
    const int64_t page = pg_j;
    const uint8_t* kbase = codes + page * (kBlock * kDim / 2) + n * (kDim / 2) + 16 * c;
    u32x4 kv[8];
#pragma unroll
    for (int T = 0; T < 8; ++T)
      kv[T] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + (size_t)T * 1024));
    const u32x4 sc16 =
        __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(scales + page * (kBlock * 8) + lane * 16));
    *reinterpret_cast<u32x4*>(lds_sc + lane * 16) = sc16;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    uint32_t sw[8];
#pragma unroll
    for (int T = 0; T < 8; ++T) sw[T] = *reinterpret_cast<const uint16_t*>(lds_sc + (16 * T + n) * 8 + 2 * c);
    const bool full = (j + 1) * kBlock - 1 <= pos0;  // wave-uniform: no mask
    int vis[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) vis[t] = lastp[t] + 1 - j * kBlock;
    float m[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) m[t] = -INFINITY;
#pragma unroll
    for (int T = 0; T < 8; ++T) {
      const uint32_t w[4] = {kv[T].x, kv[T].y, kv[T].z, kv[T].w};
      const f32x2 sf = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sw[T], 1.0f, false);  // groups 2c, 2c + 1
      bf16x8 ka[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float g = s < 2 ? sf.x : sf.y;
        const f32x2 e0 = e2m1x2_to_f32x2<0>(w[s]), e1 = e2m1x2_to_f32x2<1>(w[s]);
        const f32x2 e2 = e2m1x2_to_f32x2<2>(w[s]), e3 = e2m1x2_to_f32x2<3>(w[s]);
        ka[s] = bf16x8{(__bf16)(e0.x * g), (__bf16)(e0.y * g), (__bf16)(e1.x * g), (__bf16)(e1.y * g),
                       (__bf16)(e2.x * g), (__bf16)(e2.y * g), (__bf16)(e3.x * g), (__bf16)(e3.y * g)};
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s], qb[t][s], acc, 0, 0, 0);
        if (full) {
          m[t] = fmaxf(m[t], fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3])));
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) m[t] = fmaxf(m[t], 16 * T + 4 * c + i < vis[t] ? acc[i] : -INFINITY);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float x = fmaxf(m[t], __shfl_xor(m[t], 16));
      x = fmaxf(x, __shfl_xor(x, 32));
      if (c == 0 && 16 * t + n < ncols) *cm.at(brow[t], j) = x * idx_scale;
    }
    __builtin_amdgcn_wave_barrier();  // the next page rewrites this wave's scales
  }
}

}  // namespace msa

namespace msa {

// Shared-prefix pages with more columns than one wave's registers hold: up to
// 256 (member, query, group) columns of one sharing group (64 decode
// requests, or 64 / q_len requests of q_len query tokens).  The 8 waves of a
// workgroup take the group's pages [jbeg, jend) one at a time:
//  * the page is loaded once (FP8: 32 contiguous bytes per thread; NVFP4: 16 B
//    of codes and the 2 scale bytes of those 32 dims) and converted once,
//    exactly, to bf16 (FP8: E4M3 -> bf16; NVFP4: E2M1 -> f32, times the E4M3
//    group scale, -> bf16, at most 6 significant bits) into a 32 KB LDS copy
//    in the MFMA operand order: 16-B chunk k (dims 8k .. 8k + 7) of token t at
//    t * 256 + 16 (k ^ (t % 16)), so each 8 lanes of a column read touch 8
//    distinct 16-B slots;
//  * wave w scores it against its column tiles w and w + 8 (B operands in
//    registers, loaded once): MFMA step s = 2h + u takes dims 64h + 16c + 8u +
//    e at K index 8c + e, as in the FP8 column scan, so with FP8 keys every
//    column's products and fp32 sums are those of the unshared scan, operation
//    for operation;
//  * the next page's raw bytes are loaded while the current one is scored.
// The page is read from HBM and converted once for all the group's requests,
// whatever their number.
constexpr int kWideWaves = 8;
constexpr int kWideTiles = 2;   // column tiles per wave: 16 x 2 x 8 = 256 columns

template <bool NVFP4>
struct WideRaw {  // one thread's share of a page: 32 dims of one token
  u32x4 a, b;     // FP8: 32 bytes; NVFP4: a = 16 B of codes, b.x = the 2 scale bytes
};

template <bool NVFP4>
__device__ __forceinline__ WideRaw<NVFP4> wide_load(const uint8_t* __restrict__ pool, const uint8_t* __restrict__ scales,
                                                    int64_t page, int tid) {
  WideRaw<NVFP4> r;
  if constexpr (NVFP4) {
    r.a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(pool + page * (kBlock * kDim / 2) + 16 * tid));
    const uint32_t sw = *reinterpret_cast<const uint16_t*>(scales + page * (kBlock * 8) + 2 * tid);
    r.b = u32x4{sw, 0u, 0u, 0u};
  } else {
    const uint8_t* src = pool + page * (kBlock * kDim) + 32 * tid;
    r.a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
    r.b = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + 16));
  }
  return r;
}

// Thread tid holds token tid / 4, dims 32 (tid % 4) .. + 31: converts them to
// bf16 and stores chunks 4 (tid % 4) .. + 3 of that token's LDS row.
template <bool NVFP4>
__device__ __forceinline__ void wide_store(const WideRaw<NVFP4>& r, uint8_t* lds, int tid) {
  const int t = tid >> 2, qd = tid & 3;
  uint32_t w[16];  // 32 bf16
  if constexpr (NVFP4) {
    const f32x2 sf = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.b.x, 1.0f, false);  // groups 2 qd, 2 qd + 1
    const uint32_t c4[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float g = s < 2 ? sf.x : sf.y;
      const f32x2 e0 = e2m1x2_to_f32x2<0>(c4[s]), e1 = e2m1x2_to_f32x2<1>(c4[s]);
      const f32x2 e2 = e2m1x2_to_f32x2<2>(c4[s]), e3 = e2m1x2_to_f32x2<3>(c4[s]);
      const bf16x2 p0 = {(__bf16)(e0.x * g), (__bf16)(e0.y * g)}, p1 = {(__bf16)(e1.x * g), (__bf16)(e1.y * g)};
      const bf16x2 p2 = {(__bf16)(e2.x * g), (__bf16)(e2.y * g)}, p3 = {(__bf16)(e3.x * g), (__bf16)(e3.y * g)};
      w[4 * s + 0] = __builtin_bit_cast(uint32_t, p0);
      w[4 * s + 1] = __builtin_bit_cast(uint32_t, p1);
      w[4 * s + 2] = __builtin_bit_cast(uint32_t, p2);
      w[4 * s + 3] = __builtin_bit_cast(uint32_t, p3);
    }
  } else {
    const uint32_t b8[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      w[2 * d] = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<false>(b8[d]));
      w[2 * d + 1] = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<true>(b8[d]));
    }
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int k = 4 * qd + m;
    *reinterpret_cast<u32x4*>(lds + t * 256 + 16 * (k ^ (t & 15))) = u32x4{w[4 * m], w[4 * m + 1], w[4 * m + 2], w[4 * m + 3]};
  }
}

// Block scores of the shared pages [jbeg, jend) of one sharing group for all
// of the column map's columns; every thread of the 512-thread workgroup calls
// it (it synchronises the workgroup).  lds: 2 x 32 KB (page j in buffer j % 2,
// so one barrier per page orders both the stores and the reuse); the raw bytes
// of the next two pages are in flight while a page is scored.
template <bool NVFP4>
__device__ __forceinline__ void scan_shared_wide(const uint8_t* __restrict__ pool, const uint8_t* __restrict__ scales,
                                                 const int32_t* __restrict__ bt_row, const ShareCols& cm, int jbeg,
                                                 int jend, float idx_scale, uint8_t* lds, int tid) {
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int c = lane >> 4;
  const int n = lane & 15;
  const int ncols = cm.ncols;
  bool has[kWideTiles];
  int brow[kWideTiles];
  int lastp[kWideTiles];
  bf16x8 qb[kWideTiles][4];
#pragma unroll
  for (int q = 0; q < kWideTiles; ++q) {
    const int col = 16 * (wave + kWideWaves * q) + n;
    has[q] = 16 * (wave + kWideWaves * q) < ncols;  // wave-uniform
    brow[q] = col < ncols ? cm.brow(col) : -1;
    lastp[q] = col < ncols ? cm.last_pos(col) : 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int d = 64 * (s >> 1) + 16 * c + 8 * (s & 1);
      const uint4 w = col < ncols ? *reinterpret_cast<const uint4*>(cm.iq(col) + d) : make_uint4(0, 0, 0, 0);
      qb[q][s] = __builtin_bit_cast(bf16x8, w);
    }
  }
  // A operand chunks of this lane: token 16T + n, chunk 8h + 2c + u for step s = 2h + u
  int rd[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) rd[s] = n * 256 + 16 * ((8 * (s >> 1) + 2 * c + (s & 1)) ^ n);

  WideRaw<NVFP4> raw0 = wide_load<NVFP4>(pool, scales, bt_row[jbeg], tid);
  WideRaw<NVFP4> raw1 = raw0;
  if (jbeg + 1 < jend) raw1 = wide_load<NVFP4>(pool, scales, bt_row[jbeg + 1], tid);
  for (int j = jbeg; j < jend; ++j) {
    uint8_t* buf = lds + (j & 1) * (kBlock * kDim * 2);
    wide_store<NVFP4>(raw0, buf, tid);
    raw0 = raw1;
    if (j + 2 < jend) raw1 = wide_load<NVFP4>(pool, scales, bt_row[j + 2], tid);
    __syncthreads();  // page j stored; every wave is done with page j - 2's buffer
    if (!has[0]) continue;  // wave-uniform: this wave only converts
    const bool full = (j + 1) * kBlock - 1 <= cm.pos0;  // every column sees the whole block
    float m[kWideTiles];
#pragma unroll
    for (int q = 0; q < kWideTiles; ++q) m[q] = -INFINITY;
#pragma unroll 2
    for (int T = 0; T < 8; ++T) {
      bf16x8 ka[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) ka[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(buf + T * 4096 + rd[s]));
#pragma unroll
      for (int q = 0; q < kWideTiles; ++q) {
        if (!has[q]) continue;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s], qb[q][s], acc, 0, 0, 0);
        if (full) {
          m[q] = fmaxf(m[q], fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3])));
        } else {
          const int vis = lastp[q] + 1 - j * kBlock;
#pragma unroll
          for (int i = 0; i < 4; ++i) m[q] = fmaxf(m[q], 16 * T + 4 * c + i < vis ? acc[i] : -INFINITY);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kWideTiles; ++q) {
      if (!has[q]) continue;
      float x = fmaxf(m[q], __shfl_xor(m[q], 16));
      x = fmaxf(x, __shfl_xor(x, 32));
      if (c == 0 && brow[q] >= 0) *cm.at(brow[q], j) = x * idx_scale;
    }
  }
}

}  // namespace msa
