// indexer_mq.hip - multi-query index scores + causal block max-pool on MFMA.
//
// Method: the same index scores and block max-pool as the decode scan
// ("MSA basics", vLLM MiniMax-M3.1-Flash post), for q_len > 1 query tokens of
// a sequence, each at its own causal position ("Spec-decode in decode kernels"
// of the MiniMax M3 x vLLM post: query tokens flattened request-major, each
// mapped to its request's block table and causal position; "MSA mechanism
// details": the causal boundary inside a block is respected).  With q_len
// queries x 4 groups per sequence the scores are a real dense contraction:
//   S[t][r] = sum_d ik[t][d] * iq[r][d],  t = tokens, r = (query, group) rows.
//
// gfx950 design: the index queries stay, the keys stream.
//  * 512-thread workgroups, one per CU, split evenly over the (sequence,
//    256-row chunk) groups.  A workgroup stages its chunk's bf16 index queries
//    (64 KB) once in LDS (rows padded to 272 B: conflict-free 16-byte reads);
//    they serve as MFMA B operands.
//  * Each wave walks a contiguous range of (block, 32-row tile) items of its
//    group; the ranges are equal to one item, so no round of workgroups runs
//    mostly empty.  For each block it enters: 4 tiles of 32 tokens.  A lane
//    loads one token's 64 contiguous dims (FP8: 64 B) and converts them in
//    registers (E4M3 -> bf16, exact) into the A operands of 8 K steps; the
//    contraction axis is permuted (lane half h, step s, element e -> dim
//    64h + 8s + e) identically for A and B, so both come from contiguous
//    bytes.  The whole block's A operands stay in registers while the wave
//    walks the row tiles, so every B read from LDS feeds four
//    v_mfma_f32_32x32x16_bf16 (bf16 x bf16 products are exact, fp32
//    accumulation) and each row tile's block maximum is final at once.
//  * The epilogue applies the causal mask (row r = 4i + g sees tokens at or
//    before its query's position) and the max over the block's tokens in
//    registers; the score matrix never reaches memory and each (row, block)
//    score is written once.  Keys are re-read once per row chunk, from the
//    Infinity Cache after the first chunk.
#include "msa_device.hpp"
#include "msa_kernels.hpp"

namespace msa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMqThreads = 512;
constexpr int kMqWaves = kMqThreads / kWave;       // 8
constexpr int kRowChunk = 256;                     // index-query rows staged per workgroup
constexpr int kTokTiles = kBlock / 32;             // MFMA M tiles per block
constexpr int kLdsRow = kDim * 2 + 16;             // bf16 row + 16 B pad

// MFMA 32x32x16 bf16 lane layout (gfx950): lane l supplies A[l%32][8(l/32)+e]
// and B[8(l/32)+e][l%32], e = 0..7; result register q of lane l holds
// D[8(q/4) + 4(l/32) + q%4][l%32].
//
// Work split: a group = (sequence, 256-row chunk) has mbps x ntiles items
// (block, 32-row tile).  The group's wgs workgroups stage the chunk once each
// and give every wave one contiguous range of items in block-major order, so
// the waves of the grid finish within one item of each other and a wave
// converts a block's keys only when its range enters that block.
template <bool FP8>
__global__ __launch_bounds__(kMqThreads) void scan_mq_kernel(const uint8_t* __restrict__ idx_pool,
                                                             const int32_t* __restrict__ block_table,
                                                             const int32_t* __restrict__ seq_lens,
                                                             const uint16_t* __restrict__ iq,
                                                             float* __restrict__ block_scores, int q_len, int mbps,
                                                             int nchunks, int wgs, float idx_scale) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_q[kRowChunk * kLdsRow];  // 68 KB
  constexpr int kKeyRow = FP8 ? kDim : kDim * 2;  // bytes per token of an index-key page
  const int grp = blockIdx.x / wgs;
  const int wg = blockIdx.x % wgs;
  const int b = grp / nchunks;
  const int rc = grp % nchunks;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int L = seq_lens[b];
  const int nrows = q_len * kGroups;                 // (query, group) rows of this sequence
  const int row0 = rc * kRowChunk;                   // first row of this chunk
  const int crow = min(kRowChunk, nrows - row0);     // rows in this chunk (>= 1)
  const int ntiles = (crow + 31) / 32;
  const size_t srow = (size_t)b * nrows + row0;      // first global row of the chunk
  float* bs = block_scores + srow * mbps;            // bs[r * mbps + blk], r chunk-local
  const int nb = L > 0 ? (L - 1) / kBlock + 1 : 0;
  const int pos0 = L - q_len;                        // position of query 0
  const int pos_min = pos0 + row0 / kGroups;         // first and last query of the chunk
  const int pos_max = pos0 + (row0 + crow - 1) / kGroups;

  // ---- stage the chunk's index queries (rows past crow zero-filled)
  for (int i = tid; i < ntiles * 32 * 16; i += kMqThreads) {
    const int r = i >> 4, piece = i & 15;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < crow) v = *reinterpret_cast<const uint4*>(iq + (srow + r) * kDim + piece * 8);
    *reinterpret_cast<uint4*>(lds_q + r * kLdsRow + piece * 16) = v;
  }
  __syncthreads();

  const int h = lane >> 5;   // dim half of the A/B operands; token quarter of the results
  const int col = lane & 31; // A: token of the tile; B and results: row of the tile
  // this wave's item range, wave-uniform (scalar registers): items
  // [beg, end) of mbps x ntiles, walked as (block, row tile) without division
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const long long items = (long long)mbps * ntiles;
  const long long nw = (long long)wgs * kMqWaves;
  const long long gw = (long long)wg * kMqWaves + wave_u;
  const int beg = (int)(items * gw / nw), end = (int)(items * (gw + 1) / nw);

  bf16x8 a[kTokTiles][8];
  int cur = -1;          // block whose keys are in a[]
  bool seen = false;     // some row of the chunk sees block cur
  bool full = false;     // every row of the chunk sees all of block cur
  int vis0 = 0;          // tokens of block cur visible to query 0
  int blk = beg / ntiles, rt = beg - (beg / ntiles) * ntiles;
#pragma unroll 1
  for (int it = beg; it < end; ++it, rt = rt + 1 == ntiles ? 0 : rt + 1, blk += rt == 0 ? 1 : 0) {  // wave-uniform
    if (blk != cur) {
      cur = blk;
      seen = blk < nb && (long long)blk * kBlock <= pos_max;
      if (seen) {
        const int64_t page = block_table[(size_t)b * mbps + blk];
        const uint8_t* kp = idx_pool + page * (kBlock * kKeyRow) + col * kKeyRow + h * (kKeyRow / 2);
        full = (long long)blk * kBlock + kBlock - 1 <= pos_min;
        vis0 = pos0 - blk * kBlock + 1;
        // A operands of the whole block: 4 token tiles x 8 K steps
#pragma unroll
        for (int tt = 0; tt < kTokTiles; ++tt) {
          const uint8_t* src = kp + (size_t)(32 * tt) * kKeyRow;
          if constexpr (FP8) {
            u32x4 w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
              w[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + 16 * i));
            const uint32_t d[16] = {w[0].x, w[0].y, w[0].z, w[0].w, w[1].x, w[1].y, w[1].z, w[1].w,
                                    w[2].x, w[2].y, w[2].z, w[2].w, w[3].x, w[3].y, w[3].z, w[3].w};
#pragma unroll
            for (int s = 0; s < 8; ++s) {
              const bf16x2 p0 = e4m3x2_to_bf16x2<false>(d[2 * s]);
              const bf16x2 p1 = e4m3x2_to_bf16x2<true>(d[2 * s]);
              const bf16x2 p2 = e4m3x2_to_bf16x2<false>(d[2 * s + 1]);
              const bf16x2 p3 = e4m3x2_to_bf16x2<true>(d[2 * s + 1]);
              a[tt][s] = bf16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
            }
          } else {
#pragma unroll
            for (int s = 0; s < 8; ++s)
              a[tt][s] = __builtin_bit_cast(bf16x8,
                                            __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + 16 * s)));
          }
        }
      }
    }
    const int r = 32 * rt + col;
    if (!seen) {  // no row of the chunk sees this block
      if (h == 0 && r < crow) bs[(size_t)r * mbps + blk] = -INFINITY;
      continue;
    }
    // ---- one row tile: 4 accumulators, every B read from LDS feeds 4 MFMAs
    const uint8_t* qrow = lds_q + (32 * rt + col) * kLdsRow + h * kDim;  // dims 64h..
    bf16x8 bq[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) bq[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qrow + 16 * s));
    f32x16 acc[kTokTiles];
#pragma unroll
    for (int tt = 0; tt < kTokTiles; ++tt) acc[tt] = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int tt = 0; tt < kTokTiles; ++tt)
        acc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[tt][s], bq[s], acc[tt], 0, 0, 0);
      // keep the four independent accumulator chains interleaved: a chain's
      // next MFMA then issues only after the other three
      __builtin_amdgcn_sched_barrier(0);
    }
    float m = -INFINITY;
    if (full) {  // wave-uniform: no mask
#pragma unroll
      for (int q = 0; q < 16; ++q) m = fmaxf(m, fmaxf(fmaxf(acc[0][q], acc[1][q]), fmaxf(acc[2][q], acc[3][q])));
    } else {
      // this lane's row (column of D) sees tokens < vis of the block
      const int vis = vis0 + (row0 + r) / kGroups;
#pragma unroll
      for (int tt = 0; tt < kTokTiles; ++tt)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int tok = 32 * tt + 8 * (q >> 2) + 4 * h + (q & 3);
          m = fmaxf(m, tok < vis ? acc[tt][q] : -INFINITY);
        }
    }
    m = fmaxf(m, __shfl_xor(m, 32));
    if (h == 0 && r < crow) bs[(size_t)r * mbps + blk] = m * idx_scale;
  }
}

}  // namespace

hipError_t launch_scan_mq(const ScanArgs& a, int q_len, hipStream_t stream) {
  const int nrows = q_len * kGroups;
  const int nchunks = (nrows + kRowChunk - 1) / kRowChunk;
  // one workgroup per CU (its registers and LDS allow no second), split evenly
  // over the (sequence, row chunk) groups
  const long long groups = (long long)a.num_seqs * nchunks;
  const int cus = device_cus();
  const int wgs = (int)(groups >= cus ? 1 : cus / groups);
  dim3 grid((unsigned)(groups * wgs));
  if (a.idx_fmt == kIdxFp8)
    scan_mq_kernel<true><<<grid, kMqThreads, 0, stream>>>(static_cast<const uint8_t*>(a.idx_pool), a.block_table,
                                                           a.seq_lens, a.iq, a.block_scores, q_len, a.mbps, nchunks, wgs,
                                                           a.idx_scale);
  else
    scan_mq_kernel<false><<<grid, kMqThreads, 0, stream>>>(static_cast<const uint8_t*>(a.idx_pool), a.block_table,
                                                            a.seq_lens, a.iq, a.block_scores, q_len, a.mbps, nchunks, wgs,
                                                            a.idx_scale);
  return hipGetLastError();
}

}  // namespace msa
