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
// gfx950 design: the index queries stay in registers, the keys stream through
// LDS once per workgroup.
//  * 512-thread workgroups, one per CU, split evenly over the (sequence,
//    256-row chunk) groups; a workgroup takes a contiguous range of blocks.
//    Wave w owns row tile w (32 (query, group) rows): its B operands (the
//    rows' bf16 index queries, 8 K steps) are staged through LDS once and then
//    stay in 32 VGPRs for the whole range.
//  * The 8 waves walk their blocks together.  A block's keys (16 KB FP8, 32
//    KB bf16, 8 KB of NVFP4 codes + 1 KB of group scales) are loaded by all
//    waves in contiguous 1 KB wave-loads two blocks ahead into registers,
//    converted once per workgroup to bf16 (E4M3 -> bf16; E2M1 code x E4M3
//    group scale, at most 6 significant bits; both exact) and written to one
//    of two 32 KB LDS buffers with a swizzle
//    (16-B chunk k of token t at t * 256 + 16 (k ^ (t mod 16))), so that both
//    the row writes and the MFMA-layout reads are free of bank conflicts; one
//    barrier per block.
//  * Per 32-token tile a wave reads its A operands, 8 K steps of its lane's
//    token, straight from LDS (contraction axis permuted: lane half h, step
//    s, element e -> dim 64h + 8s + e, identically for A and B) and runs 8
//    v_mfma_f32_32x32x16_bf16 (exact products, fp32 sums); in wholly visible
//    blocks the next tile's reads overlap the current tile's MFMAs.
//  * Epilogue: causal mask (row r = 4i + g sees tokens <= its query's
//    position) only for partly visible blocks, max over the block's tokens in
//    registers; the score matrix never reaches memory and each (row, block)
//    score is written once.
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
template <int FMT>
__global__ __launch_bounds__(kMqThreads) void scan_mq_kernel(const uint8_t* __restrict__ idx_pool,
                                                             const uint8_t* __restrict__ idx_sf,
                                                             const int32_t* __restrict__ block_table,
                                                             const int32_t* __restrict__ seq_lens,
                                                             const uint16_t* __restrict__ iq,
                                                             float* __restrict__ block_scores, int q_len, int mbps,
                                                             int nchunks, int wgs, float idx_scale,
                                                             int32_t* __restrict__ zero, int zero_n) {
  zero_step_counters(zero, zero_n);
  // bytes per token of an index-key page: E4M3, bf16, or E2M1 codes (NVFP4,
  // whose 8 group scales per token sit in idx_sf, 1 KB per page)
  constexpr int kKeyRow = FMT == kIdxFp8 ? kDim : FMT == kIdxBf16 ? kDim * 2 : kDim / 2;
  constexpr int kPage = kBlock * kKeyRow;             // 16, 32 or 8 KB
  constexpr int kLoads = kPage / 1024 / kMqWaves;     // 1 KB wave-loads per wave and block (2, 4 or 1)
  static_assert(FMT != kIdxNvfp4 || kLoads == 1, "NVFP4: one wave-load, so one pair of group scales, per wave");
  constexpr int kRowB = kDim * 2;                     // bytes per token of a bf16 key row in LDS
  __shared__ __attribute__((aligned(16))) uint8_t lds_q[kRowChunk * kLdsRow];     // 68 KB
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[2][kBlock * kRowB];       // 2 x 32 KB, bf16 keys
  const int grp = blockIdx.x / wgs;
  const int wg = blockIdx.x % wgs;
  const int b = grp / nchunks;
  const int rc = grp % nchunks;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
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
  const int32_t* bt_row = block_table + (size_t)b * mbps;
  // this workgroup's blocks
  const int jbeg = (int)((long long)mbps * wg / wgs), jend = (int)((long long)mbps * (wg + 1) / wgs);

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
  const bool active = wave < ntiles;  // wave-uniform: this wave owns a row tile
  const int r = 32 * wave + col;      // this lane's row (B column, result column), chunk-local
  bf16x8 bq[8];
  {
    const uint8_t* qrow = lds_q + (active ? r : 0) * kLdsRow + h * kDim;  // dims 64h..
#pragma unroll
    for (int s = 0; s < 8; ++s) bq[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qrow + 16 * s));
  }

  // block j is seen by some row of the chunk (wave-uniform)
  auto seen = [&](int j) { return j < nb && (long long)j * kBlock <= pos_max; };
  // this wave's share of block j's keys: kLoads contiguous 1 KB wave-loads
  // (NVFP4: plus the two group scales of the lane's 32 dims, 2 bytes)
  auto load_keys = [&](int j, u32x4 (&v)[kLoads], uint32_t& sf) {
    if (j < jend && seen(j)) {
      const int64_t page = bt_row[j];
      const uint8_t* src = idx_pool + page * kPage + (size_t)(wave * kLoads) * 1024 + lane * 16;
#pragma unroll
      for (int i = 0; i < kLoads; ++i) v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + i * 1024));
      if constexpr (FMT == kIdxNvfp4) {
        const int byte = wave * 1024 + lane * 16;  // token byte / 64, dims 32 ((byte % 64) / 16) ..
        sf = *reinterpret_cast<const uint16_t*>(idx_sf + page * (kBlock * 8) + (byte / 64) * 8 + ((byte % 64) / 16) * 2);
      }
    }
  };
  // ... written to LDS buffer buf as bf16 (exact, converted once per
  // workgroup), swizzled: 16-B chunk k (dims 8k .. 8k + 7) of token t at
  // t * 256 + 16 (k ^ (t mod 16))
  auto lds_chunk = [&](int buf, int t, int k) { return &lds_k[buf][t * kRowB + ((k ^ (t & 15)) << 4)]; };
  auto store_keys = [&](int j, int buf, const u32x4 (&v)[kLoads], uint32_t sf) {
    if (j < jend && seen(j)) {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int byte = (wave * kLoads + i) * 1024 + lane * 16;  // offset in the page
        const int t = byte / kKeyRow, k = (byte % kKeyRow) / 16;  // token, 16-B chunk of the stored row
        if constexpr (FMT == kIdxNvfp4) {  // 32 dims (groups 2k, 2k + 1) -> bf16 chunks 4k .. 4k + 3
          const uint32_t d[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
          const float s0 = e4m3_to_f32(sf & 0xFFu), s1 = e4m3_to_f32((sf >> 8) & 0xFFu);
#pragma unroll
          for (int q = 0; q < 4; ++q) {  // dims 32k + 8q .. + 7, group 2k + q / 2
            const float sc = q < 2 ? s0 : s1;
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              f32x2 x;
              switch (e) {
                case 0: x = e2m1x2_to_f32x2<0>(d[q]); break;
                case 1: x = e2m1x2_to_f32x2<1>(d[q]); break;
                case 2: x = e2m1x2_to_f32x2<2>(d[q]); break;
                default: x = e2m1x2_to_f32x2<3>(d[q]); break;
              }
              // code x scale: at most 6 significant bits, so the product and
              // its bf16 conversion are exact
              const bf16x2 y = {(__bf16)(x.x * sc), (__bf16)(x.y * sc)};
              o[e] = __builtin_bit_cast(uint32_t, y);
            }
            *reinterpret_cast<u32x4*>(lds_chunk(buf, t, 4 * k + q)) = u32x4{o[0], o[1], o[2], o[3]};
          }
        } else if constexpr (FMT == kIdxFp8) {  // 16 dims -> bf16 chunks 2k, 2k + 1
          const uint32_t d[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
          uint32_t o[8];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            o[2 * q] = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<false>(d[q]));
            o[2 * q + 1] = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<true>(d[q]));
          }
          *reinterpret_cast<u32x4*>(lds_chunk(buf, t, 2 * k)) = u32x4{o[0], o[1], o[2], o[3]};
          *reinterpret_cast<u32x4*>(lds_chunk(buf, t, 2 * k + 1)) = u32x4{o[4], o[5], o[6], o[7]};
        } else {
          *reinterpret_cast<u32x4*>(lds_chunk(buf, t, k)) = v[i];
        }
      }
    }
  };

  u32x4 pf1[kLoads], pf2[kLoads];  // keys of blocks j + 1 and j + 2, in flight
  uint32_t sf1 = 0, sf2 = 0;       // their group scales (NVFP4)
  load_keys(jbeg, pf1, sf1);
  store_keys(jbeg, 0, pf1, sf1);
  load_keys(jbeg + 1, pf1, sf1);
  __syncthreads();
#pragma unroll 1
  for (int j = jbeg; j < jend; ++j) {  // wave-uniform
    const int buf = (j - jbeg) & 1;
    load_keys(j + 2, pf2, sf2);
    if (!seen(j)) {  // no row of the chunk sees this block
      if (active && h == 0 && r < crow) bs[(size_t)r * mbps + j] = -INFINITY;
    } else if (active) {
      const bool full = (long long)j * kBlock + kBlock - 1 <= pos_min;  // every row sees the whole block
      const int vis = pos0 + (row0 + r) / kGroups + 1 - j * kBlock;     // tokens this lane's row sees
      float m = -INFINITY;
      // A operands of token 32tt + col: bf16 dims 64h + 8s .. + 7 from LDS
      auto read_a = [&](int tt, bf16x8 (&a)[8]) {
        const int t = 32 * tt + col;
#pragma unroll
        for (int s = 0; s < 8; ++s)
          a[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(lds_chunk(buf, t, 8 * h + s)));
      };
      auto mfma8 = [&](const bf16x8 (&a)[8]) {
        f32x16 acc = f32x16{};
#pragma unroll
        for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], bq[s], acc, 0, 0, 0);
        return acc;
      };
      if (full) {
        // Every row sees the whole block: no masks.  Two operand sets and two
        // accumulators alternate, so tile tt + 1's LDS reads are interleaved
        // with tile tt's MFMAs (one read per MFMA, by scheduling groups) and
        // tile tt's max runs behind tile tt + 1's MFMAs.
        bf16x8 a0[8], a1[8];
        f32x16 c0, c1;
        auto max16 = [&](const f32x16& c) {
#pragma unroll
          for (int q = 0; q < 16; ++q) m = fmaxf(m, c[q]);
        };
        read_a(0, a0);
#pragma unroll
        for (int tt = 0; tt < kTokTiles; ++tt) {
          bf16x8 (&cur)[8] = (tt & 1) ? a1 : a0;
          bf16x8 (&nxt)[8] = (tt & 1) ? a0 : a1;
          if (tt + 1 < kTokTiles) read_a(tt + 1, nxt);
          ((tt & 1) ? c1 : c0) = mfma8(cur);
          if (tt + 1 < kTokTiles) {
#pragma unroll
            for (int s = 0; s < 8; ++s) {
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            }
          }
          if (tt > 0) max16((tt & 1) ? c0 : c1);
        }
        max16((kTokTiles & 1) ? c0 : c1);
      } else {
#pragma unroll
        for (int tt = 0; tt < kTokTiles; ++tt) {
          bf16x8 a[8];
          read_a(tt, a);
          const f32x16 acc = mfma8(a);
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int tok = 32 * tt + 8 * (q >> 2) + 4 * h + (q & 3);
            m = fmaxf(m, tok < vis ? acc[q] : -INFINITY);
          }
        }
      }
      m = fmaxf(m, __shfl_xor(m, 32));
      if (h == 0 && r < crow) bs[(size_t)r * mbps + j] = m * idx_scale;
    }
    // the next block's keys into the other buffer (read by nobody since the
    // last barrier), then the barrier that publishes them
    store_keys(j + 1, buf ^ 1, pf1, sf1);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) pf1[i] = pf2[i];
    sf1 = sf2;
    __syncthreads();
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
  const uint8_t* pool = static_cast<const uint8_t*>(a.idx_pool);
  if (a.idx_fmt == kIdxFp8)
    scan_mq_kernel<kIdxFp8><<<grid, kMqThreads, 0, stream>>>(pool, nullptr, a.block_table, a.seq_lens, a.iq,
                                                              a.block_scores, q_len, a.mbps, nchunks, wgs, a.idx_scale,
                                                              a.zero, a.zero_n);
  else if (a.idx_fmt == kIdxNvfp4)
    scan_mq_kernel<kIdxNvfp4><<<grid, kMqThreads, 0, stream>>>(pool, a.idx_sf, a.block_table, a.seq_lens, a.iq,
                                                                a.block_scores, q_len, a.mbps, nchunks, wgs, a.idx_scale,
                                                                a.zero, a.zero_n);
  else
    scan_mq_kernel<kIdxBf16><<<grid, kMqThreads, 0, stream>>>(pool, nullptr, a.block_table, a.seq_lens, a.iq,
                                                               a.block_scores, q_len, a.mbps, nchunks, wgs, a.idx_scale,
                                                               a.zero, a.zero_n);
  return hipGetLastError();
}

}  // namespace msa
