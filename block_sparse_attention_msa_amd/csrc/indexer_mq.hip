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
// gfx950 design: one workgroup per (sequence, 128-token block).  The block's
// index keys are converted once (E4M3 -> bf16, exact) into LDS as the MFMA A
// operand (M = tokens); each wave takes pairs of 32-row tiles of the bf16 index
// queries as B operands (N = rows) straight from global memory, and runs
// v_mfma_f32_32x32x16_bf16 over 4 token tiles x 8 K steps (bf16 x bf16 products
// are exact, fp32 accumulation).  The epilogue applies the causal mask and the
// max over the block's tokens in registers, so the score matrix never reaches
// memory; each row's block score is written once.
#include "msa_device.hpp"
#include "msa_kernels.hpp"

namespace msa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMqThreads = 256;
constexpr int kMqWaves = kMqThreads / kWave;
constexpr int kRowTile = 32;                       // MFMA N
constexpr int kTokTile = 32;                       // MFMA M
constexpr int kKStep = 16;                         // MFMA K
constexpr int kTokTiles = kBlock / kTokTile;       // 4
constexpr int kKSteps = kDim / kKStep;             // 8
constexpr int kLdsRow = kDim * 2 + 16;             // bf16 row + 16 B pad: conflict-free 16-lane groups

// MFMA 32x32x16 bf16 lane layout (gfx950): lane l supplies A[l%32][8(l/32)+e]
// and B[8(l/32)+e][l%32], e = 0..7; result register q of lane l holds
// D[8(q/4) + 4(l/32) + q%4][l%32].
template <bool FP8>
__global__ __launch_bounds__(kMqThreads) void scan_mq_kernel(const uint8_t* __restrict__ idx_pool,
                                                             const int32_t* __restrict__ block_table,
                                                             const int32_t* __restrict__ seq_lens,
                                                             const uint16_t* __restrict__ iq,
                                                             float* __restrict__ block_scores, int q_len, int mbps,
                                                             float idx_scale) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[kBlock * kLdsRow];   // 34 KB
  const int blk = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int L = seq_lens[b];
  const int nrows = q_len * kGroups;                         // (query, group) rows of this sequence
  const size_t row_base = (size_t)b * nrows;                  // first row of the sequence in [rows][4]
  float* bs = block_scores + row_base * mbps + blk;           // bs[rr * mbps] for local row rr
  const int nb = L > 0 ? (L - 1) / kBlock + 1 : 0;
  const int pos0 = L - q_len;                                 // position of query 0
  if (blk >= nb || (long long)blk * kBlock > (long long)pos0 + q_len - 1) {
    for (int rr = tid; rr < nrows; rr += kMqThreads) bs[(size_t)rr * mbps] = -INFINITY;
    return;
  }

  // ---- stage the block's index keys as bf16 [token][dim] (+pad) in LDS
  const int64_t page = block_table[(size_t)b * mbps + blk];
  if constexpr (FP8) {
    const uint8_t* src = idx_pool + page * (kBlock * kDim) + tid * 64;   // token tid/2, dims (tid%2)*64..
    u32x4 w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = *reinterpret_cast<const u32x4*>(src + i * 16);
    uint8_t* dst = lds_a + (tid >> 1) * kLdsRow + (tid & 1) * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t ws[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
      u32x4 o0, o1;
      o0.x = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<false>(ws[0]));
      o0.y = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<true>(ws[0]));
      o0.z = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<false>(ws[1]));
      o0.w = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<true>(ws[1]));
      o1.x = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<false>(ws[2]));
      o1.y = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<true>(ws[2]));
      o1.z = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<false>(ws[3]));
      o1.w = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<true>(ws[3]));
      *reinterpret_cast<u32x4*>(dst + i * 32) = o0;
      *reinterpret_cast<u32x4*>(dst + i * 32 + 16) = o1;
    }
  } else {
    const uint8_t* src = idx_pool + page * (kBlock * kDim * 2) + tid * 128;  // token tid/2, dims (tid%2)*64..
    uint8_t* dst = lds_a + (tid >> 1) * kLdsRow + (tid & 1) * 128;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<u32x4*>(dst + i * 16) = *reinterpret_cast<const u32x4*>(src + i * 16);
  }
  __syncthreads();

  const int half = lane >> 5;       // 0: k 0..7 / tokens +0..3; 1: k 8..15 / tokens +4..7
  const int col = lane & 31;        // A row (token) for operands, D column (row) for results
  const int visible_all = pos0 - blk * kBlock + 1;   // tokens of this block visible to query 0
  const int ntiles = (nrows + kRowTile - 1) / kRowTile;

  // ---- wave w takes 32-row tile pairs (2w, 2w+1), (2w + 8, ...), ...
  for (int tp = wave * 2; tp < ntiles; tp += 2 * kMqWaves) {
    // B operands of the two row tiles for all 8 K steps (rows past the end load row 0)
    bf16x8 bq[2][kKSteps];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int rr = (tp + u) * kRowTile + col;
      rr = rr < nrows ? rr : 0;
      const uint16_t* qrow = iq + (row_base + rr) * kDim + half * 8;
#pragma unroll
      for (int s = 0; s < kKSteps; ++s)
        bq[u][s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + s * kKStep));
    }
    // causal positions of this lane's two rows (row = tile*32 + col -> query row / 4)
    int vis[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) vis[u] = visible_all + ((tp + u) * kRowTile + col) / kGroups;
    const bool full = visible_all >= kBlock;   // every row of the sequence sees the whole block
    float mx[2] = {-INFINITY, -INFINITY};
#pragma unroll
    for (int m = 0; m < kTokTiles; ++m) {
      f32x16 acc[2] = {{}, {}};
#pragma unroll
      for (int s = 0; s < kKSteps; ++s) {
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(lds_a + (m * kTokTile + col) * kLdsRow + (s * kKStep + half * 8) * 2));
        acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq[0][s], acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq[1][s], acc[1], 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int tok = m * kTokTile + 8 * (q >> 2) + 4 * half + (q & 3);
          const float v = (full || tok < vis[u]) ? acc[u][q] : -INFINITY;
          mx[u] = fmaxf(mx[u], v);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      mx[u] = fmaxf(mx[u], __shfl_xor(mx[u], 32));
      const int rr = (tp + u) * kRowTile + col;
      if (half == 0 && rr < nrows) bs[(size_t)rr * mbps] = mx[u] * idx_scale;
    }
  }
}

}  // namespace

hipError_t launch_scan_mq(const ScanArgs& a, int q_len, hipStream_t stream) {
  dim3 grid(a.mbps, a.num_seqs);
  if (a.idx_fp8)
    scan_mq_kernel<true><<<grid, kMqThreads, 0, stream>>>(static_cast<const uint8_t*>(a.idx_pool), a.block_table,
                                                           a.seq_lens, a.iq, a.block_scores, q_len, a.mbps,
                                                           a.idx_scale);
  else
    scan_mq_kernel<false><<<grid, kMqThreads, 0, stream>>>(static_cast<const uint8_t*>(a.idx_pool), a.block_table,
                                                            a.seq_lens, a.iq, a.block_scores, q_len, a.mbps,
                                                            a.idx_scale);
  return hipGetLastError();
}

}  // namespace msa
