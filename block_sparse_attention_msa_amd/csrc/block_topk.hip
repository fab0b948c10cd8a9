// block_topk.hip - per (query row, group) block selection.
//
// Method ("MSA basics", vLLM MiniMax-M3.1-Flash post; "MSA mechanism details",
// MiniMax M3 x vLLM post): keep the block holding the query position
// (local_blocks = 1, init_blocks = 0) plus the best other visible blocks so
// that 16 blocks are kept; a local block that also wins top-k is not counted
// twice, so the others are the top 15 of the blocks before it.  Ties go to the
// lower block index (total order: score descending, index ascending), which
// makes the selection exact under any split of the candidates.
//
// One wave per (row, group), exact:
//  1. each lane takes the blocks j = lane + 64 e (coalesced 256 B loads) and
//     keeps its best 64-bit key (ordered score << 32 | ~j);
//  2. a 64-lane bitonic sort of the lane bests gives T0 = the 15th best lane
//     best, a lower bound of the 15th best block (15 distinct blocks >= T0);
//  3. blocks with key >= T0 (all true top-15 among them, at most 15 lanes' worth)
//     are compacted into LDS with ballots;
//  4. the candidates are merged 49 at a time into a running top-15 with the
//     same bitonic sort;
//  5. the 15 ids plus the recent block are written in ascending order.
#include "msa_device.hpp"
#include "msa_kernels.hpp"

namespace msa {
namespace {

constexpr int kMaxPerLane = (kMaxBlocksPerSeq + kWave - 1) / kWave;

__device__ __forceinline__ uint64_t block_key(float s, int j) {
  uint32_t u = __builtin_bit_cast(uint32_t, s);
  if (u == 0x80000000u) u = 0u;  // -0 ranks equal to +0
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(~(uint32_t)j);
}
__device__ __forceinline__ int key_block(uint64_t k) { return (int)(~(uint32_t)k); }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, mask);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), mask);
  return ((uint64_t)hi << 32) | lo;
}

// Bitonic sort of one key per lane, descending: lane 0 ends with the largest.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t v, int lane) {
#pragma unroll
  for (int k = 2; k <= kWave; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint64_t o = shfl_xor_u64(v, j);
      const bool lower = (lane & j) == 0;       // this lane is the lower index of its pair
      const bool desc = (lane & k) == 0;        // this sub-sequence sorts descending
      const bool take_max = (lower == desc);
      v = take_max ? (o > v ? o : v) : (o < v ? o : v);
    }
  }
  return v;
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)v, src);
  const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(v >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

__global__ __launch_bounds__(64) void block_topk_kernel(const int32_t* __restrict__ seq_lens,
                                                        const float* __restrict__ block_scores,
                                                        int32_t* __restrict__ sel, int q_len, int mbps) {
  __shared__ uint64_t cand[15 * kMaxPerLane + kWave];
  const int g = blockIdx.x;
  const int row = blockIdx.y;
  const int lane = threadIdx.x;
  const int b = row / q_len;
  const int L = seq_lens[b];
  int32_t* out = sel + ((size_t)row * kGroups + g) * kTopK;
  if (L <= 0) {
    if (lane < kTopK) out[lane] = -1;
    return;
  }
  const int pos = L - q_len + row % q_len;
  const int r = min(pos / kBlock, mbps - 1);  // recent block (clamped: never read past the row)
  if (r + 1 <= kTopK) {
    if (lane < kTopK) out[lane] = lane <= r ? lane : -1;
    return;
  }
  const float* s = block_scores + ((size_t)row * kGroups + g) * mbps;
  const int n = r;  // candidates: blocks 0 .. r-1

  // 1. best key per lane
  uint64_t best = 0;
  for (int j = lane; j < n; j += kWave) {
    const uint64_t k = block_key(s[j], j);
    best = k > best ? k : best;
  }
  // 2. T0 = 15th best lane best (lanes without blocks hold 0, below any key)
  const uint64_t sorted = wave_sort_desc(best, lane);
  const uint64_t t0 = shfl_u64(sorted, kTopK - 2);

  // 3. compact candidates >= T0 into LDS, in index order
  int count = 0;
  for (int j0 = 0; j0 < n; j0 += kWave) {
    const int j = j0 + lane;
    uint64_t k = 0;
    bool take = false;
    if (j < n) {
      k = block_key(s[j], j);
      take = k >= t0;
    }
    const uint64_t ballot = __ballot(take);
    if (take) {
      const int before = __popcll(ballot & ((1ull << lane) - 1ull));
      cand[count + before] = k;
    }
    count += __popcll(ballot);
  }
  __syncthreads();

  // 4. running top-15 in lanes 0..14, 49 new candidates per round
  uint64_t top = 0;
  for (int base = 0; base < count; base += kWave - (kTopK - 1)) {
    uint64_t v = 0;
    if (lane < kTopK - 1) {
      v = top;
    } else {
      const int idx = base + lane - (kTopK - 1);
      if (idx < count) v = cand[idx];
    }
    top = wave_sort_desc(v, lane);
  }

  // 5. 15 winners ascending by block id, then the recent block
  const int myj = lane < kTopK - 1 ? key_block(top) : 0x7fffffff;
  int rank = 0;
#pragma unroll
  for (int m = 0; m < kTopK - 1; ++m) {
    const int other = __shfl(myj, m);
    rank += other < myj ? 1 : 0;
  }
  if (lane < kTopK - 1) out[rank] = myj;
  if (lane == kTopK - 1) out[kTopK - 1] = r;
}

}  // namespace

hipError_t launch_block_topk(const TopkArgs& a, hipStream_t stream) {
  dim3 grid(kGroups, a.rows);
  block_topk_kernel<<<grid, kWave, 0, stream>>>(a.seq_lens, a.block_scores, a.sel, a.q_len, a.mbps);
  return hipGetLastError();
}

}  // namespace msa
