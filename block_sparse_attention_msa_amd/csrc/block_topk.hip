// block_topk.hip - stand-alone block selection: one 1024-thread workgroup per
// (query row, group) running the exact selection of select_device.hpp
// (recent block + top 15 of the earlier blocks by score desc, index asc).
#include "msa_device.hpp"
#include "msa_kernels.hpp"
#include "select_device.hpp"

namespace msa {
namespace {

constexpr int kThreads = 1024;
static_assert(sel_max_blocks<kThreads>() >= kMaxBlocksPerSeq, "every row length fits one workgroup");

__global__ __launch_bounds__(kThreads) void block_topk_kernel(const int32_t* __restrict__ seq_lens,
                                                              const float* __restrict__ block_scores,
                                                              int32_t* __restrict__ sel, int q_len, int mbps) {
  __shared__ SelectSmem<kThreads> sm;
  const int g = blockIdx.x;
  const int row = blockIdx.y;
  const int b = row / q_len;
  const int L = seq_lens[b];
  int32_t* out = sel + ((size_t)row * kGroups + g) * kTopK;
  if (L <= 0) {
    if (threadIdx.x < kTopK) out[threadIdx.x] = -1;
    return;
  }
  const int pos = L - q_len + row % q_len;
  const int r = min(pos / kBlock, mbps - 1);  // recent block (clamped: never read past the row)
  select_blocks<kThreads, false>(block_scores + ((size_t)row * kGroups + g) * mbps, nullptr, r, sm, out, nullptr);
}

}  // namespace

hipError_t launch_block_topk(const TopkArgs& a, hipStream_t stream) {
  dim3 grid(kGroups, a.rows);
  block_topk_kernel<<<grid, kThreads, 0, stream>>>(a.seq_lens, a.block_scores, a.sel, a.q_len, a.mbps);
  return hipGetLastError();
}

}  // namespace msa
