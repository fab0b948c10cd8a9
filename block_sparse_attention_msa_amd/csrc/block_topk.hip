// block_topk.hip - stand-alone block selection: one workgroup per (query
// row, group) running the exact selection of select_device.hpp (recent block
// + top 15 of the earlier blocks by score desc, index asc).  The workgroup has
// one wave per 1,024 candidate blocks of the row length (64 to 1024 threads),
// so short rows leave room for many workgroups per CU.
#include "msa_device.hpp"
#include "msa_kernels.hpp"
#include "select_device.hpp"

namespace msa {
namespace {

static_assert(sel_max_blocks<1024>() >= kMaxBlocksPerSeq, "every row length fits one workgroup");

template <int NT>
__global__ __launch_bounds__(NT) void block_topk_kernel(const int32_t* __restrict__ seq_lens,
                                                        const float* __restrict__ block_scores,
                                                        int32_t* __restrict__ sel, int q_len, int mbps) {
  __shared__ SelectSmem<NT> sm;
  const int g = blockIdx.x;
  const int row = blockIdx.y;
  const int b = row / q_len;
  const int L = seq_lens[b];
  SelLoads ld;  // issued before the row length arrives
  select_load<NT, false>(block_scores + ((size_t)row * kGroups + g) * mbps, nullptr, mbps, ld);
  int32_t* out = sel + ((size_t)row * kGroups + g) * kTopK;
  if (L <= 0) {
    if (threadIdx.x < kTopK) out[threadIdx.x] = -1;
    return;
  }
  const int pos = L - q_len + row % q_len;
  const int r = min(pos / kBlock, mbps - 1);  // recent block (clamped: never read past the row)
  select_blocks<NT, false>(ld, nullptr, r, mbps, sm, out, nullptr);
}

template <int NT>
void launch_nt(const TopkArgs& a, hipStream_t stream) {
  block_topk_kernel<NT><<<dim3(kGroups, a.rows), NT, 0, stream>>>(a.seq_lens, a.block_scores, a.sel, a.q_len, a.mbps);
}

}  // namespace

hipError_t launch_block_topk(const TopkArgs& a, hipStream_t stream) {
  // candidates are the blocks before the recent one: fewer than mbps
  if (a.mbps <= sel_max_blocks<64>())
    launch_nt<64>(a, stream);
  else if (a.mbps <= sel_max_blocks<128>())
    launch_nt<128>(a, stream);
  else if (a.mbps <= sel_max_blocks<256>())
    launch_nt<256>(a, stream);
  else if (a.mbps <= sel_max_blocks<512>())
    launch_nt<512>(a, stream);
  else
    launch_nt<1024>(a, stream);
  return hipGetLastError();
}

}  // namespace msa
