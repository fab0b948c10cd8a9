// sparse_attn.hip - the stand-alone sparse attention kernel (selection fused
// in the decode path, ids given in the stand-alone entry point); the body is
// attn_device.hpp.
#include "attn_device.hpp"
#include "msa_kernels.hpp"

namespace msa {
namespace {

template <bool FP4, bool SELECT>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(
    const uint8_t* __restrict__ kpool, const uint8_t* __restrict__ vpool, const uint8_t* __restrict__ k_sf,
    const uint8_t* __restrict__ v_sf, const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    const uint16_t* __restrict__ q, const float* __restrict__ block_scores, const int32_t* __restrict__ sel_in,
    int32_t* __restrict__ sel_out, float* __restrict__ out, int rows, int q_len, int mbps, float qk_scale_log2,
    float v_scale) {
  __shared__ AttnSmem<FP4> sm;
  int row, g, hp;
  attn_decode_wg(blockIdx.x, row, g, hp);
  if (row >= rows) return;  // grid padded to a multiple of 16 workgroups
  attn_workgroup<FP4, SELECT>(kpool, vpool, k_sf, v_sf, block_table, seq_lens, q, block_scores, sel_in,
                                     sel_out, out, q_len, mbps, qk_scale_log2, v_scale, row, g, hp, sm);
}

template <bool SELECT>
void launch(const AttnArgs& a, hipStream_t stream) {
  const long long pairs = (long long)a.rows * kGroups;
  dim3 grid((unsigned)(((pairs + 7) / 8) * 8 * kAttnHeadPairs));
  const uint8_t* kp = static_cast<const uint8_t*>(a.k);
  const uint8_t* vp = static_cast<const uint8_t*>(a.v);
  if (a.kv_nvfp4)
    attn_kernel<true, SELECT><<<grid, kAttnThreads, 0, stream>>>(kp, vp, a.k_sf, a.v_sf, a.block_table, a.seq_lens, a.q,
                                                             a.block_scores, a.sel, a.sel_out, a.out, a.rows, a.q_len, a.mbps,
                                                             a.qk_scale_log2, a.v_scale);
  else
    attn_kernel<false, SELECT><<<grid, kAttnThreads, 0, stream>>>(kp, vp, a.k_sf, a.v_sf, a.block_table, a.seq_lens, a.q,
                                                              a.block_scores, a.sel, a.sel_out, a.out, a.rows, a.q_len, a.mbps,
                                                              a.qk_scale_log2, a.v_scale);
}

}  // namespace

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t stream) {
  if (a.block_scores)
    launch<true>(a, stream);
  else
    launch<false>(a, stream);
  return hipGetLastError();
}

}  // namespace msa
