// sparse_attn.hip - the sparse attention kernel (selection fused in the
// decode path, ids given in the stand-alone entry point); the body is
// attn_device.hpp.  One workgroup per (query row, group, output part).
#include <atomic>

#include "attn_device.hpp"
#include "msa_kernels.hpp"

namespace msa {
namespace {

// Workgroups are dispatched round-robin over the 8 XCDs (id % 8).  The DSPLIT
// parts of one (row, group) get ids 8 apart, so they run on one XCD and the
// repeated reads of the group's K blocks hit its L2.
template <int DSPLIT>
__device__ __forceinline__ void attn_decode_wg(int id, int& pair, int& part) {
  const int x = id & 7;
  const int k = id >> 3;
  part = k % DSPLIT;
  pair = (k / DSPLIT) * 8 + x;
}

// Four waves per SIMD: for the 512-thread form, room for two workgroups per CU.
template <bool FP4, bool SELECT, int DSPLIT, int NT>
__global__ __launch_bounds__(NT, 4) void attn_kernel(
    const uint8_t* __restrict__ kpool, const uint8_t* __restrict__ vpool, const uint8_t* __restrict__ k_sf,
    const uint8_t* __restrict__ v_sf, const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    const uint16_t* __restrict__ q, const float* __restrict__ block_scores, const int32_t* __restrict__ sel_in,
    int32_t* __restrict__ sel_out, float* __restrict__ out, int rows, int q_len, int mbps, float qk_scale_log2,
    float v_scale) {
  __shared__ AttnSmem<NT> sm;
  int pair, part;
  attn_decode_wg<DSPLIT>(blockIdx.x, pair, part);
  if (pair >= rows * kGroups) return;  // grid padded to a multiple of 8 (row, group) pairs
  attn_workgroup<FP4, SELECT, DSPLIT, NT>(kpool, vpool, k_sf, v_sf, block_table, seq_lens, q, block_scores, sel_in,
                                      sel_out, out, q_len, mbps, qk_scale_log2, v_scale, pair / kGroups,
                                      pair % kGroups, part, sm);
}

template <bool FP4, bool SELECT, int DSPLIT, int NT>
void launch3(const AttnArgs& a, hipStream_t stream) {
  const long long pairs = (long long)a.rows * kGroups;
  const dim3 grid((unsigned)(((pairs + 7) / 8) * 8 * DSPLIT));
  attn_kernel<FP4, SELECT, DSPLIT, NT><<<grid, NT, 0, stream>>>(
      static_cast<const uint8_t*>(a.k), static_cast<const uint8_t*>(a.v), a.k_sf, a.v_sf, a.block_table, a.seq_lens,
      a.q, a.block_scores, a.sel, a.sel_out, a.out, a.rows, a.q_len, a.mbps, a.qk_scale_log2, a.v_scale);
}

template <bool FP4, bool SELECT>
void launch2(const AttnArgs& a, hipStream_t stream) {
  // Split each (row, group) over 2 or 4 workgroups by output dims while that
  // still leaves at least one workgroup per CU: few rows are latency-bound.
  const long long pairs = (long long)a.rows * kGroups;
  const int cus = device_cus();
  // With more (row, group) pairs than CUs, 512-thread workgroups (two kept
  // blocks per wave) let two workgroups share a CU when the row fits their
  // selection (at most 8,192 blocks); bf16 K/V keep the 1024-thread form
  // (their two-block body does not fit 128 VGPRs).
  if (pairs * 4 <= cus) {
    launch3<FP4, SELECT, 4, 1024>(a, stream);
  } else if (pairs * 2 <= cus) {
    launch3<FP4, SELECT, 2, 1024>(a, stream);
  } else {
    if constexpr (FP4) {
      if (!SELECT || a.mbps <= sel_max_blocks<512>()) {
        launch3<FP4, SELECT, 1, 512>(a, stream);
        return;
      }
    }
    launch3<FP4, SELECT, 1, 1024>(a, stream);
  }
}

}  // namespace

int device_cus() {
  // per device, filled on first use; calls from several host threads may
  // race to fill an entry, which they do with the same value
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int cus = cached[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cached[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t stream) {
  if (a.kv_nvfp4) {
    if (a.block_scores)
      launch2<true, true>(a, stream);
    else
      launch2<true, false>(a, stream);
  } else {
    if (a.block_scores)
      launch2<false, true>(a, stream);
    else
      launch2<false, false>(a, stream);
  }
  return hipGetLastError();
}

}  // namespace msa
