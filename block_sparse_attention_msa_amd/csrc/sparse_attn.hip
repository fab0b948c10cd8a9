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

// Loads of a split part's partial (COHERENT: device-coherent, for partials
// stored by other workgroups of the same launch).
template <bool COHERENT>
__device__ __forceinline__ float2 load_f32x2(const float* p) {
  if constexpr (COHERENT) {
    const uint64_t u =
        __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(__builtin_bit_cast(float, (uint32_t)u), __builtin_bit_cast(float, (uint32_t)(u >> 32)));
  } else {
    return *reinterpret_cast<const float2*>(p);
  }
}

// Log-sum-exp merge of the SPLIT partials of (row, group) pair `id` by one
// wave.  For the factors lane l takes (part l / 4, head l % 4); for the sums
// head l / 16, dims 8 (l % 16) .. + 7.  Every load is issued up front, none
// waiting on another: each part of a non-padded row writes its partial (zeros
// and (-inf, 0) without keys); a padded row's partials are never written,
// are read anyway (inside the buffer) and discarded: its output is 0.
template <int SPLIT, bool COHERENT>
__device__ __forceinline__ void split_merge_pair(int id, int lane, const int32_t* __restrict__ seq_lens, int q_len,
                                                 const float* __restrict__ po, const float2* __restrict__ pml,
                                                 float v_scale, float* __restrict__ out) {
  static_assert(SPLIT * kHeadsPerGroup <= kWave, "one factor per lane");
  const int row = id / kGroups;
  const int h = lane >> 4, d0 = 8 * (lane & 15);
  const int L = seq_lens[row / q_len];
  const float* ml_src = reinterpret_cast<const float*>(pml + (size_t)id * SPLIT * kHeadsPerGroup + lane);
  const float2 ml = lane < SPLIT * kHeadsPerGroup ? load_f32x2<COHERENT>(ml_src) : make_float2(-INFINITY, 0.f);
  const float* src = po + ((size_t)id * SPLIT * kHeadsPerGroup + h) * kDim + d0;
  float2 v[SPLIT][4];
#pragma unroll
  for (int p = 0; p < SPLIT; ++p)
#pragma unroll
    for (int k = 0; k < 4; ++k) v[p][k] = load_f32x2<COHERENT>(src + p * kHeadsPerGroup * kDim + 2 * k);
  float M = ml.x;
#pragma unroll
  for (int off = kHeadsPerGroup; off < kWave; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
  const float f = ml.x == -INFINITY ? 0.f : exp2_nonpos(ml.x - M);
  float fl = f * ml.y;
#pragma unroll
  for (int off = kHeadsPerGroup; off < kWave; off <<= 1) fl += __shfl_xor(fl, off);
  float acc[8] = {};
#pragma unroll
  for (int p = 0; p < SPLIT; ++p) {
    const float w = __shfl(f, kHeadsPerGroup * p + h);  // 0 for a part without keys (its partial is 0)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc[2 * k] = fmaf(w, v[p][k].x, acc[2 * k]);
      acc[2 * k + 1] = fmaf(w, v[p][k].y, acc[2 * k + 1]);
    }
  }
  const float flh = __shfl(fl, h);  // lanes 0 .. 3 hold heads 0 .. 3
  const float sc = L > 0 && flh > 0.f ? v_scale / flh : 0.f;
  float4* dst = reinterpret_cast<float4*>(out + ((size_t)id * kHeadsPerGroup + h) * kDim + d0);
  dst[0] = L > 0 ? make_float4(acc[0] * sc, acc[1] * sc, acc[2] * sc, acc[3] * sc) : make_float4(0.f, 0.f, 0.f, 0.f);
  dst[1] = L > 0 ? make_float4(acc[4] * sc, acc[5] * sc, acc[6] * sc, acc[7] * sc) : make_float4(0.f, 0.f, 0.f, 0.f);
}

// Kept blocks split over SPLIT workgroups of NT = 1024 / SPLIT x TS threads,
// each block's tokens over TS waves; each workgroup writes its partial
// (o, M, sum) per head.
// MERGE: the parts count their arrival on the pair's counter (zero at
// launch) once their partial stores are complete, and the last one merges
// the pair's partials and writes the output; otherwise a second launch
// merges them.
template <bool FP4, bool SELECT, int SPLIT, bool MERGE, int TS>
__global__ __launch_bounds__(1024 / SPLIT * TS) void attn_split_kernel(
    const uint8_t* __restrict__ kpool, const uint8_t* __restrict__ vpool, const uint8_t* __restrict__ k_sf,
    const uint8_t* __restrict__ v_sf, const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    const uint16_t* __restrict__ q, const float* __restrict__ block_scores, const int32_t* __restrict__ sel_in,
    int32_t* __restrict__ sel_out, float* __restrict__ po, float2* __restrict__ pml, int32_t* __restrict__ counters,
    float* __restrict__ out, int rows, int q_len, int mbps, float qk_scale_log2, float v_scale) {
  constexpr int NT = 1024 / SPLIT * TS;
  __shared__ AttnSmem<NT> sm;
  __shared__ int last;
  int pair, part;
  attn_decode_wg<SPLIT>(blockIdx.x, pair, part);
  if (pair >= rows * kGroups) return;
  attn_workgroup<FP4, SELECT, 1, NT, SPLIT, MERGE, TS>(kpool, vpool, k_sf, v_sf, block_table, seq_lens, q, block_scores,
                                                  sel_in, sel_out, nullptr, q_len, mbps, qk_scale_log2, 1.f,
                                                  pair / kGroups, pair % kGroups, part, sm, po, pml);
  if constexpr (MERGE) {
    // this thread's partial stores complete (write-through, device scope)
    // before the workgroup's arrival is counted
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
      last = __hip_atomic_fetch_add(counters + pair, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP) == SPLIT - 1;
    __syncthreads();
    if (last && threadIdx.x < kWave)
      split_merge_pair<SPLIT, true>(pair, threadIdx.x, seq_lens, q_len, po, pml, v_scale, out);
  }
}

// The merge launch: one wave per (row, group) pair.
template <int SPLIT>
__global__ __launch_bounds__(256) void attn_split_merge_kernel(const int32_t* __restrict__ seq_lens, int pairs,
                                                               int q_len, const float* __restrict__ po,
                                                               const float2* __restrict__ pml, float v_scale,
                                                               float* __restrict__ out) {
  const int id = blockIdx.x * 4 + threadIdx.x / kWave;
  if (id >= pairs) return;
  split_merge_pair<SPLIT, false>(id, threadIdx.x & (kWave - 1), seq_lens, q_len, po, pml, v_scale, out);
}

// bf16 K/V: each kept block's 128 tokens over TS = 4 waves, so that no wave
// streams a whole 64 KB block through its own outstanding loads; the 8-block
// parts (SPLIT = 2) keep one wave per block (16 waves would exceed 128 VGPRs).
template <bool FP4, int SPLIT>
constexpr int split_token_waves() { return !FP4 && SPLIT >= 4 ? 4 : 1; }

template <bool FP4, bool SELECT, int SPLIT>
void launch_split(const AttnArgs& a, hipStream_t stream) {
  constexpr int TS = split_token_waves<FP4, SPLIT>();
  constexpr int NT = 1024 / SPLIT * TS;
  const long long pairs = (long long)a.rows * kGroups;
  float* po = a.partials;
  float2* pml = reinterpret_cast<float2*>(a.partials + (size_t)pairs * kTopK * kHeadsPerGroup * kDim);
  const dim3 grid((unsigned)(((pairs + 7) / 8) * 8 * SPLIT));
  if (a.counters) {  // merged by the last part of each pair: one launch
    attn_split_kernel<FP4, SELECT, SPLIT, true, TS><<<grid, NT, 0, stream>>>(
        static_cast<const uint8_t*>(a.k), static_cast<const uint8_t*>(a.v), a.k_sf, a.v_sf, a.block_table,
        a.seq_lens, a.q, a.block_scores, a.sel, a.sel_out, po, pml, a.counters, a.out, a.rows, a.q_len, a.mbps,
        a.qk_scale_log2, a.v_scale);
    return;
  }
  attn_split_kernel<FP4, SELECT, SPLIT, false, TS><<<grid, NT, 0, stream>>>(
      static_cast<const uint8_t*>(a.k), static_cast<const uint8_t*>(a.v), a.k_sf, a.v_sf, a.block_table, a.seq_lens,
      a.q, a.block_scores, a.sel, a.sel_out, po, pml, nullptr, nullptr, a.rows, a.q_len, a.mbps, a.qk_scale_log2,
      a.v_scale);
  attn_split_merge_kernel<SPLIT><<<dim3((unsigned)((pairs + 3) / 4)), 256, 0, stream>>>(
      a.seq_lens, (int)pairs, a.q_len, po, pml, a.v_scale, a.out);
}

// Kept blocks split over workgroups (bf16 K/V, few (row, group) pairs, a
// partials buffer): SPLIT = 16 / w, w the waves the selection needs for the row
// length (1,024 blocks per wave, rounded up to a power of two); the same
// split with the selection fused or the ids given, so that both give the
// same sums.  Returns false where it does not apply.
template <bool FP4, bool SELECT>
bool try_launch_split(const AttnArgs& a, hipStream_t stream) {
  const long long pairs = (long long)a.rows * kGroups;
  if (!a.partials || pairs > kSplitMaxPairs) return false;
  int w = 1;
  while (w * sel_max_blocks<kWave>() < a.mbps) w *= 2;
  switch (w) {
    case 1: launch_split<FP4, SELECT, 16>(a, stream); return true;
    case 2: launch_split<FP4, SELECT, 8>(a, stream); return true;
    case 4: launch_split<FP4, SELECT, 4>(a, stream); return true;
    case 8: launch_split<FP4, SELECT, 2>(a, stream); return true;
    default: return false;
  }
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
  // NVFP4 K/V: the on-chip merge (no partials) also for few pairs; against the
  // kept blocks split over 16 one-wave workgroups merged by the last of them
  // (same box): batch 8 x 32K 19.2 us per step against 20.4 us, batch
  // 4 x 512K 55.5 against 55.0, batch 32 x 128K (128 pairs) 97.6 against
  // 107.7.  bf16 K/V (a 64 KB block per wave) keep the split: one workgroup
  // per pair would read all 16 K blocks through one CU.
  if (a.kv_nvfp4) {
    if (a.block_scores)
      launch2<true, true>(a, stream);
    else
      launch2<true, false>(a, stream);
  } else {
    if (a.block_scores) {
      if (!try_launch_split<false, true>(a, stream)) launch2<false, true>(a, stream);
    } else if (!try_launch_split<false, false>(a, stream)) {
      launch2<false, false>(a, stream);
    }
  }
  return hipGetLastError();
}

}  // namespace msa
