// indexer_scan.hip - decode index scan fused with the block max-pool.
//
// Method ("MSA basics", vLLM MiniMax-M3.1-Flash post): every visible context
// token t is scored against one index query per GQA group with a single shared
// index-key head, s_g[t] = sum_d iq[g][d] * ik[t][d], and the scores are
// max-pooled to one value per 128-token block.  The scan reads 128 B (FP8) of
// index key per token and is the dominant HBM stream of a decode step
// ("Decode indexer-score kernel" of the M3 post: a dedicated scan over the
// ragged per-request block ranges, not a padded dense GEMM).
//
// The per-wave body (layout, conversions, reduction) is in scan_device.hpp.
#include "msa_device.hpp"
#include "msa_kernels.hpp"
#include "scan_device.hpp"

namespace msa {
namespace {

constexpr int kScanWaves = 8;

template <bool FP8>
// At most 102 VGPRs (5 waves per SIMD): one more resident wave per SIMD than
// the unconstrained allocation (100 VGPRs, 4 waves) keeps more page loads in
// flight.
__global__ __launch_bounds__(kScanWaves * kWave, 5) void scan_decode_kernel(const uint8_t* __restrict__ idx_pool,
                                                                          const int32_t* __restrict__ block_table,
                                                                          const int32_t* __restrict__ seq_lens,
                                                                          const uint16_t* __restrict__ iq,
                                                                          float* __restrict__ block_scores, int mbps,
                                                                          int blocks_per_wave, float idx_scale) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int jbeg = (blockIdx.x * (blockDim.x / kWave) + wave) * blocks_per_wave;
  if (jbeg >= mbps) return;
  const int jend = min(jbeg + blocks_per_wave, mbps);
  scan_wave<FP8>(idx_pool, block_table + (size_t)b * mbps, seq_lens[b], iq + (size_t)b * kGroups * kDim,
                        block_scores + (size_t)b * kGroups * mbps, mbps, jbeg, jend, idx_scale, lane);
}

// NVFP4 index keys: one page per wave; 1 KB of LDS per wave for the scales.
// 4-wave workgroups at 6 waves per SIMD (at most 85 VGPRs), from a sweep on
// the batch-32 x 128K shape: 48.0-48.4 us, against 49.4-54.2 us for 8 waves
// at 5 per SIMD, 53.7-55.5 us for 16 waves, 59-62 us for two pages per wave
// with the second page's loads issued ahead, and 70 us at 7 per SIMD.
constexpr int kNvfp4ScanWaves = 4;
__global__ __launch_bounds__(kNvfp4ScanWaves * kWave, 6) void scan_decode_nvfp4_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const uint16_t* __restrict__ iq, float* __restrict__ block_scores, int mbps,
    float idx_scale) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_sc[kNvfp4ScanWaves][kBlock * 8];
  const int b = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int j = blockIdx.x * kNvfp4ScanWaves + wave;
  if (j >= mbps) return;
  scan_wave_nvfp4(codes, scales, block_table + (size_t)b * mbps, seq_lens[b], iq + (size_t)b * kGroups * kDim,
                  block_scores + (size_t)b * kGroups * mbps, mbps, j, j + 1, idx_scale, lds_sc[wave], lane);
}

// FP8 index keys, q_len <= 8: 16 x NT (query, group) columns per sequence on
// MFMA, pages_per_wave consecutive pages per wave (the B operands are loaded
// once per wave).
constexpr int kColsScanWaves = 8;
template <int NT>
__global__ __launch_bounds__(kColsScanWaves * kWave) void scan_cols_kernel(const uint8_t* __restrict__ idx_pool,
                                                                         const int32_t* __restrict__ block_table,
                                                                         const int32_t* __restrict__ seq_lens,
                                                                         const uint16_t* __restrict__ iq,
                                                                         float* __restrict__ block_scores, int q_len,
                                                                         int mbps, int pages_per_wave, float idx_scale) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_t[kColsScanWaves][2 * 2048];
  const int b = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int jbeg = (blockIdx.x * kColsScanWaves + wave) * pages_per_wave;
  if (jbeg >= mbps) return;
  const int jend = min(jbeg + pages_per_wave, mbps);
  const int L = seq_lens[b];
  const int ncols = q_len * kGroups;
  const SeqCols cm{iq + (size_t)b * ncols * kDim, block_scores + (size_t)b * ncols * mbps, mbps, ncols, L - q_len,
                   L > 0 ? (L - 1) / kBlock + 1 : 0};
  scan_wave_fp8_mfma<NT>(idx_pool, block_table + (size_t)b * mbps, cm, jbeg, jend, idx_scale, lds_t[wave], lane);
}

// Prefix sharing (FP8 index keys, q_len 1) in one launch: grid rows y <
// num_groups are the shared pass, one wave per (sharing group, shared block):
// the group leader's page is read once and scored against the index queries
// of all the group's members (up to 8: 32 MFMA columns); rows y >= num_groups
// are the sequences' own blocks (the column scan, the shared blocks skipped).
// The shared rows come first in dispatch order, so the two parts overlap.
__global__ __launch_bounds__(kColsScanWaves * kWave, 4) void scan_shared_kernel(
    const uint8_t* __restrict__ idx_pool, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const uint16_t* __restrict__ iq, float* __restrict__ block_scores,
    const int32_t* __restrict__ members, const int32_t* __restrict__ shared_blocks,
    const int32_t* __restrict__ seq_shared_blocks, int num_groups, int mbps, float idx_scale) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_t[kColsScanWaves][2 * 2048];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int j = blockIdx.x * kColsScanWaves + wave;
  if ((int)blockIdx.y >= num_groups) {  // a sequence's own blocks
    const int b = blockIdx.y - num_groups;
    if (j >= mbps || j < seq_shared_blocks[b]) return;
    const int L = seq_lens[b];
    const SeqCols cm{iq + (size_t)b * kGroups * kDim, block_scores + (size_t)b * kGroups * mbps, mbps, kGroups, L - 1,
                     L > 0 ? (L - 1) / kBlock + 1 : 0};
    scan_wave_fp8_mfma<1>(idx_pool, block_table + (size_t)b * mbps, cm, j, j + 1, idx_scale, lds_t[wave], lane);
    return;
  }
  const int gi = blockIdx.y;
  if (j >= min(shared_blocks[gi], mbps)) return;
  const int32_t* mem = members + (size_t)gi * kShareMax;
  int nmem = 0, pos0 = 0x7fffffff;
  for (int k = 0; k < kShareMax; ++k) {  // wave-uniform
    if (mem[k] < 0) break;
    ++nmem;
    pos0 = min(pos0, seq_lens[mem[k]] - 1);
  }
  if (nmem == 0) return;
  const ShareCols cm{mem, seq_lens, iq, block_scores, mbps, nmem * kGroups, pos0, 0x7fffffff};
  scan_wave_fp8_mfma<2>(idx_pool, block_table + (size_t)mem[0] * mbps, cm, j, j + 1, idx_scale, lds_t[wave], lane);
}

// The same with NVFP4 index keys: the shared rows dequantise each shared page
// exactly to bf16 once for the group's members (up to 32 (member, group)
// columns); the own rows are the NVFP4 decode scan's, so those scores equal
// the unshared call's.
__global__ __launch_bounds__(kColsScanWaves * kWave, 4) void scan_shared_nvfp4_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const uint16_t* __restrict__ iq, float* __restrict__ block_scores,
    const int32_t* __restrict__ members, const int32_t* __restrict__ shared_blocks,
    const int32_t* __restrict__ seq_shared_blocks, int num_groups, int mbps, float idx_scale) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_sc[kColsScanWaves][kBlock * 8];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int j = blockIdx.x * kColsScanWaves + wave;
  if ((int)blockIdx.y >= num_groups) {  // a sequence's own blocks
    const int b = blockIdx.y - num_groups;
    if (j >= mbps || j < seq_shared_blocks[b]) return;
    scan_wave_nvfp4(codes, scales, block_table + (size_t)b * mbps, seq_lens[b], iq + (size_t)b * kGroups * kDim,
                    block_scores + (size_t)b * kGroups * mbps, mbps, j, j + 1, idx_scale, lds_sc[wave], lane);
    return;
  }
  const int gi = blockIdx.y;
  if (j >= min(shared_blocks[gi], mbps)) return;
  const int32_t* mem = members + (size_t)gi * kShareMax;
  int nmem = 0, pos0 = 0x7fffffff;
  for (int k = 0; k < kShareMax; ++k) {  // wave-uniform
    if (mem[k] < 0) break;
    ++nmem;
    pos0 = min(pos0, seq_lens[mem[k]] - 1);
  }
  if (nmem == 0) return;
  const ShareCols cm{mem, seq_lens, iq, block_scores, mbps, nmem * kGroups, pos0, 0x7fffffff};
  scan_wave_nvfp4_exact_cols<2>(codes, scales, block_table + (size_t)mem[0] * mbps, cm, j, j + 1, idx_scale,
                                lds_sc[wave], lane);
}

// NVFP4 index keys, 2 <= q_len <= 8: the same columns, keys dequantised
// exactly to bf16 in registers (no LDS).
template <int NT>
__global__ __launch_bounds__(kColsScanWaves * kWave) void scan_cols_nvfp4_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const uint16_t* __restrict__ iq, float* __restrict__ block_scores, int q_len,
    int mbps, int pages_per_wave, float idx_scale) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_sc[kColsScanWaves][kBlock * 8];
  const int b = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int jbeg = (blockIdx.x * kColsScanWaves + wave) * pages_per_wave;
  if (jbeg >= mbps) return;
  const int jend = min(jbeg + pages_per_wave, mbps);
  const size_t ncols = (size_t)q_len * kGroups;
  scan_wave_nvfp4_cols<NT>(codes, scales, block_table + (size_t)b * mbps, seq_lens[b], q_len, iq + b * ncols * kDim,
                           block_scores + b * ncols * mbps, mbps, jbeg, jend, idx_scale, lds_sc[wave], lane);
}

}  // namespace

hipError_t launch_scan_cols(const ScanArgs& a, int q_len, hipStream_t stream) {
  if (q_len < 1 || q_len > 8 || a.idx_fmt == kIdxBf16 || (a.idx_fmt == kIdxNvfp4 && q_len < 2))
    return hipErrorInvalidValue;
  // 8-wave workgroups at 4 waves per SIMD; from a sweep on the batch-32 x 128K
  // shape: q_len 1 80.6 us with one page per wave (81.3-81.8 us with 2 or 4),
  // q_len 4 88 us with two (91.5 us with one, 88 us with four); 4- and 16-wave
  // workgroups 1-10 % slower, 5 waves per SIMD (at most 102 VGPRs) 11-13 %.
  const int ppw = q_len == 1 ? 1 : 2;
  const int per_wg = kColsScanWaves * ppw;
  dim3 grid((a.mbps + per_wg - 1) / per_wg, a.num_seqs);
  dim3 block(kColsScanWaves * kWave);
  const uint8_t* pool = static_cast<const uint8_t*>(a.idx_pool);
  if (a.idx_fmt == kIdxNvfp4) {
    if (q_len <= 4)
      scan_cols_nvfp4_kernel<1><<<grid, block, 0, stream>>>(pool, a.idx_sf, a.block_table, a.seq_lens, a.iq,
                                                             a.block_scores, q_len, a.mbps, ppw, a.idx_scale);
    else
      scan_cols_nvfp4_kernel<2><<<grid, block, 0, stream>>>(pool, a.idx_sf, a.block_table, a.seq_lens, a.iq,
                                                             a.block_scores, q_len, a.mbps, ppw, a.idx_scale);
    return hipGetLastError();
  }
  if (q_len <= 4)
    scan_cols_kernel<1><<<grid, block, 0, stream>>>(pool, a.block_table, a.seq_lens, a.iq, a.block_scores, q_len,
                                                     a.mbps, ppw, a.idx_scale);
  else
    scan_cols_kernel<2><<<grid, block, 0, stream>>>(pool, a.block_table, a.seq_lens, a.iq, a.block_scores, q_len,
                                                     a.mbps, ppw, a.idx_scale);
  return hipGetLastError();
}

hipError_t launch_scan_shared(const ScanArgs& a, const int32_t* members, const int32_t* shared_blocks,
                              const int32_t* seq_shared_blocks, int num_groups, hipStream_t stream) {
  if (a.idx_fmt == kIdxBf16 || num_groups + a.num_seqs > 65535) return hipErrorInvalidValue;
  dim3 grid((a.mbps + kColsScanWaves - 1) / kColsScanWaves, num_groups + a.num_seqs);
  if (a.idx_fmt == kIdxNvfp4) {
    scan_shared_nvfp4_kernel<<<grid, dim3(kColsScanWaves * kWave), 0, stream>>>(
        static_cast<const uint8_t*>(a.idx_pool), a.idx_sf, a.block_table, a.seq_lens, a.iq, a.block_scores, members,
        shared_blocks, seq_shared_blocks, num_groups, a.mbps, a.idx_scale);
    return hipGetLastError();
  }
  scan_shared_kernel<<<grid, dim3(kColsScanWaves * kWave), 0, stream>>>(
      static_cast<const uint8_t*>(a.idx_pool), a.block_table, a.seq_lens, a.iq, a.block_scores, members,
      shared_blocks, seq_shared_blocks, num_groups, a.mbps, a.idx_scale);
  return hipGetLastError();
}

hipError_t launch_scan_decode(const ScanArgs& a, hipStream_t stream) {
  // FP8 index keys: the MFMA column scan (80.6 us on the batch-32 x 128K
  // shape against 82-85 us for the VALU scan below with FP8 keys).
  if (a.idx_fmt == kIdxFp8) return launch_scan_cols(a, 1, stream);
  // bf16 index keys: the VALU scan, 8-wave workgroups, one page per wave (with
  // FP8 keys on the batch-32 x 128K workload: 81.4-84.2 us at 5 waves per
  // SIMD vs 82.2-83.3 us for 2 or 4 pages per wave, 82.8-85.7 us at 4 waves
  // per SIMD, 84.0-85.1 us for 2- or 4-wave workgroups, 116 us at 6 per SIMD).
  const int bpw = 1;
  constexpr int waves_per_wg = kScanWaves;
  dim3 grid((a.mbps + waves_per_wg * bpw - 1) / (waves_per_wg * bpw), a.num_seqs);
  dim3 block(waves_per_wg * kWave);
  if (a.idx_fmt == kIdxNvfp4) {
    dim3 g2((a.mbps + kNvfp4ScanWaves - 1) / kNvfp4ScanWaves, a.num_seqs);
    scan_decode_nvfp4_kernel<<<g2, dim3(kNvfp4ScanWaves * kWave), 0, stream>>>(static_cast<const uint8_t*>(a.idx_pool), a.idx_sf,
                                                       a.block_table, a.seq_lens, a.iq, a.block_scores, a.mbps,
                                                       a.idx_scale);
  } else
    scan_decode_kernel<false><<<grid, block, 0, stream>>>(static_cast<const uint8_t*>(a.idx_pool), a.block_table,
                                                           a.seq_lens, a.iq, a.block_scores, a.mbps, bpw, a.idx_scale);
  return hipGetLastError();
}

}  // namespace msa
