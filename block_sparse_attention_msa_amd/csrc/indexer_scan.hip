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
                                                                          int blocks_per_wave, float idx_scale,
                                                                          int32_t* __restrict__ zero, int zero_n) {
  zero_step_counters(zero, zero_n);
  const int b = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int jbeg = (blockIdx.x * (blockDim.x / kWave) + wave) * blocks_per_wave;
  if (jbeg >= mbps) return;
  const int jend = min(jbeg + blocks_per_wave, mbps);
  scan_wave<FP8>(idx_pool, block_table + (size_t)b * mbps, seq_lens[b], iq + (size_t)b * kGroups * kDim,
                        block_scores + (size_t)b * kGroups * mbps, mbps, jbeg, jend, idx_scale, lane);
}

// bf16 index keys, few pages: each page's 32 wave-loads split over S waves of
// a workgroup (kScanWaves / S pages per workgroup), whose per-wave block
// maxima are combined through LDS.  A batch of a few short rows otherwise
// runs one wave per page, a long serial chain on an almost empty GPU.  The
// scores are the one-wave scan's (the same products and sums per token; the
// maximum does not depend on the order).
template <int S>
__global__ __launch_bounds__(kScanWaves * kWave) void scan_decode_split_kernel(
    const uint8_t* __restrict__ idx_pool, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const uint16_t* __restrict__ iq, float* __restrict__ block_scores, int mbps,
    float idx_scale, int32_t* __restrict__ zero, int zero_n) {
  zero_step_counters(zero, zero_n);
  using Geo = ScanGeom<false>;
  static_assert(kScanWaves % S == 0 && Geo::kLoadsPerBlock % S == 0, "whole pages per workgroup");
  constexpr int kN = Geo::kLoadsPerBlock / S;  // wave-loads per wave
  __shared__ float part_max[kScanWaves][kGroups];
  const int b = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int j = blockIdx.x * (kScanWaves / S) + wave / S;
  const int part = wave % S;
  const bool in = j < mbps;  // wave-uniform; every wave reaches the barrier
  const int32_t* bt_row = block_table + (size_t)b * mbps;
  const int32_t pg = in ? bt_row[j] : 0;  // read before the visibility test, never followed unless visible
  const int L = seq_lens[b];
  const int nbv = L > 0 ? ((L - 1) / kBlock) + 1 : 0;
  const bool vis = in && j < nbv;
  float m = -INFINITY;
  if (vis) {
    uint32_t qr[4][Geo::kPairsPerLane];
    scan_query_slice<false>(iq + (size_t)b * kGroups * kDim, lane, qr);
    const uint8_t* base = idx_pool + (int64_t)pg * Geo::kPageBytes + lane * 16;
    m = scan_loads<false, kN>(base, qr, L - j * kBlock, part * kN, lane, m);
    m = wave_max_xor(m, Geo::kLanesPerToken);
  }
  if (lane < kGroups) part_max[wave][lane_group(lane)] = m;
  __syncthreads();
  if (part == 0 && in && lane < kGroups) {
    const int g = lane_group(lane);
    float x = part_max[wave][g];
#pragma unroll
    for (int p = 1; p < S; ++p) x = fmaxf(x, part_max[wave + p][g]);
    block_scores[((size_t)b * kGroups + g) * mbps + j] = vis ? x * idx_scale : -INFINITY;
  }
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
    float idx_scale, int32_t* __restrict__ zero, int zero_n) {
  zero_step_counters(zero, zero_n);
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
                                                                         int mbps, int pages_per_wave, float idx_scale,
                                                                         int32_t* __restrict__ zero, int zero_n) {
  zero_step_counters(zero, zero_n);
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

// Prefix sharing in one launch (FP8 or NVFP4 index keys, 1 <= q_len <= 8).
// The first workgroups are the shared pass: workgroup (x, group) takes the
// group's shared blocks 8x .. 8x + 7, each page read once from HBM and scored
// against the index queries of all the group's members:
//  * WIDE = false (at most 32 (member, query, group) columns: max_members x
//    q_len <= 8): one wave per page, two 16-column tiles in registers (FP8: the
//    column scan's body; NVFP4: the page dequantised exactly to bf16 in
//    registers);
//  * WIDE = true (up to 256 columns: 64 decode requests, or 64 / q_len
//    requests of q_len tokens): the workgroup converts each page once into
//    LDS and its 8 waves score it against 2 column tiles each.
// The rest are the sequences' own blocks from block min_shared on (a lower
// bound of every sequence's shared count, so no workgroup is spent on blocks
// known to be shared), with the unshared scans' bodies, the shared blocks
// skipped.  The shared pass comes first in dispatch order, so the two parts
// overlap.  With FP8 keys every block score equals
// the unshared scan's bit for bit (the same products and fp32 sums in the
// same order); with NVFP4 keys the shared pages are dequantised exactly to
// bf16 and their scores agree with the unshared scan's to fp32 rounding.
// NT_OWN: 16-column tiles of a sequence's own (query, group) columns (0: NVFP4
// keys at q_len 1, the decode scan's body); Q1: q_len is 1 (a compile-time
// column count keeps the q_len 1 forms within their registers).
template <bool NVFP4, int NT_OWN, int MINW, bool WIDE, bool Q1>
__global__ __launch_bounds__(kColsScanWaves * kWave, MINW) void scan_shared_kernel(
    const uint8_t* __restrict__ pool, const uint8_t* __restrict__ scales, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const uint16_t* __restrict__ iq, float* __restrict__ block_scores,
    const int32_t* __restrict__ members, const int32_t* __restrict__ shared_blocks,
    const int32_t* __restrict__ seq_shared_blocks, int num_groups, int max_members, int q_len_arg, int mbps,
    int min_shared, float idx_scale, int32_t* __restrict__ zero, int zero_n) {
  zero_step_counters(zero, zero_n);
  const int q_len = Q1 ? 1 : q_len_arg;
  // one flat grid: num_groups x xs workgroups of the shared pass, then
  // num_seqs x xo of the own blocks (which start at block min_shared)
  const int xs = (mbps + kColsScanWaves - 1) / kColsScanWaves;
  const int xo = (mbps - min_shared + kColsScanWaves - 1) / kColsScanWaves;
  const int id = blockIdx.x;
  const bool own_row = id >= num_groups * xs;
  const int row = own_row ? (id - num_groups * xs) / xo : id / xs;
  const int wx = own_row ? (id - num_groups * xs) % xo : id % xs;
  // wide: two 32 KB page buffers; otherwise 4 KB (FP8) or 1 KB (NVFP4) per wave
  __shared__ __attribute__((aligned(16))) uint8_t lds[WIDE ? 2 * kBlock * kDim * 2 : kColsScanWaves * 2 * 2048];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int ncols_seq = q_len * kGroups;
  if (own_row) {  // a sequence's own blocks
    const int b = row;
    const int j = min_shared + wx * kColsScanWaves + wave;
    if (j >= mbps || j < seq_shared_blocks[b]) return;
    const int L = seq_lens[b];
    const uint16_t* iq_seq = iq + (size_t)b * ncols_seq * kDim;
    float* bs_seq = block_scores + (size_t)b * ncols_seq * mbps;
    if constexpr (NVFP4) {
      uint8_t* lds_sc = lds + wave * (kBlock * 8);
      if constexpr (NT_OWN == 0)  // q_len 1
        scan_wave_nvfp4(pool, scales, block_table + (size_t)b * mbps, L, iq_seq, bs_seq, mbps, j, j + 1, idx_scale,
                        lds_sc, lane);
      else
        scan_wave_nvfp4_cols<NT_OWN>(pool, scales, block_table + (size_t)b * mbps, L, q_len, iq_seq, bs_seq, mbps, j,
                                     j + 1, idx_scale, lds_sc, lane);
    } else {
      const SeqCols cm{iq_seq, bs_seq, mbps, ncols_seq, L - q_len, L > 0 ? (L - 1) / kBlock + 1 : 0};
      scan_wave_fp8_mfma<NT_OWN>(pool, block_table + (size_t)b * mbps, cm, j, j + 1, idx_scale,
                                 lds + wave * (2 * 2048), lane);
    }
    return;
  }
  const int gi = row;
  const int jbeg = wx * kColsScanWaves;
  const int jend = min(min(shared_blocks[gi], mbps), jbeg + kColsScanWaves);
  if (jbeg >= jend) return;  // workgroup-uniform
  // the group's members in one lane each (two loads in flight, not a chain):
  // the member count runs to the first -1, pos0 is their least first-query position
  const int32_t* mem = members + (size_t)gi * max_members;
  const int mk = lane < max_members ? mem[lane] : -1;
  const uint64_t stop = __ballot(mk < 0);
  const int nmem = stop ? __builtin_ctzll(stop) : kWave;  // workgroup-uniform
  if (nmem == 0) return;
  int p = lane < nmem ? seq_lens[mk] - q_len : 0x7fffffff;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) p = min(p, __shfl_xor(p, off));
  const int pos0 = p;
  const ShareCols cm{mem, seq_lens, iq, block_scores, mbps, nmem * ncols_seq, pos0, 0x7fffffff, q_len};
  const int32_t* bt_lead = block_table + (size_t)mem[0] * mbps;
  if constexpr (WIDE) {
    scan_shared_wide<NVFP4>(pool, scales, bt_lead, cm, jbeg, jend, idx_scale, lds, tid);
  } else {
    const int j = jbeg + wave;
    if (j >= jend) return;
    if constexpr (NVFP4)
      scan_wave_nvfp4_exact_cols<2>(pool, scales, bt_lead, cm, j, j + 1, idx_scale, lds + wave * (kBlock * 8), lane);
    else
      scan_wave_fp8_mfma<2>(pool, bt_lead, cm, j, j + 1, idx_scale, lds + wave * (2 * 2048), lane);
  }
}

// NVFP4 index keys, 2 <= q_len <= 8: the same columns, keys dequantised
// exactly to bf16 in registers (no LDS).
template <int NT>
__global__ __launch_bounds__(kColsScanWaves * kWave) void scan_cols_nvfp4_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const uint16_t* __restrict__ iq, float* __restrict__ block_scores, int q_len,
    int mbps, int pages_per_wave, float idx_scale, int32_t* __restrict__ zero, int zero_n) {
  zero_step_counters(zero, zero_n);
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
  // NVFP4 keys (q_len 2-8) on the same shape: 53.0-53.7 us with four pages
  // per wave against 54.8-54.9 with two, 61.6-62.2 with one and 63.5 / 70.2
  // with eight / sixteen (too few workgroups to fill the GPU), so four where
  // the batch has at least 128 pages per CU (1,024 workgroups at 256 CUs).
  const bool deep = a.idx_fmt == kIdxNvfp4 && (long long)a.num_seqs * a.mbps >= 128LL * device_cus();
  const int ppw = q_len == 1 ? 1 : deep ? 4 : 2;
  const int per_wg = kColsScanWaves * ppw;
  dim3 grid((a.mbps + per_wg - 1) / per_wg, a.num_seqs);
  dim3 block(kColsScanWaves * kWave);
  const uint8_t* pool = static_cast<const uint8_t*>(a.idx_pool);
  if (a.idx_fmt == kIdxNvfp4) {
    if (q_len <= 4)
      scan_cols_nvfp4_kernel<1><<<grid, block, 0, stream>>>(pool, a.idx_sf, a.block_table, a.seq_lens, a.iq,
                                                             a.block_scores, q_len, a.mbps, ppw, a.idx_scale,
                                                             a.zero, a.zero_n);
    else
      scan_cols_nvfp4_kernel<2><<<grid, block, 0, stream>>>(pool, a.idx_sf, a.block_table, a.seq_lens, a.iq,
                                                             a.block_scores, q_len, a.mbps, ppw, a.idx_scale,
                                                             a.zero, a.zero_n);
    return hipGetLastError();
  }
  if (q_len <= 4)
    scan_cols_kernel<1><<<grid, block, 0, stream>>>(pool, a.block_table, a.seq_lens, a.iq, a.block_scores, q_len,
                                                     a.mbps, ppw, a.idx_scale, a.zero, a.zero_n);
  else
    scan_cols_kernel<2><<<grid, block, 0, stream>>>(pool, a.block_table, a.seq_lens, a.iq, a.block_scores, q_len,
                                                     a.mbps, ppw, a.idx_scale, a.zero, a.zero_n);
  return hipGetLastError();
}

hipError_t launch_scan_shared(const ScanArgs& a, const int32_t* members, const int32_t* shared_blocks,
                              const int32_t* seq_shared_blocks, int num_groups, int max_members, int min_shared,
                              int q_len, hipStream_t stream) {
  if (a.idx_fmt == kIdxBf16 || q_len < 1 || q_len > 8 || max_members < 1 || max_members * q_len > kShareMax ||
      min_shared < 0 || min_shared >= a.mbps)
    return hipErrorInvalidValue;
  const long long xs = (a.mbps + kColsScanWaves - 1) / kColsScanWaves;
  const long long xo = (a.mbps - min_shared + kColsScanWaves - 1) / kColsScanWaves;
  const long long wgs = num_groups * xs + (long long)a.num_seqs * xo;
  if (wgs <= 0 || wgs > 0x7fffffffLL) return hipErrorInvalidValue;
  dim3 grid((unsigned)wgs);
  dim3 block(kColsScanWaves * kWave);
  const uint8_t* pool = static_cast<const uint8_t*>(a.idx_pool);
#define MSA_SHARED_ARGS                                                                                      \
  pool, a.idx_sf, a.block_table, a.seq_lens, a.iq, a.block_scores, members, shared_blocks, seq_shared_blocks, \
      num_groups, max_members, q_len, a.mbps, min_shared, a.idx_scale, a.zero, a.zero_n
  // at most 32 (member, query, group) columns: one wave per shared page
  const bool wide = max_members * q_len * kGroups > 32;
  if (a.idx_fmt == kIdxNvfp4) {
    if (!wide) {
      if (q_len == 1)
        scan_shared_kernel<true, 0, 4, false, true><<<grid, block, 0, stream>>>(MSA_SHARED_ARGS);
      else if (q_len <= 4)
        scan_shared_kernel<true, 1, 4, false, false><<<grid, block, 0, stream>>>(MSA_SHARED_ARGS);
      else
        scan_shared_kernel<true, 2, 4, false, false><<<grid, block, 0, stream>>>(MSA_SHARED_ARGS);
    } else if (q_len == 1) {
      // the wide forms' two 32 KB page buffers leave room for two workgroups
      // per CU: 4 waves per SIMD whatever the registers
      scan_shared_kernel<true, 0, 4, true, true><<<grid, block, 0, stream>>>(MSA_SHARED_ARGS);
    } else if (q_len <= 4) {
      scan_shared_kernel<true, 1, 4, true, false><<<grid, block, 0, stream>>>(MSA_SHARED_ARGS);
    } else {
      scan_shared_kernel<true, 2, 4, true, false><<<grid, block, 0, stream>>>(MSA_SHARED_ARGS);
    }
  } else {
    if (!wide) {
      if (q_len == 1)
        scan_shared_kernel<false, 1, 4, false, true><<<grid, block, 0, stream>>>(MSA_SHARED_ARGS);
      else if (q_len <= 4)
        scan_shared_kernel<false, 1, 4, false, false><<<grid, block, 0, stream>>>(MSA_SHARED_ARGS);
      else
        scan_shared_kernel<false, 2, 4, false, false><<<grid, block, 0, stream>>>(MSA_SHARED_ARGS);
    } else if (q_len == 1) {
      scan_shared_kernel<false, 1, 4, true, true><<<grid, block, 0, stream>>>(MSA_SHARED_ARGS);
    } else if (q_len <= 4) {
      scan_shared_kernel<false, 1, 4, true, false><<<grid, block, 0, stream>>>(MSA_SHARED_ARGS);
    } else {
      scan_shared_kernel<false, 2, 4, true, false><<<grid, block, 0, stream>>>(MSA_SHARED_ARGS);
    }
  }
#undef MSA_SHARED_ARGS
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
    scan_decode_nvfp4_kernel<<<g2, dim3(kNvfp4ScanWaves * kWave), 0, stream>>>(
        static_cast<const uint8_t*>(a.idx_pool), a.idx_sf, a.block_table, a.seq_lens, a.iq, a.block_scores, a.mbps,
        a.idx_scale, a.zero, a.zero_n);
  } else if ((long long)a.num_seqs * a.mbps <= 2LL * device_cus()) {
    // few pages: 8 waves per page (4 wave-loads, 16 tokens each)
    constexpr int S = kScanWaves;
    dim3 g2((a.mbps + kScanWaves / S - 1) / (kScanWaves / S), a.num_seqs);
    scan_decode_split_kernel<S><<<g2, block, 0, stream>>>(static_cast<const uint8_t*>(a.idx_pool), a.block_table,
                                                           a.seq_lens, a.iq, a.block_scores, a.mbps, a.idx_scale,
                                                           a.zero, a.zero_n);
  } else {
    scan_decode_kernel<false><<<grid, block, 0, stream>>>(static_cast<const uint8_t*>(a.idx_pool), a.block_table,
                                                           a.seq_lens, a.iq, a.block_scores, a.mbps, bpw, a.idx_scale,
                                                           a.zero, a.zero_n);
  }
  return hipGetLastError();
}

}  // namespace msa
