// msa_kernels.hpp - internal launchers of the MSA kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

constexpr int kBlock = 128;               // tokens per KV block / page
constexpr int kDim = 128;                 // head dim == index dim
constexpr int kTopK = 16;                 // kept blocks per (row, group)
constexpr int kGroups = 4;                // KV heads == GQA groups
constexpr int kHeadsPerGroup = 4;         // query heads per group
constexpr int kMaxBlocksPerSeq = 16384;   // 2M tokens per sequence

enum IdxFormat { kIdxBf16 = 0, kIdxFp8 = 1, kIdxNvfp4 = 2 };

struct ScanArgs {
  const void* idx_pool;        // [P][128][128] FP8 or bf16, or [P][128][64] NVFP4 codes
  const uint8_t* idx_sf;       // NVFP4: E4M3 scales [P][128][8]
  const int32_t* block_table;  // [S][mbps]
  const int32_t* seq_lens;     // [S]
  const uint16_t* iq;          // bf16 [S][4][128]
  float* block_scores;         // [S][4][mbps]
  int num_seqs;
  int mbps;
  float idx_scale;
  int idx_fmt;                 // IdxFormat
  // counters of the attention launch that follows in the same decode step,
  // zeroed by the scan's first workgroup (at most 64), or nullptr
  int32_t* zero = nullptr;
  int zero_n = 0;
};
// Decode (one query row per sequence) index scan + block max-pool.
hipError_t launch_scan_decode(const ScanArgs& a, hipStream_t stream);
// Multi-query (q_len > 1) index scores + causal block max-pool on MFMA.
hipError_t launch_scan_mq(const ScanArgs& a, int q_len, hipStream_t stream);
// FP8 index keys with 1 <= q_len <= 8, NVFP4 with 2 <= q_len <= 8: the (query, group) columns on
// MFMA, pages streamed by waves.
hipError_t launch_scan_cols(const ScanArgs& a, int q_len, hipStream_t stream);
// Index scan with prefix sharing (FP8 or NVFP4 index keys, 1 <= q_len <= 8), one
// launch: each sharing group's shared pages read once for all its members
// (members rows of max_members entries, max_members x q_len <= kShareMax),
// the sequences' own blocks as in the unshared scans.
constexpr int kShareMax = 64;
hipError_t launch_scan_shared(const ScanArgs& a, const int32_t* members, const int32_t* shared_blocks,
                              const int32_t* seq_shared_blocks, int num_groups, int max_members, int min_shared,
                              int q_len, hipStream_t stream);

struct TopkArgs {
  const int32_t* seq_lens;
  const float* block_scores;   // [rows][4][mbps]
  int32_t* sel;                // [rows][4][16]
  int rows;
  int q_len;
  int mbps;
};
hipError_t launch_block_topk(const TopkArgs& a, hipStream_t stream);

struct AttnArgs {
  const void* k;
  const void* v;
  const uint8_t* k_sf;
  const uint8_t* v_sf;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const uint16_t* q;           // bf16 [rows][16][128]
  const float* block_scores;   // [rows][4][mbps]: select in-kernel (fused path), or nullptr
  const int32_t* sel;          // [rows][4][16] ids when block_scores is nullptr
  int32_t* sel_out;            // fused path: where to store the selection, or nullptr
  float* out;                  // [rows][16][128]
  int rows;
  int q_len;
  int mbps;
  float qk_scale_log2;         // sm_scale * k_scale * log2(e)
  float v_scale;
  bool kv_nvfp4;
  // bf16 K/V with at most kSplitMaxPairs (row, group) pairs: room for the
  // kept-block split's partials (split_partials_bytes), or nullptr
  float* partials = nullptr;
  // with partials: one arrival counter per (row, group), zero at launch (the
  // decode step's scan zeroes them); the last part to arrive merges the
  // partials.  nullptr: a second launch merges them.
  int32_t* counters = nullptr;
};
// Few (row, group) pairs with bf16 K/V: the kept blocks are split over
// workgroups whose partials are merged by the last one to finish, or by a
// second launch (NVFP4 K/V merge on chip: no partials).  The partials buffer:
// o [pairs][16][4][128] fp32, (M, sum) [pairs][16][4] float2, then the
// counters [pairs] int32.
constexpr int kSplitMaxPairs = 64;
inline size_t split_counters_offset(long long pairs) {
  return (size_t)pairs * kTopK * kHeadsPerGroup * (kDim * 4 + 8);
}
inline size_t split_partials_bytes(long long pairs, bool kv_nvfp4) {
  return !kv_nvfp4 && pairs <= kSplitMaxPairs ? split_counters_offset(pairs) + (size_t)pairs * 4 : 0;
}
// Selection (fused path) + attention: one launch.
hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t stream);

// KV-block-major attention over given ids (a.sel), NVFP4 K/V: inversion of
// the selections into per-block row lists, block-major partials, merge (three
// launches).  scratch: block_major_scratch_bytes(num_seqs, q_len) bytes.
constexpr int kBmMaxQ = 256;         // query rows per sequence (16 x 256 selections per (sequence, group))
constexpr int kBmMaxBlocks = 8192;   // block-table row length (1M tokens)
size_t block_major_scratch_bytes(int num_seqs, int q_len);
hipError_t launch_block_major_attn(const AttnArgs& a, int num_seqs, void* scratch, hipStream_t stream);

// Write side: new tokens quantised into the paged pools (one launch).
struct InsertArgs {
  uint8_t* k;                  // NVFP4 [P][4][128][64] or bf16 [P][4][128][128]
  uint8_t* v;
  uint8_t* k_sf;               // NVFP4: [P][4][128][8]
  uint8_t* v_sf;
  uint8_t* idx;                // FP8 [P][128][128], bf16 [P][128][128] or NVFP4 [P][128][64]
  uint8_t* idx_sf;             // NVFP4 index keys: [P][128][8]
  const int32_t* block_table;
  const int32_t* seq_lens;
  const uint16_t* k_new;       // bf16 [rows][4][128]
  const uint16_t* v_new;
  const uint16_t* idx_new;     // bf16 [rows][128]
  int rows;
  int q_len;
  int mbps;
  float k_scale;
  float v_scale;
  float idx_scale;
  bool kv_nvfp4;
  int idx_fmt;                 // IdxFormat
};
hipError_t launch_kv_insert(const InsertArgs& a, hipStream_t stream);

// Compute units of the current device (cached per device).
int device_cus();

}  // namespace msa
