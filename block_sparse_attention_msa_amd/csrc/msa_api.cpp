// msa_api.cpp - C ABI of the MSA decode path: host-side validation, workspace
// layout and launch orchestration.  Every argument is checked before the first
// HIP call, so invalid calls return without touching the device.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "msa.h"
#include "msa_kernels.hpp"

static_assert(MSA_MAX_BLOCKS_PER_SEQ == msa::kMaxBlocksPerSeq, "block limit mismatch");
static_assert(MSA_BLOCK_SIZE == msa::kBlock && MSA_HEAD_DIM == msa::kDim && MSA_INDEX_DIM == msa::kDim,
              "geometry mismatch");
static_assert(MSA_TOPK == msa::kTopK && MSA_NUM_KV_HEADS == msa::kGroups &&
                  MSA_NUM_Q_HEADS == msa::kGroups * msa::kHeadsPerGroup,
              "head geometry mismatch");

namespace {

thread_local char g_last_error[512] = "";

msa_status fail(msa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

msa_status ok() {
  g_last_error[0] = '\0';
  return MSA_OK;
}

bool finite_pos(float x) { return isfinite(x) && x > 0.f; }

msa_status check_shape(const msa_shape* s) {
  if (!s) return fail(MSA_ERR_INVALID_ARGUMENT, "shape is NULL");
  if (s->num_seqs < 0) return fail(MSA_ERR_INVALID_ARGUMENT, "num_seqs = %d < 0", s->num_seqs);
  if (s->q_len < 1) return fail(MSA_ERR_INVALID_ARGUMENT, "q_len = %d < 1", s->q_len);
  if (s->num_kv_heads != MSA_NUM_KV_HEADS)
    return fail(MSA_ERR_UNSUPPORTED, "num_kv_heads = %d (only %d supported)", s->num_kv_heads, MSA_NUM_KV_HEADS);
  if (s->num_q_heads != MSA_NUM_Q_HEADS)
    return fail(MSA_ERR_UNSUPPORTED, "num_q_heads = %d (only %d supported)", s->num_q_heads, MSA_NUM_Q_HEADS);
  if (s->max_blocks_per_seq < 1 || s->max_blocks_per_seq > MSA_MAX_BLOCKS_PER_SEQ)
    return fail(MSA_ERR_INVALID_ARGUMENT, "max_blocks_per_seq = %d outside [1, %d]", s->max_blocks_per_seq,
                MSA_MAX_BLOCKS_PER_SEQ);
  if (s->num_pages < 1) return fail(MSA_ERR_INVALID_ARGUMENT, "num_pages = %d < 1", s->num_pages);
  if (s->kv_dtype != MSA_KV_BF16 && s->kv_dtype != MSA_KV_NVFP4)
    return fail(MSA_ERR_UNSUPPORTED, "kv_dtype = %d", s->kv_dtype);
  if (s->idx_dtype != MSA_IDX_BF16 && s->idx_dtype != MSA_IDX_FP8_E4M3 && s->idx_dtype != MSA_IDX_NVFP4)
    return fail(MSA_ERR_UNSUPPORTED, "idx_dtype = %d", s->idx_dtype);
  if (!finite_pos(s->sm_scale) || !finite_pos(s->k_scale) || !finite_pos(s->v_scale) || !finite_pos(s->idx_scale))
    return fail(MSA_ERR_INVALID_ARGUMENT, "scales must be finite and > 0 (sm %g, k %g, v %g, idx %g)",
                (double)s->sm_scale, (double)s->k_scale, (double)s->v_scale, (double)s->idx_scale);
  if ((long long)s->q_len > (long long)s->max_blocks_per_seq * MSA_BLOCK_SIZE)
    return fail(MSA_ERR_INVALID_ARGUMENT, "q_len = %d exceeds the sequence capacity", s->q_len);
  if ((long long)s->num_seqs * s->q_len > 65535)
    return fail(MSA_ERR_UNSUPPORTED, "num_seqs * q_len = %lld rows > 65535", (long long)s->num_seqs * s->q_len);
  return MSA_OK;
}

msa_status check_cache(const msa_shape* s, const msa_cache* c, bool need_idx, bool need_kv) {
  if (!c) return fail(MSA_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (!c->block_table || !c->seq_lens) return fail(MSA_ERR_INVALID_ARGUMENT, "block_table / seq_lens is NULL");
  if (need_idx && !c->idx_k) return fail(MSA_ERR_INVALID_ARGUMENT, "idx_k is NULL");
  if (need_idx && s->idx_dtype == MSA_IDX_NVFP4 && !c->idx_sf)
    return fail(MSA_ERR_INVALID_ARGUMENT, "idx_sf is NULL for NVFP4 index keys");
  if (need_kv) {
    if (!c->k || !c->v) return fail(MSA_ERR_INVALID_ARGUMENT, "k / v is NULL");
    if (s->kv_dtype == MSA_KV_NVFP4 && (!c->k_sf || !c->v_sf))
      return fail(MSA_ERR_INVALID_ARGUMENT, "k_sf / v_sf is NULL for NVFP4 K/V");
  }
  return MSA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
size_t rows_of(const msa_shape* s) { return (size_t)s->num_seqs * (size_t)s->q_len; }
size_t scores_bytes(const msa_shape* s) { return rows_of(s) * MSA_NUM_KV_HEADS * (size_t)s->max_blocks_per_seq * 4; }
size_t sel_bytes(const msa_shape* s) { return rows_of(s) * MSA_NUM_KV_HEADS * (size_t)MSA_TOPK * 4; }

msa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

msa::AttnArgs attn_args(const msa_shape* s, const msa_cache* c, const void* q, const float* block_scores,
                        const int32_t* sel, int32_t* sel_out, float* out) {
  msa::AttnArgs a;
  a.k = c->k;
  a.v = c->v;
  a.k_sf = c->k_sf;
  a.v_sf = c->v_sf;
  a.block_table = c->block_table;
  a.seq_lens = c->seq_lens;
  a.q = static_cast<const uint16_t*>(q);
  a.block_scores = block_scores;
  a.sel = sel;
  a.sel_out = sel_out;
  a.out = out;
  a.rows = (int)rows_of(s);
  a.q_len = s->q_len;
  a.mbps = s->max_blocks_per_seq;
  a.qk_scale_log2 = (float)((double)s->sm_scale * (double)s->k_scale * 1.4426950408889634);
  a.v_scale = s->v_scale;
  a.kv_nvfp4 = s->kv_dtype == MSA_KV_NVFP4;
  return a;
}

msa::ScanArgs scan_args(const msa_shape* s, const msa_cache* c, const void* idx_q, float* block_scores) {
  msa::ScanArgs a;
  a.idx_pool = c->idx_k;
  a.block_table = c->block_table;
  a.seq_lens = c->seq_lens;
  a.iq = static_cast<const uint16_t*>(idx_q);
  a.block_scores = block_scores;
  a.num_seqs = s->num_seqs;
  a.mbps = s->max_blocks_per_seq;
  a.idx_scale = s->idx_scale;
  a.idx_sf = c->idx_sf;
  a.idx_fmt = s->idx_dtype == MSA_IDX_NVFP4 ? msa::kIdxNvfp4 : s->idx_dtype == MSA_IDX_FP8_E4M3 ? msa::kIdxFp8 : msa::kIdxBf16;
  return a;
}

// q_len == 1: the decode scan; FP8 or NVFP4 index keys with q_len <= 8: pages
// streamed by waves with the few (query, group) columns on MFMA; otherwise
// the multi-query scan (query rows staged in LDS, keys streamed per row
// chunk and converted to bf16 once per workgroup).
hipError_t launch_scan(const msa_shape* s, const msa::ScanArgs& a, hipStream_t stream) {
  if (s->q_len == 1) return msa::launch_scan_decode(a, stream);
  if (a.idx_fmt != msa::kIdxBf16 && s->q_len <= 8) return msa::launch_scan_cols(a, s->q_len, stream);
  return msa::launch_scan_mq(a, s->q_len, stream);
}

static_assert(msa::kShareMax == MSA_SHARE_MAX, "one member limit on both sides of the boundary");

msa_status check_share(const msa_shape* s, const msa_prefix_share* sh) {
  if (!sh) return fail(MSA_ERR_INVALID_ARGUMENT, "share is NULL");
  if (sh->num_groups < 0) return fail(MSA_ERR_INVALID_ARGUMENT, "share num_groups = %d < 0", sh->num_groups);
  if (sh->num_groups == 0) return MSA_OK;
  if (!sh->members || !sh->shared_blocks || !sh->seq_shared_blocks)
    return fail(MSA_ERR_INVALID_ARGUMENT, "share members / shared_blocks / seq_shared_blocks is NULL");
  if (s->q_len > 8)
    return fail(MSA_ERR_UNSUPPORTED, "prefix sharing with q_len = %d (supported for q_len 1 to 8)", s->q_len);
  if (sh->max_members < 1 || sh->max_members > MSA_SHARE_MAX)
    return fail(MSA_ERR_INVALID_ARGUMENT, "share max_members = %d outside [1, %d]", sh->max_members, MSA_SHARE_MAX);
  if ((long long)sh->max_members * s->q_len > MSA_SHARE_MAX)
    return fail(MSA_ERR_UNSUPPORTED, "share max_members x q_len = %lld > %d (query columns per shared page)",
                (long long)sh->max_members * s->q_len, MSA_SHARE_MAX);
  if (s->idx_dtype == MSA_IDX_BF16)
    return fail(MSA_ERR_UNSUPPORTED, "prefix sharing with bf16 index keys (supported for FP8 and NVFP4)");
  if (sh->min_shared_blocks < 0 || sh->min_shared_blocks >= s->max_blocks_per_seq)
    return fail(MSA_ERR_INVALID_ARGUMENT, "share min_shared_blocks = %d outside [0, %d)", sh->min_shared_blocks,
                s->max_blocks_per_seq);
  const long long xs = (s->max_blocks_per_seq + 7) / 8, xo = (s->max_blocks_per_seq - sh->min_shared_blocks + 7) / 8;
  if (sh->num_groups * xs + (long long)s->num_seqs * xo > 0x7fffffffLL)
    return fail(MSA_ERR_UNSUPPORTED, "share: %d groups and %d sequences need too many workgroups", sh->num_groups,
                s->num_seqs);
  return MSA_OK;
}

// The index scan, with prefix sharing when share has groups (one launch: each
// group's shared blocks once, every sequence's own blocks).
hipError_t launch_scan_any(const msa_shape* s, const msa::ScanArgs& a, const msa_prefix_share* share,
                           hipStream_t stream) {
  if (!share || share->num_groups == 0) return launch_scan(s, a, stream);
  return msa::launch_scan_shared(a, share->members, share->shared_blocks, share->seq_shared_blocks,
                                 share->num_groups, share->max_members, share->min_shared_blocks, s->q_len, stream);
}

msa_status check_aligned(const void* p, size_t a, const char* what) {
  if (((uintptr_t)p) % a) return fail(MSA_ERR_INVALID_ARGUMENT, "%s must be %zu-byte aligned", what, a);
  return MSA_OK;
}

// The group-scale arrays are read with 16-byte vector loads (a page's scales
// are whole 1 KB runs), so their base pointers must be 16-byte aligned.
msa_status check_scale_alignment(const msa_shape* s, const msa_cache* c, bool need_idx, bool need_kv) {
  msa_status st = MSA_OK;
  if (need_kv && s->kv_dtype == MSA_KV_NVFP4) {
    if ((st = check_aligned(c->k_sf, 16, "k_sf")) != MSA_OK) return st;
    if ((st = check_aligned(c->v_sf, 16, "v_sf")) != MSA_OK) return st;
  }
  if (need_idx && s->idx_dtype == MSA_IDX_NVFP4 && (st = check_aligned(c->idx_sf, 16, "idx_sf")) != MSA_OK) return st;
  return MSA_OK;
}

msa_status check_block_major(const msa_shape* s) {
  if (s->kv_dtype != MSA_KV_NVFP4) return fail(MSA_ERR_UNSUPPORTED, "block-major attention needs NVFP4 K/V");
  if (s->q_len > msa::kBmMaxQ)
    return fail(MSA_ERR_UNSUPPORTED, "block-major attention with q_len = %d (at most %d)", s->q_len, msa::kBmMaxQ);
  if (s->max_blocks_per_seq > msa::kBmMaxBlocks)
    return fail(MSA_ERR_UNSUPPORTED, "block-major attention with max_blocks_per_seq = %d (at most %d)",
                s->max_blocks_per_seq, msa::kBmMaxBlocks);
  return MSA_OK;
}

// ---- static scratch of the allocation-free entry point --------------------
// The workspace of msa_decode_noalloc: a file-scope device array, one copy per
// GPU the library runs on, held until the process ends.  Host code never uses
// the array's name as an address (on the host it is only a stand-in symbol):
// each device's own address is looked up once with hipGetSymbolAddress, with
// that device current, and that pointer is what the kernels receive.
constexpr size_t kScratchBytes = (size_t)MSA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's address of `scratch` (looked up on the first call per device).
msa_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MSA_ERR_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MSA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MSA_OK;
}

}  // namespace

extern "C" {

size_t msa_attn_workspace_size(const msa_shape* shape) {
  if (check_shape(shape) != MSA_OK) return 0;
  // the kept-block split's partials (bf16 K/V, few (row, group) pairs);
  // otherwise the attention merges its split work on chip
  return align256(msa::split_partials_bytes(rows_of(shape) * (long long)MSA_NUM_KV_HEADS,
                                            shape->kv_dtype == MSA_KV_NVFP4));
}

size_t msa_workspace_size(const msa_shape* shape) {
  if (check_shape(shape) != MSA_OK) return 0;
  return align256(scores_bytes(shape)) + align256(sel_bytes(shape)) +
         align256(msa::split_partials_bytes(rows_of(shape) * (long long)MSA_NUM_KV_HEADS,
                                            shape->kv_dtype == MSA_KV_NVFP4));
}

static msa_status indexer_impl(const msa_shape* shape, const msa_cache* cache, const msa_prefix_share* share,
                               const void* idx_q, float* block_scores, hipStream_t stream) {
  msa_status st = check_shape(shape);
  if (st != MSA_OK) return st;
  if ((st = check_cache(shape, cache, true, false)) != MSA_OK) return st;
  if (share && (st = check_share(shape, share)) != MSA_OK) return st;
  if (!idx_q || !block_scores) return fail(MSA_ERR_INVALID_ARGUMENT, "idx_q / block_scores is NULL");
  if ((st = check_aligned(cache->idx_k, 16, "idx_k")) != MSA_OK) return st;
  if ((st = check_aligned(idx_q, 16, "idx_q")) != MSA_OK) return st;
  if ((st = check_scale_alignment(shape, cache, true, false)) != MSA_OK) return st;
  if (shape->num_seqs == 0) return ok();
  return hip_status(launch_scan_any(shape, scan_args(shape, cache, idx_q, block_scores), share, stream), "index scan");
}

msa_status msa_indexer_score(const msa_shape* shape, const msa_cache* cache, const void* idx_q, float* block_scores,
                             hipStream_t stream) {
  return indexer_impl(shape, cache, nullptr, idx_q, block_scores, stream);
}

msa_status msa_indexer_score_shared(const msa_shape* shape, const msa_cache* cache, const msa_prefix_share* share,
                                    const void* idx_q, float* block_scores, hipStream_t stream) {
  if (!share) return fail(MSA_ERR_INVALID_ARGUMENT, "share is NULL");
  return indexer_impl(shape, cache, share, idx_q, block_scores, stream);
}

msa_status msa_block_topk(const msa_shape* shape, const int32_t* seq_lens, const float* block_scores,
                          int32_t* sel_blocks, hipStream_t stream) {
  msa_status st = check_shape(shape);
  if (st != MSA_OK) return st;
  if (!seq_lens || !block_scores || !sel_blocks)
    return fail(MSA_ERR_INVALID_ARGUMENT, "seq_lens / block_scores / sel_blocks is NULL");
  if (shape->num_seqs == 0) return ok();
  msa::TopkArgs a{seq_lens, block_scores, sel_blocks, (int)rows_of(shape), shape->q_len, shape->max_blocks_per_seq};
  return hip_status(msa::launch_block_topk(a, stream), "block top-k");
}

msa_status msa_sparse_attn_decode(const msa_shape* shape, const msa_cache* cache, const void* q,
                                  const int32_t* sel_blocks, float* out, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  msa_status st = check_shape(shape);
  if (st != MSA_OK) return st;
  if ((st = check_cache(shape, cache, false, true)) != MSA_OK) return st;
  if (!q || !sel_blocks || !out) return fail(MSA_ERR_INVALID_ARGUMENT, "q / sel_blocks / out is NULL");
  if ((st = check_aligned(q, 16, "q")) != MSA_OK) return st;
  if ((st = check_aligned(cache->k, 16, "k")) != MSA_OK) return st;
  if ((st = check_aligned(cache->v, 16, "v")) != MSA_OK) return st;
  if ((st = check_aligned(out, 16, "out")) != MSA_OK) return st;
  if ((st = check_scale_alignment(shape, cache, false, true)) != MSA_OK) return st;
  if (shape->num_seqs == 0) return ok();
  const size_t need = msa_attn_workspace_size(shape);
  msa::AttnArgs a = attn_args(shape, cache, q, nullptr, sel_blocks, nullptr, out);
  if (need > 0) {  // few pairs: the kept-block split, as in msa_decode
    if (!workspace) return fail(MSA_ERR_INVALID_ARGUMENT, "workspace is NULL");
    if ((st = check_aligned(workspace, 256, "workspace")) != MSA_OK) return st;
    if (workspace_bytes < need)
      return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu B < %zu B needed", workspace_bytes, need);
    a.partials = static_cast<float*>(workspace);
  }
  return hip_status(msa::launch_sparse_attn(a, stream), "sparse attention");
}

static msa_status decode_impl(const msa_shape* shape, const msa_cache* cache, const msa_prefix_share* share,
                              const void* q, const void* idx_q, float* out, int32_t* sel_blocks, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  msa_status st = check_shape(shape);
  if (st != MSA_OK) return st;
  if ((st = check_cache(shape, cache, true, true)) != MSA_OK) return st;
  if (share && (st = check_share(shape, share)) != MSA_OK) return st;
  if (!q || !idx_q || !out) return fail(MSA_ERR_INVALID_ARGUMENT, "q / idx_q / out is NULL");
  if ((st = check_aligned(q, 16, "q")) != MSA_OK) return st;
  if ((st = check_aligned(idx_q, 16, "idx_q")) != MSA_OK) return st;
  if ((st = check_aligned(cache->idx_k, 16, "idx_k")) != MSA_OK) return st;
  if ((st = check_aligned(cache->k, 16, "k")) != MSA_OK) return st;
  if ((st = check_aligned(cache->v, 16, "v")) != MSA_OK) return st;
  if ((st = check_aligned(out, 16, "out")) != MSA_OK) return st;
  if ((st = check_scale_alignment(shape, cache, true, true)) != MSA_OK) return st;
  const size_t need = msa_workspace_size(shape);
  if (shape->num_seqs > 0) {
    if (!workspace) return fail(MSA_ERR_INVALID_ARGUMENT, "workspace is NULL");
    if ((st = check_aligned(workspace, 256, "workspace")) != MSA_OK) return st;
    if (workspace_bytes < need)
      return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu B < %zu B needed", workspace_bytes, need);
  }
  if (shape->num_seqs == 0) return ok();

  // Index scan fused with the block max-pool, then either the selection fused
  // with the attention (each attention workgroup selects its (row, group): 2
  // launches), or, when the attention workgroups run in more than one round
  // (more (row, group) pairs than two per CU), the selection as a launch of
  // its own between them (3 launches), so that the per-workgroup selection
  // latency is not paid once per round.
  float* scores = static_cast<float*>(workspace);
  const long long pairs = (long long)rows_of(shape) * shape->num_kv_heads;
  const bool fused = pairs <= 2LL * msa::device_cus();
  msa::ScanArgs sa = scan_args(shape, cache, idx_q, scores);
  msa::AttnArgs a = attn_args(shape, cache, q, scores, nullptr, sel_blocks, out);
  if (fused && msa::split_partials_bytes(pairs, a.kv_nvfp4) > 0) {
    // few pairs, bf16 K/V: the kept-block split, its partials merged by the
    // last part of each pair; the scan zeroes the arrival counters
    a.partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + align256(scores_bytes(shape)) +
                                          align256(sel_bytes(shape)));
    a.counters = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(a.partials) + msa::split_counters_offset(pairs));
    sa.zero = a.counters;
    sa.zero_n = (int)pairs;
  }
  hipError_t e = launch_scan_any(shape, sa, share, stream);
  if (e != hipSuccess) return hip_status(e, "index scan");
  if (fused) return hip_status(msa::launch_sparse_attn(a, stream), "selection + sparse attention");
  int32_t* sel = sel_blocks ? sel_blocks
                            : reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + align256(scores_bytes(shape)));
  msa::TopkArgs ta{cache->seq_lens, scores, sel, (int)rows_of(shape), shape->q_len, shape->max_blocks_per_seq};
  if ((e = msa::launch_block_topk(ta, stream)) != hipSuccess) return hip_status(e, "block top-k");
  return hip_status(msa::launch_sparse_attn(attn_args(shape, cache, q, nullptr, sel, nullptr, out), stream),
                    "sparse attention");
}

msa_status msa_decode(const msa_shape* shape, const msa_cache* cache, const void* q, const void* idx_q, float* out,
                      int32_t* sel_blocks, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_impl(shape, cache, nullptr, q, idx_q, out, sel_blocks, workspace, workspace_bytes, stream);
}

msa_status msa_decode_noalloc(const msa_shape* shape, const msa_cache* cache, const void* q, const void* idx_q,
                              float* out, int32_t* sel_blocks, hipStream_t stream) {
  msa_status st = check_shape(shape);
  if (st != MSA_OK) return st;
  const size_t need = msa_workspace_size(shape);
  if (need > kScratchBytes)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL,
                "msa_decode_noalloc: this shape needs %zu B of scratch, the static scratch holds %zu B "
                "(use msa_decode with a caller workspace)", need, kScratchBytes);
  if (shape->num_seqs == 0) return decode_impl(shape, cache, nullptr, q, idx_q, out, sel_blocks, nullptr, 0, stream);
  // the arguments are validated before the scratch lookup (the first HIP call)
  if ((st = check_cache(shape, cache, true, true)) != MSA_OK) return st;
  if (!q || !idx_q || !out) return fail(MSA_ERR_INVALID_ARGUMENT, "q / idx_q / out is NULL");
  void* ws = nullptr;
  if ((st = scratch_for_current_device(&ws)) != MSA_OK) return st;
  return decode_impl(shape, cache, nullptr, q, idx_q, out, sel_blocks, ws, kScratchBytes, stream);
}

size_t msa_block_major_workspace_size(const msa_shape* shape) {
  if (check_shape(shape) != MSA_OK || check_block_major(shape) != MSA_OK) return 0;
  return align256(scores_bytes(shape)) + align256(sel_bytes(shape)) +
         msa::block_major_scratch_bytes(shape->num_seqs, shape->q_len);
}

msa_status msa_decode_block_major(const msa_shape* shape, const msa_cache* cache, const void* q, const void* idx_q,
                                  float* out, int32_t* sel_blocks, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  msa_status st = check_shape(shape);
  if (st != MSA_OK) return st;
  if ((st = check_block_major(shape)) != MSA_OK) return st;
  if ((st = check_cache(shape, cache, true, true)) != MSA_OK) return st;
  if (!q || !idx_q || !out) return fail(MSA_ERR_INVALID_ARGUMENT, "q / idx_q / out is NULL");
  const void* aligned16[] = {q, idx_q, cache->idx_k, cache->k, cache->v, out};
  const char* names[] = {"q", "idx_q", "idx_k", "k", "v", "out"};
  for (int i = 0; i < 6; ++i)
    if ((st = check_aligned(aligned16[i], 16, names[i])) != MSA_OK) return st;
  if ((st = check_scale_alignment(shape, cache, true, true)) != MSA_OK) return st;
  if (shape->num_seqs == 0) return ok();
  const size_t need = msa_block_major_workspace_size(shape);
  if (!workspace) return fail(MSA_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if ((st = check_aligned(workspace, 256, "workspace")) != MSA_OK) return st;
  if (workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu B < %zu B needed", workspace_bytes, need);
  // index scan + block max-pool, the stand-alone selection, then the
  // block-major attention (inversion, partials, merge)
  char* ws = static_cast<char*>(workspace);
  float* scores = reinterpret_cast<float*>(ws);
  int32_t* sel = sel_blocks ? sel_blocks : reinterpret_cast<int32_t*>(ws + align256(scores_bytes(shape)));
  void* scratch = ws + align256(scores_bytes(shape)) + align256(sel_bytes(shape));
  hipError_t e = launch_scan(shape, scan_args(shape, cache, idx_q, scores), stream);
  if (e != hipSuccess) return hip_status(e, "index scan");
  msa::TopkArgs ta{cache->seq_lens, scores, sel, (int)rows_of(shape), shape->q_len, shape->max_blocks_per_seq};
  if ((e = msa::launch_block_topk(ta, stream)) != hipSuccess) return hip_status(e, "block top-k");
  return hip_status(msa::launch_block_major_attn(attn_args(shape, cache, q, nullptr, sel, nullptr, out),
                                                 shape->num_seqs, scratch, stream),
                    "block-major attention");
}

msa_status msa_decode_shared(const msa_shape* shape, const msa_cache* cache, const msa_prefix_share* share,
                             const void* q, const void* idx_q, float* out, int32_t* sel_blocks, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  if (!share) return fail(MSA_ERR_INVALID_ARGUMENT, "share is NULL");
  return decode_impl(shape, cache, share, q, idx_q, out, sel_blocks, workspace, workspace_bytes, stream);
}

msa_status msa_kv_insert(const msa_shape* shape, const msa_cache* cache, const void* k_new, const void* v_new,
                         const void* idx_new, hipStream_t stream) {
  msa_status st = check_shape(shape);
  if (st != MSA_OK) return st;
  if ((st = check_cache(shape, cache, true, true)) != MSA_OK) return st;
  if (!k_new || !v_new || !idx_new) return fail(MSA_ERR_INVALID_ARGUMENT, "k_new / v_new / idx_new is NULL");
  const void* aligned16[] = {k_new, v_new, idx_new, cache->k, cache->v, cache->idx_k};
  const char* names[] = {"k_new", "v_new", "idx_new", "k", "v", "idx_k"};
  for (int i = 0; i < 6; ++i)
    if ((st = check_aligned(aligned16[i], 16, names[i])) != MSA_OK) return st;
  if ((st = check_scale_alignment(shape, cache, true, true)) != MSA_OK) return st;
  if (shape->num_seqs == 0) return ok();
  msa::InsertArgs a;
  // the pools are written: the cache's pointers are taken as writable
  a.k = static_cast<uint8_t*>(const_cast<void*>(cache->k));
  a.v = static_cast<uint8_t*>(const_cast<void*>(cache->v));
  a.k_sf = const_cast<uint8_t*>(cache->k_sf);
  a.v_sf = const_cast<uint8_t*>(cache->v_sf);
  a.idx = static_cast<uint8_t*>(const_cast<void*>(cache->idx_k));
  a.idx_sf = const_cast<uint8_t*>(cache->idx_sf);
  a.block_table = cache->block_table;
  a.seq_lens = cache->seq_lens;
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.idx_new = static_cast<const uint16_t*>(idx_new);
  a.rows = (int)rows_of(shape);
  a.q_len = shape->q_len;
  a.mbps = shape->max_blocks_per_seq;
  a.k_scale = shape->k_scale;
  a.v_scale = shape->v_scale;
  a.idx_scale = shape->idx_scale;
  a.kv_nvfp4 = shape->kv_dtype == MSA_KV_NVFP4;
  a.idx_fmt = shape->idx_dtype == MSA_IDX_NVFP4 ? msa::kIdxNvfp4 : shape->idx_dtype == MSA_IDX_FP8_E4M3 ? msa::kIdxFp8 : msa::kIdxBf16;
  return hip_status(msa::launch_kv_insert(a, stream), "kv insert");
}

const char* msa_status_string(msa_status status) {
  switch (status) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_INVALID_ARGUMENT: return "MSA_ERR_INVALID_ARGUMENT";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED";
    case MSA_ERR_WORKSPACE_TOO_SMALL: return "MSA_ERR_WORKSPACE_TOO_SMALL";
    case MSA_ERR_HIP: return "MSA_ERR_HIP";
  }
  return "MSA_ERR_UNKNOWN";
}

const char* msa_last_error(void) { return g_last_error; }

}  // extern "C"
