/*
 * msa.h - C ABI of the MI355X (gfx950) MiniMax Sparse Attention decode path.
 *
 * The method (vLLM "Day-0 support for MiniMax-M3.1-Flash", section "MSA
 * basics"; "MiniMax M3 x vLLM", sections "MSA mechanism details", "MiniMax
 * sparse attention backend", "Decode execution" and "KV cache layout"):
 * the KV cache is cut into 128-token blocks; a lightweight indexer scores
 * every context key with one index query per GQA group against one shared
 * 128-dim index-key head; the scores are max-pooled to one score per block;
 * per group the most recent block plus the 15 best other blocks are kept
 * (at most 16 x 128 = 2,048 keys); exact GQA attention then runs over only
 * the kept keys.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    allocates nothing, keeps no state between calls and never synchronises:
 *    work is enqueued on `stream` and results are valid once the stream has
 *    reached that point.  Launch grids depend only on the host-side shape, so
 *    calls can be captured into HIP graphs.
 *  - Host arguments are validated before any HIP call.  Failures return
 *    MSA_ERR_INVALID_ARGUMENT / MSA_ERR_UNSUPPORTED / MSA_ERR_WORKSPACE_TOO_SMALL
 *    with a message in msa_last_error(); nothing is launched then.  A launch
 *    failure returns MSA_ERR_HIP.
 *  - Device-resident values are preconditions, not checked: for every sequence
 *    b, 0 <= seq_lens[b] <= max_blocks_per_seq * 128 and seq_lens[b] is 0 or
 *    >= q_len; block_table[b][j] lies in [0, num_pages) for every block j that
 *    holds a visible token.  A sequence with seq_lens[b] == 0 is a padded row:
 *    its block scores are -inf, its selected ids -1 and its output 0.
 *  - Query rows are flattened request-major: row = b * q_len + i, and row i of
 *    sequence b sits at position seq_lens[b] - q_len + i (its own K/V and index
 *    key are already in the cache, so it attends to itself).
 *  - Block ids are LOGICAL block indices of the sequence (block j holds tokens
 *    128 j .. 128 j + 127), never physical pages.
 *
 * Stored formats
 *  - q      bf16 [rows][num_q_heads][128]; iq bf16 [rows][num_kv_heads][128].
 *  - idx_k  index-key pool, one shared head: FP8 E4M3 (OCP, bias 7) bytes
 *           [num_pages][128 tokens][128], or bf16 [num_pages][128][128];
 *           value = stored x idx_scale.  NVFP4 ("NVFP4 indexer DCP" of the
 *           M3.1 post: the index cache in NVFP4, 72 B per token): uint8
 *           [num_pages][128 tokens][64] (element 2i in the low nibble of byte
 *           i, E2M1) plus idx_sf uint8 E4M3 [num_pages][128 tokens][8];
 *           value = e2m1 x scale x idx_scale.
 *  - k      NVFP4: uint8 [num_pages][num_kv_heads][128 tokens][64], element 2i
 *           in the low nibble of byte i (E2M1), plus k_sf uint8 E4M3
 *           [num_pages][num_kv_heads][128 tokens][8] (one scale per 16
 *           consecutive elements); value = e2m1 x scale x k_scale.
 *  - v      NVFP4, stored by dim: uint8 [num_pages][num_kv_heads][128 dims][64],
 *           row d holding dim d of the page's 128 tokens, token 2i in the low
 *           nibble of byte i (E2M1), plus v_sf as k_sf (one scale per token
 *           and 16 consecutive dims); value = e2m1 x scale x v_scale.  (The
 *           attention's PV contraction runs over tokens, so a dim's tokens are
 *           contiguous here.)
 *  - k, v   bf16: [num_pages][num_kv_heads][128][128], value = stored x scale.
 *  - block_table int32 [num_seqs][max_blocks_per_seq]; seq_lens int32 [num_seqs].
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

/* hipStream_t.  C callers compile with ROCm's include directory and
 * -D__HIP_PLATFORM_AMD__ (hipcc sets both); the header is C99. */
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_BLOCK_SIZE 128    /* tokens per KV block (one page)              */
#define MSA_HEAD_DIM 128      /* q / k / v head dimension                    */
#define MSA_INDEX_DIM 128     /* index query / index key dimension           */
#define MSA_TOPK 16           /* kept blocks per (query, group), recent incl. */
#define MSA_NUM_KV_HEADS 4    /* GQA groups = KV heads = index queries/token */
#define MSA_NUM_Q_HEADS 16    /* query heads (4 per group)                   */
#define MSA_MAX_BLOCKS_PER_SEQ 16384 /* 2M tokens                            */

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARGUMENT = 1,
  MSA_ERR_UNSUPPORTED = 2,
  MSA_ERR_WORKSPACE_TOO_SMALL = 3,
  MSA_ERR_HIP = 4
} msa_status;

typedef enum { MSA_KV_BF16 = 0, MSA_KV_NVFP4 = 1 } msa_kv_dtype;
typedef enum { MSA_IDX_BF16 = 0, MSA_IDX_FP8_E4M3 = 1, MSA_IDX_NVFP4 = 2 } msa_idx_dtype;

/* Host-side problem shape; read only during the call. */
typedef struct {
  int32_t num_seqs;           /* S >= 0 (0: nothing to do)                          */
  int32_t q_len;              /* query tokens per sequence; 1 = decode              */
  int32_t num_q_heads;        /* must be MSA_NUM_Q_HEADS                            */
  int32_t num_kv_heads;       /* must be MSA_NUM_KV_HEADS                           */
  int32_t max_blocks_per_seq; /* row stride of block_table, 1..MSA_MAX_BLOCKS_PER_SEQ */
  int32_t num_pages;          /* pool size P >= 1                                   */
  int32_t kv_dtype;           /* msa_kv_dtype                                       */
  int32_t idx_dtype;          /* msa_idx_dtype                                      */
  float sm_scale;             /* softmax logit scale (normally 1/sqrt(128)), > 0    */
  float k_scale, v_scale;     /* K / V tensor scales, > 0                           */
  float idx_scale;            /* index-key tensor scale, > 0                        */
} msa_shape;

/* Paged caches: device pointers, caller-owned, layouts as above. */
typedef struct {
  const void* k;
  const void* v;
  const uint8_t* k_sf;        /* NVFP4 only; NULL for bf16 */
  const uint8_t* v_sf;        /* NVFP4 only; NULL for bf16 */
  const void* idx_k;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const uint8_t* idx_sf;      /* NVFP4 index keys only; NULL otherwise */
} msa_cache;

/* Bytes of device workspace msa_decode needs for this shape: the fp32 block
 * scores [rows][num_kv_heads][max_blocks_per_seq], then the int32 selected
 * ids [rows][num_kv_heads][16] (used when sel_blocks is NULL and the
 * selection runs as a launch of its own), then, with bf16 K/V and at most 64
 * (row, group) pairs (rows x num_kv_heads), the partial outputs of the
 * kept-block split (2,080 B per (pair, kept block)) and one int32 arrival
 * counter per pair, each part 256-B aligned.  Its contents need no
 * initialisation: msa_decode's first launch zeroes the counters.  Returns 0 for an invalid shape (see
 * msa_last_error()).  msa_attn_workspace_size(): the stand-alone attention's
 * workspace, the same partials for bf16 K/V and at most 64 pairs (it then
 * splits the kept blocks as msa_decode does), 0 otherwise (it merges its split
 * work on chip). */
size_t msa_workspace_size(const msa_shape* shape);
size_t msa_attn_workspace_size(const msa_shape* shape);

/* Steps 1-2 of the method ("MSA basics": index scores against the shared
 * index-key head, max-pooled per 128-token block; "Decode indexer-score
 * kernel" of the M3 post: a dedicated scan, not a padded dense GEMM).
 *   idx_q        bf16 [rows][num_kv_heads][128]
 *   block_scores fp32 [rows][num_kv_heads][max_blocks_per_seq], written in
 *                full: for the row's visible blocks j <= pos/128,
 *                idx_scale * max over tokens t <= pos of block j of
 *                sum_d idx_q[row][g][d] * idx_k[t][d]; -inf elsewhere.
 * fp32 accumulation; products are exact in fp32. */
msa_status msa_indexer_score(const msa_shape* shape, const msa_cache* cache, const void* idx_q,
                             float* block_scores, hipStream_t stream);

/* Step 3 ("MSA basics": top-16 blocks with the most recent one always kept;
 * "MSA mechanism details": init_blocks = 0, local_blocks = 1, a local block
 * that also wins top-k is not counted twice).
 *   seq_lens     int32 [num_seqs] (device)
 *   block_scores fp32 [rows][num_kv_heads][max_blocks_per_seq] (device)
 *   sel_blocks   int32 [rows][num_kv_heads][16]: with r = pos/128 the recent
 *                block, all of 0..r if r < 16, else r plus the 15 blocks j < r
 *                first under (score descending, index ascending); ascending,
 *                padded with -1. */
msa_status msa_block_topk(const msa_shape* shape, const int32_t* seq_lens, const float* block_scores,
                          int32_t* sel_blocks, hipStream_t stream);

/* Step 4 ("MSA basics": exact attention over the kept blocks only; "Prefill
 * execution" step 4 of the M3 post: equal to dense attention restricted to
 * the selected set; "Decode sparse GQA": split work, partial outputs merged).
 *   q          bf16 [rows][num_q_heads][128]; head h uses KV head h / 4
 *   sel_blocks int32 [rows][num_kv_heads][16] logical ids (-1 = none)
 *   out        fp32 [rows][num_q_heads][128], 16-B aligned
 *   workspace  >= msa_attn_workspace_size(shape) bytes, 256-B aligned; may be
 *              NULL when that is 0 (NVFP4 K/V, or more than 64 (row, group)
 *              pairs)
 * Keys: tokens t <= pos of the listed blocks; logits sm_scale * q.k.  Ids
 * outside [0, pos/128] contribute nothing; a row left with no keys outputs 0. */
msa_status msa_sparse_attn_decode(const msa_shape* shape, const msa_cache* cache, const void* q,
                                  const int32_t* sel_blocks, float* out, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* The fused path: steps 1-4 in one call, no host synchronisation: the index
 * scan fused with the block max-pool, then the selection fused with the
 * attention (two launches), or, when there are more (row, group) pairs than
 * two per compute unit (the attention workgroups would run in several
 * rounds), the selection as a launch of its own before the attention (three
 * launches).  With bf16 K/V and at most 64 (row, group) pairs the kept blocks
 * of each pair are instead split over 2-16 workgroups ("Decode sparse GQA" of
 * the MiniMax M3 x vLLM post: split work, partial outputs merged), each
 * repeating the selection; the last workgroup of a pair to finish merges the
 * pair's partials by log-sum-exp (still two launches; msa_sparse_attn_decode
 * merges them in a second launch of its own, with the same arithmetic).
 * Results are the same in every form up to fp32 summation order (the ids are
 * identical).
 *   out        fp32 [rows][num_q_heads][128], 16-B aligned.
 *   sel_blocks int32 [rows][num_kv_heads][16], or NULL if not wanted.
 *   workspace  >= msa_workspace_size(shape) bytes, 256-B aligned. */
msa_status msa_decode(const msa_shape* shape, const msa_cache* cache, const void* q, const void* idx_q, float* out,
                      int32_t* sel_blocks, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The fused path with KV-block-major attention for multi-query rows ("KV-
 * block-major prefill" of the MiniMax M3 x vLLM post: the per-query block
 * lists are inverted into per-block query lists, each selected block is
 * loaded and dequantised once for all the queries of its (sequence, group)
 * that chose it, and every query's per-block partials are merged by
 * log-sum-exp).  Steps: the index scan, the stand-alone selection, the
 * inversion, the block-major partials (each block's K and V dequantised once
 * per work item of up to 16 rows), the merge: five launches.  Results: ids as
 * msa_decode's (the same selection); outputs equal the same exact attention
 * to fp32 rounding (another summation order than msa_decode's).  It pays off
 * when many rows of a chunk select the same blocks; with rows that select
 * mostly different blocks msa_decode's per-row attention is faster.
 * Supported: NVFP4 K/V, q_len <= 256, max_blocks_per_seq <= 8192
 * (MSA_ERR_UNSUPPORTED otherwise).
 *   out       as in msa_decode, 16-B aligned (the merge stores float4s).
 *   workspace >= msa_block_major_workspace_size(shape) bytes, 256-B aligned
 *             (block scores, ids, inverted lists, per-(row, slot) partials:
 *             about 133 KB per query row); no initialisation needed.
 * Other arguments as in msa_decode. */
size_t msa_block_major_workspace_size(const msa_shape* shape);
msa_status msa_decode_block_major(const msa_shape* shape, const msa_cache* cache, const void* q, const void* idx_q,
                                  float* out, int32_t* sel_blocks, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* msa_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same launches, with the workspace taken from a
 * static device array of MSA_NOALLOC_SCRATCH_BYTES (32 MiB) that the library
 * holds on each GPU it runs on until the process ends.  Nothing is allocated
 * and nothing in the scratch needs clearing (every byte a step reads is
 * written earlier in that step).  Shapes whose msa_workspace_size() exceeds
 * the scratch return MSA_ERR_WORKSPACE_TOO_SMALL before any launch (the
 * block scores take 16 B per (row, block of the table row), so 32 MiB holds
 * rows x max_blocks_per_seq up to about 2M: e.g. batch 64 at 2M tokens per
 * sequence, or 256 query rows at 512K).  Every call on one GPU shares its scratch:
 * calls that may overlap on that GPU (other streams, other host threads)
 * race and must be ordered by the caller.  The first call on a device looks
 * up its copy of the scratch (hipGetSymbolAddress); other arguments as in
 * msa_decode. */
#define MSA_NOALLOC_SCRATCH_BYTES (32u << 20)
msa_status msa_decode_noalloc(const msa_shape* shape, const msa_cache* cache, const void* q, const void* idx_q,
                              float* out, int32_t* sel_blocks, hipStream_t stream);

/* The write side of a decode step ("Decode execution" of the M3 post: the
 * step updates the cache before scoring; "What is new in M3.1": NVFP4 K/V,
 * E2M1 values with one E4M3 scale per 16 elements and a tensor scale): the
 * new tokens of every query row are quantised into the pools of `cache`,
 * which are WRITTEN through its pointers.  Row (b, i) goes to position
 * seq_lens[b] - q_len + i (seq_lens already counting the new tokens): token
 * row pos % 128 of page block_table[b][pos / 128], which must be allocated.
 * Padded rows (seq_lens[b] == 0) write nothing; nothing else is touched.
 *   k_new, v_new bf16 [rows][num_kv_heads][128]; idx_new bf16 [rows][128].
 * Quantiser, per group of 16 values x with tensor scale gs (k_scale, v_scale,
 * idx_scale): s = E4M3 nearest-even of amax|x| / (6 gs) (at most 448),
 * code_i = E2M1 nearest-even of x_i / (s gs) saturating at +-6 (zero as +0);
 * amax 0 or s == 0 store scale 0 and codes 0.  Each step is one fp32
 * operation in that order.  FP8 index keys: E4M3 nearest-even of
 * x / idx_scale clamped to +-448, sign kept on zero.  bf16 pools: bf16
 * nearest-even of x / scale.  Calls that write the same pages must be
 * ordered; with msa_decode on the same stream the insert comes first.  Rows
 * whose new tokens map to the same physical slot (a shared-prefix page, see
 * msa_prefix_share) write it concurrently: the caller passes such a token
 * once, or the same values for every row that maps it. */
msa_status msa_kv_insert(const msa_shape* shape, const msa_cache* cache, const void* k_new, const void* v_new,
                         const void* idx_new, hipStream_t stream);

/* Prefix sharing ("NVFP4 MSA kernel" of the vLLM MiniMax-M3.1-Flash post: a
 * shared-prefix page is dequantised once for up to 64 requests that share
 * it; here the index scan reads such a page once for the group's members,
 * converts it once and scores it against all their index queries).
 * Sequences form sharing groups; in a group, the first shared_blocks[g]
 * logical blocks of every member map to the same physical pages as the first
 * member's (its leader's) block_table row.  Host fields:
 *   num_groups        number of groups; 0 means no sharing (the arrays may
 *                     then be NULL)
 *   max_members       row stride of `members` and the most members a group
 *                     may hold: 1 .. MSA_SHARE_MAX, with max_members x q_len
 *                     <= MSA_SHARE_MAX (a shared page is scored against at
 *                     most 64 query tokens x 4 groups = 256 index queries)
 *   min_shared_blocks a lower bound of seq_shared_blocks[b] over ALL
 *                     sequences, 0 .. max_blocks_per_seq - 1 (0 is always
 *                     valid, and is the value when some sequence is in no
 *                     group): the scan of the sequences' own blocks starts at
 *                     this block, so the workgroups of blocks known to be
 *                     shared are never launched.  A value above the true
 *                     minimum leaves blocks unscored (precondition).
 * Device arrays, read by the kernels, unchecked like seq_lens (preconditions):
 *   members           int32 [num_groups][max_members] sequence ids, -1 padded
 *                     after the last member; a sequence is in at most one group
 *   shared_blocks     int32 [num_groups], each 0 ..
 *                     (seq_lens[b] - q_len + 1) / 128 for every member b: every
 *                     shared token is visible to all the member's queries
 *   seq_shared_blocks int32 [num_seqs]: shared_blocks of the sequence's group,
 *                     0 for a sequence in no group
 * With FP8 index keys block scores, selection and outputs equal those of the
 * unshared calls bit for bit; with NVFP4 keys see below. */
#define MSA_SHARE_MAX 64
typedef struct {
  int32_t num_groups;
  int32_t max_members;
  int32_t min_shared_blocks;
  const int32_t* members;
  const int32_t* shared_blocks;
  const int32_t* seq_shared_blocks;
} msa_prefix_share;

/* msa_indexer_score and msa_decode with prefix sharing (one scan launch that
 * scores each group's shared blocks once and every sequence's own blocks).
 * Supported for q_len 1 to 8 with FP8 or NVFP4 index keys (MSA_ERR_UNSUPPORTED
 * otherwise).  With NVFP4 keys the shared pages are dequantised exactly to
 * bf16 once for the group's members (exact products, fp32 sums), a summation
 * order other than the unshared scan's: those block scores agree with the
 * unshared call's to fp32 rounding, the sequences' own blocks bit for bit;
 * other arguments as in the unshared calls. */
msa_status msa_indexer_score_shared(const msa_shape* shape, const msa_cache* cache, const msa_prefix_share* share,
                                    const void* idx_q, float* block_scores, hipStream_t stream);
msa_status msa_decode_shared(const msa_shape* shape, const msa_cache* cache, const msa_prefix_share* share,
                             const void* q, const void* idx_q, float* out, int32_t* sel_blocks, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

const char* msa_status_string(msa_status status);
/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* msa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
