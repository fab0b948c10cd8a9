/*
 * msa_oracle.c - plain fp64 CPU oracle of the MiniMax Sparse Attention (MSA)
 * decode path.  TEST INFRASTRUCTURE ONLY: it exists so that tests, the smoke
 * check and the bench's CPU-baseline leg can check the HIP library against an
 * independent, obviously-correct definition.  Nothing in the product path may
 * call it, and it shares no code, header, table or helper with the HIP library.
 *
 * What it computes (per query row, per GQA group), in the order the method is
 * described on the pages:
 *   1. decode every stored byte to fp64 (bf16, OCP FP8 E4M3, NVFP4 = E2M1
 *      value x E4M3 scale of its 16-element group x fp32 tensor scale);
 *   2. index score of every visible key: raw dot product of the group's index
 *      query with the single shared index-key head
 *      ("MSA basics" section of the vLLM MiniMax-M3.1-Flash post);
 *   3. max-pool the scores of the visible tokens of each 128-token block
 *      (same section: "max pooling to one score per block");
 *   4. keep the block holding the query's own position plus the 15 best other
 *      visible blocks by (score descending, block index ascending); with at
 *      most 16 visible blocks, keep all of them (same section: top-16 blocks,
 *      most recent block always kept, at most 2,048 keys; "MSA mechanism
 *      details" of the MiniMax M3 x vLLM post: init_blocks = 0,
 *      local_blocks = 1, a local block that also wins top-k is not counted
 *      twice, the trailing partial block is masked);
 *   5. exact softmax attention of each query head of the group over the keys
 *      of the kept blocks that are at or before the query position, i.e. dense
 *      attention restricted to the selected set ("Prefill execution", step 4,
 *      of the MiniMax M3 x vLLM post), computed two-pass in fp64.
 *
 * Parity pins: every function here is pinned by tests that do not re-type its
 * formulas (torch's FP8 cast, the OCP E2M1 table, fp64 SDPA, brute-force
 * selection, torch.amax, invariants).  Readings where the pages are silent
 * (raw dot product without activation or 1/sqrt(d), lower block index wins
 * ties, low nibble holds the even element) are listed with the tests.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_BLOCK 128 /* tokens per KV block (page) */
#define OR_DIM 128   /* head dim and index dim */
#define OR_TOPK 16   /* kept blocks per (query, group), recent block included */

/* Problem description, mirrored field-for-field by the ctypes wrapper.  All
 * pointers are host copies of exactly the bytes the GPU path reads. */
typedef struct {
  int32_t num_seqs;
  int32_t q_len;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_blocks_per_seq;
  int32_t num_pages;
  int32_t kv_nvfp4;  /* 0: K/V bf16 [P][Hkv][128 tok][128]; 1: NVFP4 K values [P][Hkv][128 tok][64], V values
                        transposed [P][Hkv][128 dims][64 (128 tokens)], E4M3 scales [P][Hkv][128 tok][8] */
  int32_t idx_fmt;   /* index keys: 0 bf16 [P][128][128]; 1 FP8 E4M3 [P][128][128];
                        2 NVFP4 values [P][128][64] + E4M3 scales idx_sf [P][128][8] */
  double sm_scale;
  double k_scale;
  double v_scale;
  double idx_scale;
  const uint16_t* q;        /* bf16 bits [rows][Hq][128] */
  const uint16_t* iq;       /* bf16 bits [rows][Hkv][128] */
  const void* k;
  const void* v;
  const uint8_t* k_sf;
  const uint8_t* v_sf;
  const void* idx_k;
  const int32_t* block_table; /* [num_seqs][max_blocks_per_seq] */
  const int32_t* seq_lens;    /* [num_seqs] */
  const uint8_t* idx_sf;      /* NVFP4 index keys only: E4M3 scale of each 16-element group */
} oracle_problem;

/* ---- 1. decoding stored bytes ------------------------------------------ */

/* bfloat16: the upper half of an IEEE binary32. */
double msa_oracle_bf16(uint16_t bits) {
  uint32_t w = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

/* OCP FP8 E4M3 ("fn"): 1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
 * exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinity. */
double msa_oracle_e4m3(uint8_t byte) {
  int s = byte >> 7, e = (byte >> 3) & 15, m = byte & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* OCP FP4 E2M1: 1 sign, 2 exponent bits with bias 1, 1 mantissa bit;
 * exponent field 0 is subnormal (m * 0.5).  Magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6. */
double msa_oracle_e2m1(uint8_t nibble) {
  int s = (nibble >> 3) & 1, e = (nibble >> 1) & 3, m = nibble & 1;
  double mag;
  if (e == 0)
    mag = 0.5 * (double)m;
  else
    mag = ldexp(1.0 + 0.5 * (double)m, e - 1);
  return s ? -mag : mag;
}

/* One element d of token row `tok` (0..127) of KV head `h` in physical page
 * `page` of the K or V pool.  NVFP4 K: element 2k of the token's row sits in
 * the low nibble of byte k.  NVFP4 V (`transposed`): the page's (head) slab is
 * stored by dim, 128 rows of 64 B, row d holding dim d of the 128 tokens,
 * token 2k in the low nibble of byte k.  Both: elements 16c..16c+15 of a token
 * share its scale byte c. */
static double kv_elem(const oracle_problem* p, const void* pool, const uint8_t* sf, double tensor_scale,
                      int64_t page, int h, int tok, int d, int transposed) {
  int64_t row = (page * p->num_kv_heads + h) * OR_BLOCK + tok;
  if (!p->kv_nvfp4) {
    const uint16_t* x = (const uint16_t*)pool;
    return msa_oracle_bf16(x[row * OR_DIM + d]) * tensor_scale;
  }
  const uint8_t* x = (const uint8_t*)pool;
  uint8_t nib;
  if (transposed) {
    int64_t drow = (page * p->num_kv_heads + h) * OR_DIM + d;
    uint8_t byte = x[drow * (OR_BLOCK / 2) + tok / 2];
    nib = (tok & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
  } else {
    uint8_t byte = x[row * (OR_DIM / 2) + d / 2];
    nib = (d & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
  }
  double group_scale = msa_oracle_e4m3(sf[row * (OR_DIM / 16) + d / 16]);
  return msa_oracle_e2m1(nib) * group_scale * tensor_scale;
}

/* One index-key element d of token `tok` of physical page `page`.  NVFP4 index
 * keys ("NVFP4 indexer DCP" of the vLLM MiniMax-M3.1-Flash post: the index
 * cache in NVFP4) use the K/V layout with one head: element 2k in the low
 * nibble of byte k of the token row, elements 16c..16c+15 sharing scale byte c. */
static double idx_elem(const oracle_problem* p, int64_t page, int tok, int d) {
  int64_t row = page * OR_BLOCK + tok;
  if (p->idx_fmt == 2) {
    uint8_t byte = ((const uint8_t*)p->idx_k)[row * (OR_DIM / 2) + d / 2];
    uint8_t nib = (d & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
    return msa_oracle_e2m1(nib) * msa_oracle_e4m3(p->idx_sf[row * (OR_DIM / 16) + d / 16]) * p->idx_scale;
  }
  int64_t off = row * OR_DIM + d;
  if (p->idx_fmt == 1) return msa_oracle_e4m3(((const uint8_t*)p->idx_k)[off]) * p->idx_scale;
  return msa_oracle_bf16(((const uint16_t*)p->idx_k)[off]) * p->idx_scale;
}

/* Query position of flattened row (request-major: row = b*q_len + i) and the
 * number of visible tokens (pos + 1); 0 visible tokens marks a padded row. */
static int row_geometry(const oracle_problem* p, int row, int* b_out, int64_t* pos_out) {
  int b = row / p->q_len, i = row % p->q_len;
  int L = p->seq_lens[b];
  *b_out = b;
  if (L <= 0) {
    *pos_out = -1;
    return 0;
  }
  *pos_out = (int64_t)L - p->q_len + i;
  return 1;
}

/* ---- 2 + 3. index scores and block max-pool ---------------------------- */

/* bs[j] for j < max_blocks_per_seq: max over the visible tokens t <= pos of
 * block j of sum_d iq[row][g][d] * ik[t][d]; -inf for blocks past the
 * query's block.  Returns the number of visible blocks (0 for a padded row). */
int msa_oracle_block_scores(const oracle_problem* p, int row, int g, double* bs) {
  int b;
  int64_t pos;
  for (int j = 0; j < p->max_blocks_per_seq; ++j) bs[j] = -INFINITY;
  if (!row_geometry(p, row, &b, &pos)) return 0;
  int nbv = (int)(pos / OR_BLOCK) + 1;
  double q[OR_DIM];
  for (int d = 0; d < OR_DIM; ++d) q[d] = msa_oracle_bf16(p->iq[((int64_t)row * p->num_kv_heads + g) * OR_DIM + d]);
  for (int j = 0; j < nbv; ++j) {
    int64_t page = p->block_table[(int64_t)b * p->max_blocks_per_seq + j];
    double best = -INFINITY;
    for (int tok = 0; tok < OR_BLOCK; ++tok) {
      int64_t t = (int64_t)j * OR_BLOCK + tok;
      if (t > pos) break;
      double s = 0.0;
      for (int d = 0; d < OR_DIM; ++d) s += q[d] * idx_elem(p, page, tok, d);
      if (s > best) best = s;
    }
    bs[j] = best;
  }
  return nbv;
}

/* ---- 4. block selection ------------------------------------------------ */

/* a ranks before b: higher score first, lower block index on equal scores. */
static int ranks_before(double sa, int a, double sb, int bidx) { return sa > sb || (sa == sb && a < bidx); }

/* Keeps the recent block nbv-1 plus the first 15 other blocks under the order
 * above (all blocks when nbv <= 16).  sel: 16 ids ascending, -1 padded.
 * Returns the number kept. */
int msa_oracle_select(const double* bs, int nbv, int32_t* sel) {
  int n = 0;
  for (int k = 0; k < OR_TOPK; ++k) sel[k] = -1;
  if (nbv <= 0) return 0;
  if (nbv <= OR_TOPK) {
    for (int j = 0; j < nbv; ++j) sel[n++] = j;
    return n;
  }
  int r = nbv - 1;
  /* selection sort of the non-recent blocks, 15 picks */
  char* taken = (char*)calloc((size_t)r, 1);
  for (int k = 0; k < OR_TOPK - 1; ++k) {
    int best = -1;
    for (int j = 0; j < r; ++j) {
      if (taken[j]) continue;
      if (best < 0 || ranks_before(bs[j], j, bs[best], best)) best = j;
    }
    taken[best] = 1;
  }
  for (int j = 0; j < r; ++j)
    if (taken[j]) sel[n++] = j;
  sel[n++] = r;
  free(taken);
  return n;
}

/* ---- 5. attention over the selected blocks ----------------------------- */

/* out[hh][d] for the heads hh of group g (head = g * heads_per_group + hh):
 * softmax over the keys t <= pos of the selected blocks, two-pass in fp64.
 * Ids outside the visible blocks 0 .. pos/128 are ignored.  A padded row or
 * an empty selection gives zeros.  Returns the key count. */
int msa_oracle_attend(const oracle_problem* p, int row, int g, const int32_t* sel, double* out) {
  int hpg = p->num_q_heads / p->num_kv_heads;
  int b;
  int64_t pos;
  for (int i = 0; i < hpg * OR_DIM; ++i) out[i] = 0.0;
  if (!row_geometry(p, row, &b, &pos)) return 0;
  /* key list */
  int64_t keys_page[OR_TOPK * OR_BLOCK];
  int keys_tok[OR_TOPK * OR_BLOCK];
  int nk = 0;
  for (int k = 0; k < OR_TOPK; ++k) {
    int j = sel[k];
    /* ids that name no visible block contribute nothing (and index no table entry) */
    if (j < 0 || j >= p->max_blocks_per_seq || (int64_t)j * OR_BLOCK > pos) continue;
    int64_t page = p->block_table[(int64_t)b * p->max_blocks_per_seq + j];
    for (int tok = 0; tok < OR_BLOCK; ++tok) {
      if ((int64_t)j * OR_BLOCK + tok > pos) break;
      keys_page[nk] = page;
      keys_tok[nk] = tok;
      ++nk;
    }
  }
  if (nk == 0) return 0;
  double* z = (double*)malloc(sizeof(double) * (size_t)nk);
  double* vrow = (double*)malloc(sizeof(double) * OR_DIM);
  for (int hh = 0; hh < hpg; ++hh) {
    int h = g * hpg + hh;
    double q[OR_DIM];
    for (int d = 0; d < OR_DIM; ++d) q[d] = msa_oracle_bf16(p->q[((int64_t)row * p->num_q_heads + h) * OR_DIM + d]);
    double m = -INFINITY;
    for (int n = 0; n < nk; ++n) {
      double s = 0.0;
      for (int d = 0; d < OR_DIM; ++d)
        s += q[d] * kv_elem(p, p->k, p->k_sf, p->k_scale, keys_page[n], g, keys_tok[n], d, 0);
      z[n] = p->sm_scale * s;
      if (z[n] > m) m = z[n];
    }
    double denom = 0.0;
    double* o = out + hh * OR_DIM;
    for (int n = 0; n < nk; ++n) {
      double w = exp(z[n] - m);
      denom += w;
      for (int d = 0; d < OR_DIM; ++d)
        vrow[d] = kv_elem(p, p->v, p->v_sf, p->v_scale, keys_page[n], g, keys_tok[n], d, 1);
      for (int d = 0; d < OR_DIM; ++d) o[d] += w * vrow[d];
    }
    for (int d = 0; d < OR_DIM; ++d) o[d] /= denom;
  }
  free(vrow);
  free(z);
  return nk;
}

/* ---- the whole path ---------------------------------------------------- */

/* Rows [row_begin, row_end) of the flattened (request-major) query rows.
 * Outputs, indexed from row_begin:
 *   bs  [rows][Hkv][max_blocks_per_seq] (may be NULL)
 *   sel [rows][Hkv][16]
 *   out [rows][Hq][128]
 * (row, group) pairs are independent; OpenMP spreads them over threads. */
int msa_oracle_decode(const oracle_problem* p, int row_begin, int row_end, double* bs, int32_t* sel, double* out,
                      int nthreads) {
  int G = p->num_kv_heads, hpg = p->num_q_heads / p->num_kv_heads;
  int64_t npairs = (int64_t)(row_end - row_begin) * G;
  int mb = p->max_blocks_per_seq;
  (void)nthreads;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
  for (int64_t pair = 0; pair < npairs; ++pair) {
    int rr = (int)(pair / G), g = (int)(pair % G);
    int row = row_begin + rr;
    double* my_bs = bs ? bs + pair * mb : (double*)malloc(sizeof(double) * (size_t)mb);
    int nbv = msa_oracle_block_scores(p, row, g, my_bs);
    int32_t* my_sel = sel + pair * OR_TOPK;
    msa_oracle_select(my_bs, nbv, my_sel);
    msa_oracle_attend(p, row, g, my_sel, out + ((int64_t)rr * p->num_q_heads + (int64_t)g * hpg) * OR_DIM);
    if (!bs) free(my_bs);
  }
  return 0;
}

/* ---- the write side: quantising new tokens into the paged pools -------- */

/* The method keeps K/V in NVFP4 and the index cache in FP8 or NVFP4 ("What is
 * new in M3.1" and "NVFP4 indexer DCP" of the vLLM MiniMax-M3.1-Flash post);
 * the pages do not print the quantiser.  Reading taken (the generator's): per
 * group of 16 elements x with tensor scale gs,
 *   s = E4M3 nearest-even of amax|x| / (6 gs), at most 448;
 *   code_i = E2M1 nearest-even of x_i / (s gs), saturating at +-6;
 * a group with amax 0 or s == 0 stores scale 0 and codes 0; an E2M1 code that
 * rounds to zero is +0, an E4M3 byte keeps the sign.  Every step is a
 * single fp32 operation, in this order (6 * gs, amax / that, s * gs,
 * x_i / that): an integer decision must come out the same on both sides, so
 * the oracle takes it in the kernel's precision.  Rounding to nearest-even is
 * done here by search over the format's values, in exact (double) arithmetic. */

/* E4M3 byte of the value nearest to y (finite, |y| <= 448); ties to the code
 * with an even mantissa; the sign is kept, also when the result is zero. */
uint8_t msa_oracle_e4m3_rne(float y) {
  double a = fabs((double)y);
  int best = 0;
  double bd = a;
  for (int c = 1; c <= 0x7E; ++c) {
    double d = fabs(msa_oracle_e4m3((uint8_t)c) - a);
    if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
      bd = d;
      best = c;
    }
  }
  return (uint8_t)(signbit(y) ? (best | 0x80) : best);
}

/* E2M1 code of the value nearest to y, ties to the code with an even
 * mantissa, |y| > 6 saturating to 6; -0 is not produced. */
uint8_t msa_oracle_e2m1_rne(float y) {
  double a = fabs((double)y);
  int best = 0;
  double bd = a;
  for (int c = 1; c <= 7; ++c) {
    double d = fabs(msa_oracle_e2m1((uint8_t)c) - a);
    if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
      bd = d;
      best = c;
    }
  }
  return (uint8_t)((y < 0 && best != 0) ? (best | 8) : best);
}

/* One NVFP4 group: 16 values -> 8 packed bytes (element 2k in the low nibble
 * of byte k) and its E4M3 scale byte. */
void msa_oracle_quant_nvfp4_group(const float* x, float gs, uint8_t* packed, uint8_t* scale) {
  float amax = 0.0f;
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  uint8_t codes[16] = {0};
  uint8_t s = 0;
  if (amax > 0.0f) {
    float denom = 6.0f * gs;
    float t = amax / denom;
    s = msa_oracle_e4m3_rne(fminf(t, 448.0f));
  }
  if (s != 0) {
    float d = (float)msa_oracle_e4m3(s) * gs;
    for (int i = 0; i < 16; ++i) codes[i] = msa_oracle_e2m1_rne(x[i] / d);
  }
  for (int k = 0; k < 8; ++k) packed[k] = (uint8_t)(codes[2 * k] | (codes[2 * k + 1] << 4));
  *scale = s;
}

/* bf16 nearest-even of a finite float, from the definition: of the two bf16
 * values that bracket x (x with its low 16 bits cleared, and the next bf16
 * away from zero) take the one nearer in exact (double) arithmetic; on a tie
 * the one whose last kept bit is 0.  A value beyond the largest finite bf16
 * by at least half a unit rounds to infinity, as IEEE rounding does. */
uint16_t msa_oracle_bf16_rne(float x) {
  uint32_t w;
  memcpy(&w, &x, sizeof w);
  uint16_t lo = (uint16_t)(w >> 16);     /* toward zero */
  uint16_t hi = (uint16_t)(lo + 1u);     /* away from zero (0x7F80 = inf past the top) */
  double a = fabs((double)x);
  double dlo = a - fabs(msa_oracle_bf16(lo));
  double dhi = ((hi & 0x7FFFu) == 0x7F80u) ? ldexp(1.0, 128) - a : fabs(msa_oracle_bf16(hi)) - a;
  if (dlo < dhi) return lo;
  if (dhi < dlo) return hi;
  return (lo & 1u) ? hi : lo;
}

/* Quantise the new tokens of every query row into the pools of p (whose
 * pointers must then be writable host copies).  Row (b, i) sits at position
 * seq_lens[b] - q_len + i, i.e. token row pos % 128 of page
 * block_table[b][pos / 128]; padded rows (seq_lens[b] == 0) write nothing.
 *   k_new, v_new float [rows][Hkv][128] (the bf16 inputs, exactly);
 *   idx_new      float [rows][128].
 * K / V: NVFP4 with tensor scales k_scale / v_scale, or bf16 of x / scale.
 * Index keys: FP8 E4M3 nearest-even of x / idx_scale clamped to +-448, NVFP4
 * with tensor scale idx_scale, or bf16 of x / idx_scale. */
int msa_oracle_kv_insert(const oracle_problem* p, const float* k_new, const float* v_new, const float* idx_new) {
  int rows = p->num_seqs * p->q_len, G = p->num_kv_heads;
  for (int row = 0; row < rows; ++row) {
    int b;
    int64_t pos;
    if (!row_geometry(p, row, &b, &pos)) continue;
    int64_t page = p->block_table[(int64_t)b * p->max_blocks_per_seq + pos / OR_BLOCK];
    int tok = (int)(pos % OR_BLOCK);
    for (int which = 0; which < 2; ++which) {
      const float* src = which ? v_new : k_new;
      void* pool = (void*)(which ? p->v : p->k);
      uint8_t* sf = (uint8_t*)(which ? p->v_sf : p->k_sf);
      float gs = (float)(which ? p->v_scale : p->k_scale);
      for (int h = 0; h < G; ++h) {
        const float* x = src + ((int64_t)row * G + h) * OR_DIM;
        int64_t r = (page * G + h) * OR_BLOCK + tok;
        if (p->kv_nvfp4 && which) {
          /* V: the group's 16 codes go to 16 dim rows of the transposed slab */
          for (int c = 0; c < OR_DIM / 16; ++c) {
            uint8_t packed[8];
            msa_oracle_quant_nvfp4_group(x + 16 * c, gs, packed, sf + r * (OR_DIM / 16) + c);
            for (int i = 0; i < 16; ++i) {
              uint8_t code = (uint8_t)((packed[i / 2] >> (4 * (i & 1))) & 15);
              int64_t drow = (page * G + h) * OR_DIM + 16 * c + i;
              uint8_t* byte = (uint8_t*)pool + drow * (OR_BLOCK / 2) + tok / 2;
              *byte = (tok & 1) ? (uint8_t)((*byte & 0x0F) | (code << 4)) : (uint8_t)((*byte & 0xF0) | code);
            }
          }
        } else if (p->kv_nvfp4) {
          for (int c = 0; c < OR_DIM / 16; ++c)
            msa_oracle_quant_nvfp4_group(x + 16 * c, gs, (uint8_t*)pool + r * (OR_DIM / 2) + 8 * c, sf + r * (OR_DIM / 16) + c);
        } else {
          for (int d = 0; d < OR_DIM; ++d) ((uint16_t*)pool)[r * OR_DIM + d] = msa_oracle_bf16_rne(x[d] / gs);
        }
      }
    }
    const float* x = idx_new + (int64_t)row * OR_DIM;
    int64_t r = page * OR_BLOCK + tok;
    float is = (float)p->idx_scale;
    if (p->idx_fmt == 2) {
      for (int c = 0; c < OR_DIM / 16; ++c)
        msa_oracle_quant_nvfp4_group(x + 16 * c, is, (uint8_t*)p->idx_k + r * (OR_DIM / 2) + 8 * c,
                                     (uint8_t*)p->idx_sf + r * (OR_DIM / 16) + c);
    } else if (p->idx_fmt == 1) {
      for (int d = 0; d < OR_DIM; ++d) {
        float y = x[d] / is;
        ((uint8_t*)p->idx_k)[r * OR_DIM + d] = msa_oracle_e4m3_rne(fmaxf(-448.0f, fminf(448.0f, y)));
      }
    } else {
      for (int d = 0; d < OR_DIM; ++d) ((uint16_t*)p->idx_k)[r * OR_DIM + d] = msa_oracle_bf16_rne(x[d] / is);
    }
  }
  return 0;
}
