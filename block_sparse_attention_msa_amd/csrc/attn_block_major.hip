// attn_block_major.hip - KV-block-major attention for multi-query rows
// (verify / prefill chunks): each selected KV block is loaded and dequantised
// once for all the query rows of its (sequence, group) that selected it.
//
// Method ("KV-block-major prefill" of the MiniMax M3 x vLLM post: the
// per-query block lists are inverted into per-block query lists, each
// selected block is processed once for the queries that chose it, and the
// per-block partial results of every query are merged by log-sum-exp;
// "MSA basics" of the vLLM MiniMax-M3.1-Flash post: exact attention over the
// kept blocks).  Three launches after the selection:
//  1. inversion: one 1024-thread workgroup per (sequence, group) counting-sorts the
//     (query row, slot) pairs of its q_len x 16 selections by block id in LDS
//     and cuts each block's list into work items of at most 16 rows;
//  2. block-major attention: a persistent grid walks the work items; per item
//     the block's K is dequantised once (exactly) to bf16 and its V to f16
//     into LDS (V is stored by dim, so each 4-byte word of a dim row is 8
//     tokens of it, already in the PV operand order); each wave then takes 4 of the item's rows x the 4
//     heads of the group (16 MFMA columns): QK on bf16 MFMAs, the causal mask
//     of each row inside the block, softmax statistics, PV on f16 MFMAs, and
//     writes the row's partial (m, l, o) for that slot;
//  3. merge: per (row, group) the 16 slot partials are combined by
//     log-sum-exp and scaled by v_scale / l.
// Work and results depend only on the selections: the order in which a
// block's rows are grouped into items does not change any value.
#include "attn_device.hpp"
#include "msa_device.hpp"
#include "msa_kernels.hpp"

namespace msa {
namespace {

constexpr int kBmItemRows = 16;   // query rows per work item: 4 waves x 4 rows
constexpr int kBmWaves = 4;
constexpr int kBmThreads = kBmWaves * kWave;

// ---- 1. inversion ----------------------------------------------------------

// cnt[] first counts each block's valid selections, then holds the packed
// exclusive prefixes start | item_offset << 16 (both below 2^16: at most
// q_len x 16 <= 4,096 entries), whose low half is then the scatter cursor.
// 1024 threads, each holding up to 4 of the (row, slot) selections in
// registers (loaded once, all in flight together).
constexpr int kInvThreads = 1024;
constexpr int kInvPer = kBmMaxQ * kTopK / kInvThreads;
__global__ __launch_bounds__(kInvThreads) void bm_invert_kernel(const int32_t* __restrict__ sel,
                                                              const int32_t* __restrict__ seq_lens,
                                                              const int32_t* __restrict__ block_table, int q_len,
                                                              int mbps, int4* __restrict__ items,
                                                              int32_t* __restrict__ entries,
                                                              int32_t* __restrict__ n_items) {
  __shared__ uint32_t cnt[kBmMaxBlocks];
  __shared__ uint32_t wtot[kInvThreads / kWave];
  __shared__ uint32_t total;
  const int sg = blockIdx.x;
  const int b = sg / kGroups, g = sg % kGroups;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int E = q_len * kTopK;
  int4* it = items + (size_t)sg * E;
  int32_t* en = entries + (size_t)sg * E;
  const int L = seq_lens[b];
  if (L <= 0) {
    if (tid == 0) n_items[sg] = 0;
    return;
  }
  const int nblk = min((L - 1) / kBlock + 1, mbps);
  // entry e = tid + kInvThreads k: row i = e / 16, slot e % 16; -1 where it
  // names no block with visible tokens
  int id[kInvPer];
#pragma unroll
  for (int k = 0; k < kInvPer; ++k) {
    const int e = tid + kInvThreads * k;
    id[k] = e < E ? sel[((size_t)(b * q_len + e / kTopK) * kGroups + g) * kTopK + e % kTopK] : -1;
  }
  for (int k = tid; k < nblk; k += kInvThreads) cnt[k] = 0;
#pragma unroll
  for (int k = 0; k < kInvPer; ++k) {
    const int e = tid + kInvThreads * k;
    if (!(id[k] >= 0 && id[k] < nblk && id[k] * kBlock <= L - q_len + e / kTopK)) id[k] = -1;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kInvPer; ++k)
    if (id[k] >= 0) atomicAdd(&cnt[id[k]], 1u);
  __syncthreads();
  // exclusive scan of (count, items) over the blocks: each thread a contiguous chunk
  const int per = (nblk + kInvThreads - 1) / kInvThreads;
  const int k0 = min(tid * per, nblk), k1 = min(k0 + per, nblk);
  uint32_t v = 0;
  for (int k = k0; k < k1; ++k) {
    const uint32_t c = cnt[k];
    v += c | (((c + kBmItemRows - 1) / kBmItemRows) << 16);
  }
  uint32_t x = v;  // inclusive scan within the wave
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) wtot[wave] = x;
  __syncthreads();
  uint32_t base = 0;
  for (int w = 0; w < wave; ++w) base += wtot[w];
  uint32_t run = base + x - v;
  for (int k = k0; k < k1; ++k) {
    const uint32_t c = cnt[k];
    cnt[k] = run;
    run += c | (((c + kBmItemRows - 1) / kBmItemRows) << 16);
  }
  if (tid == kInvThreads - 1) {
    total = base + x;
    n_items[sg] = (int)((base + x) >> 16);
  }
  __syncthreads();
  // work items: (block, page, first entry, entries)
  for (int k = tid; k < nblk; k += kInvThreads) {
    const uint32_t pk = cnt[k];
    const int st = (int)(pk & 0xFFFFu), io = (int)(pk >> 16);
    const int nxt = (int)((k + 1 < nblk ? cnt[k + 1] : total) & 0xFFFFu);
    const int c = nxt - st;
    if (c == 0) continue;
    const int page = block_table[(size_t)b * mbps + k];
    for (int m = 0; m * kBmItemRows < c; ++m)
      it[io + m] = make_int4(k, page, st + m * kBmItemRows, min(kBmItemRows, c - m * kBmItemRows));
  }
  __syncthreads();
  // entries (row i << 4 | slot), grouped by block
#pragma unroll
  for (int k = 0; k < kInvPer; ++k) {
    if (id[k] < 0) continue;
    const int e = tid + kInvThreads * k;
    const uint32_t p = atomicAdd(&cnt[id[k]], 1u) & 0xFFFFu;
    en[p] = ((e / kTopK) << 4) | (e % kTopK);
  }
}

// ---- 2. block-major attention ------------------------------------------------

struct BmSmem {
  // K of the block, bf16 [token][128 dims]: 16-B chunk k (dims 8k .. 8k + 7) of
  // token t at t * 256 + 16 (k ^ (t % 16))
  uint8_t k[kBlock * kDim * 2];
  // V of the block, f16, transposed [dim][128 tokens]: chunk k (tokens 8k ..
  // 8k + 7) of dim d at d * 256 + 16 (k ^ (d % 16))
  uint8_t vt[kDim * kBlock * 2];
  // softmax weights per wave, f16 [16 (row, head) columns][128 tokens]: chunk
  // k (tokens 8k .. 8k + 7) of column n at n * 256 + 16 (k ^ n)
  // (while an item's K and V are staged, before any wave writes its weights,
  // p[0]'s first 1 KB holds the block's V scales by group, [8][128 tokens])
  uint8_t p[kBmWaves][16 * kBlock * 2];
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * 256 + 16 * (chunk ^ (row & 15)); }

__global__ __launch_bounds__(kBmThreads, 2) void bm_attn_kernel(
    const int4* __restrict__ items, const int32_t* __restrict__ entries, const int32_t* __restrict__ n_items,
    int num_sg, const uint8_t* __restrict__ kpool, const uint8_t* __restrict__ vpool,
    const uint8_t* __restrict__ k_sf, const uint8_t* __restrict__ v_sf, const uint16_t* __restrict__ q,
    const int32_t* __restrict__ seq_lens, int q_len, float qk_scale_log2, float* __restrict__ po,
    float2* __restrict__ pml) {
  __shared__ BmSmem sm;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int E = q_len * kTopK;  // item and entry array stride per (sequence, group)
  int max_items = 0;            // items are walked item-index-major: stop past the longest list
  for (int k = 0; k < num_sg; ++k) max_items = max(max_items, n_items[k]);
  const long long n_it = (long long)max_items * num_sg;
  for (long long itx = blockIdx.x; itx < n_it; itx += gridDim.x) {
    const int u = (int)(itx / num_sg), sg = (int)(itx % num_sg);
    if (u >= n_items[sg]) continue;  // workgroup-uniform
    const int4 item = items[(size_t)sg * E + u];
    const int blk = item.x, ebeg = item.z, ecnt = item.w;
    const int64_t page = item.y;
    const int b = sg / kGroups, g = sg % kGroups;
    const int L = seq_lens[b];
    const int64_t row0 = (page * kGroups + g) * kBlock;  // first (token, head) row of the slab
    const int tvis = min(L - kBlock * blk, kBlock);      // tokens of the block the last row sees
    __syncthreads();  // every wave is done with the previous item's LDS
    uint8_t* vs = sm.p[0];  // V scales by group [8][128 tokens]; 0 past the last token any row sees
    {  // V scales, transposed to [group][token]: thread = (token t, 4 groups)
      const int t = tid >> 1, g4 = 4 * (tid & 1);
      const uint32_t w = t < tvis ? *reinterpret_cast<const uint32_t*>(v_sf + (row0 + t) * 8 + g4) : 0u;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) vs[(g4 + q4) * kBlock + t] = (uint8_t)(w >> (8 * q4));
    }
    {  // K: thread = (token t, half): 64 dims -> bf16, 8 chunks
      const int t = tid >> 1, h2 = tid & 1;
      const uint4 c0 = *reinterpret_cast<const uint4*>(kpool + (row0 + t) * 64 + 32 * h2);
      const uint4 c1 = *reinterpret_cast<const uint4*>(kpool + (row0 + t) * 64 + 32 * h2 + 16);
      const uint32_t sw = *reinterpret_cast<const uint32_t*>(k_sf + (row0 + t) * 8 + 4 * h2);
      const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
      for (int m = 0; m < 8; ++m) {  // chunk 8 h2 + m: dims 64 h2 + 8m .. + 7, group 4 h2 + m / 2
        const float sc = e4m3_to_f32((sw >> (8 * (m >> 1))) & 0xFFu);
        const f32x2 a = e2m1x2_to_f32x2<0>(w[m]), bb = e2m1x2_to_f32x2<1>(w[m]);
        const f32x2 cc = e2m1x2_to_f32x2<2>(w[m]), d = e2m1x2_to_f32x2<3>(w[m]);
        const bf16x8 v8 = {(__bf16)(a.x * sc), (__bf16)(a.y * sc), (__bf16)(bb.x * sc), (__bf16)(bb.y * sc),
                           (__bf16)(cc.x * sc), (__bf16)(cc.y * sc), (__bf16)(d.x * sc), (__bf16)(d.y * sc)};
        *reinterpret_cast<bf16x8*>(sm.k + swz(t, 8 * h2 + m)) = v8;
      }
    }
    __syncthreads();  // the V scales
    {  // V (stored by dim): thread = (8-token chunk k, 8 dims of group G): each
       // dim row's 4 bytes of tokens 8k .. 8k + 7 -> one 16-B chunk of vt
      const int k = tid & 15, G = tid >> 5, d0 = 16 * G + 8 * ((tid >> 4) & 1);
      uint32_t w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        w[i] = *reinterpret_cast<const uint32_t*>(vpool + (row0 + d0 + i) * 64 + 4 * k);
      // group G's scales of the 8 tokens, as (2p, 2p + 1) pairs
      const uint2 s8 = *reinterpret_cast<const uint2*>(vs + G * kBlock + 8 * k);
      const f16x2 sc[4] = {__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s8.x, 1.0f, false),
                           __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s8.x, 1.0f, true),
                           __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s8.y, 1.0f, false),
                           __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s8.y, 1.0f, true)};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        f16x2 v[4];
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) v[pp] = e2m1x2_to_f16x2(w[i], pp) * sc[pp];
        const f16x8 v8 = {v[0].x, v[0].y, v[1].x, v[1].y, v[2].x, v[2].y, v[3].x, v[3].y};
        *reinterpret_cast<f16x8*>(sm.vt + swz(d0 + i, k)) = v8;
      }
    }
    __syncthreads();
    if (4 * wave >= ecnt) continue;  // wave-uniform: no rows for this wave
    const int c = lane >> 4, n = lane & 15;
    const int el = n >> 2, h = n & 3;  // QK column n: row el of the wave's 4, head h
    const bool has = 4 * wave + el < ecnt;
    const int ent = has ? entries[(size_t)sg * E + ebeg + 4 * wave + el] : 0;
    const int i = ent >> 4, slot = ent & 15;
    const int row = b * q_len + i;
    const int vis = has ? L - q_len + i - kBlock * blk + 1 : 0;  // tokens 0 .. vis - 1 (>= 1)
    bf16x8 qb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 w = has ? *reinterpret_cast<const uint4*>(q + ((size_t)row * (kGroups * kHeadsPerGroup) +
                                                                  g * kHeadsPerGroup + h) * kDim + 32 * s + 8 * c)
                          : make_uint4(0, 0, 0, 0);
      qb[s] = __builtin_bit_cast(bf16x8, w);
    }
    // QK: z[T][r] = logit (log2 domain) of token 16T + 4c + r for column n
    float z[kQkTiles][4];
    float mx = -INFINITY;
#pragma unroll
    for (int T = 0; T < kQkTiles; ++T) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(sm.k + swz(16 * T + n, 4 * s + c));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[s], acc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        z[T][r] = 16 * T + 4 * c + r < vis ? acc[r] * qk_scale_log2 : -INFINITY;
        mx = fmaxf(mx, z[T][r]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    float ls = 0.f;
    uint8_t* pw = sm.p[wave];
#pragma unroll
    for (int T = 0; T < kQkTiles; ++T) {
      f16x2 pr[2];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pv = has ? exp2_nonpos(z[T][r] - mx) : 0.f;
        ls += pv;
        pr[r >> 1][r & 1] = (_Float16)pv;
      }
      // tokens 16T + 4c .. + 3: chunk 2T + c / 2, half (c % 2) of it
      *reinterpret_cast<uint2*>(pw + swz(n, 2 * T + (c >> 1)) + 8 * (c & 1)) =
          make_uint2(__builtin_bit_cast(uint32_t, pr[0]), __builtin_bit_cast(uint32_t, pr[1]));
    }
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    if (has && c == 0) pml[(((size_t)row * kGroups + g) * kTopK + slot) * kHeadsPerGroup + h] = make_float2(mx, ls);
    // the (row, slot) of output rows 4c .. 4c + 3 (row c of the wave, heads 0..3)
    const int orow = __shfl(row, 4 * c), oslot = __shfl(slot, 4 * c);
    const bool ohas = 4 * wave + c < ecnt;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // PV: A = p (column n's 32 tokens of step s: 8c .. 8c + 7), B = V^T (dim 16D + n)
    f32x4 o[8];
#pragma unroll
    for (int D = 0; D < 8; ++D) o[D] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kPvSteps; ++s) {
      const f16x8 pa = *reinterpret_cast<const f16x8*>(pw + swz(n, 4 * s + c));
#pragma unroll
      for (int D = 0; D < 8; ++D) {
        const f16x8 vb = *reinterpret_cast<const f16x8*>(sm.vt + swz(16 * D + n, 4 * s + c));
        o[D] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, vb, o[D], 0, 0, 0);
      }
    }
    if (ohas) {  // o[D][r]: head r of row c, dim 16D + n
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float* dst = po + ((((size_t)orow * kGroups + g) * kTopK + oslot) * kHeadsPerGroup + r) * kDim;
#pragma unroll
        for (int D = 0; D < 8; ++D) dst[16 * D + n] = o[D][r];
      }
    }
  }
}

// ---- 3. merge ----------------------------------------------------------------

// One wave per (row, group). For the factors lane l takes (slot l / 4, head
// l % 4); for the sums it takes head l / 16, dims 8 (l % 16) .. + 7, so that
// one slot's four heads (2 KB) are one coalesced wave-wide read.
__global__ __launch_bounds__(kBmThreads) void bm_merge_kernel(const int32_t* __restrict__ sel,
                                                            const int32_t* __restrict__ seq_lens, int rows,
                                                            int q_len, int mbps, const float* __restrict__ po,
                                                            const float2* __restrict__ pml, float v_scale,
                                                            float* __restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int id = blockIdx.x * kBmWaves + threadIdx.x / kWave;
  if (id >= rows * kGroups) return;
  const int row = id / kGroups, g = id % kGroups;
  const int b = row / q_len;
  const int L = seq_lens[b];
  const size_t rg = (size_t)row * kGroups + g;
  // factors: slot fs = lane / 4, head fh = lane % 4
  const int fs = lane >> 2;
  bool valid = false;
  if (L > 0) {
    const int pos = L - q_len + row % q_len;
    const int nblk = min((L - 1) / kBlock + 1, mbps);
    const int j = sel[rg * kTopK + fs];
    valid = j >= 0 && j < nblk && j * kBlock <= pos;
  }
  const uint64_t vmask = __ballot(valid);  // bit 4 s + h: slot s valid
  const float2 ml = valid ? pml[rg * kTopK * kHeadsPerGroup + lane] : make_float2(-INFINITY, 0.f);
  float M = ml.x;
#pragma unroll
  for (int off = kHeadsPerGroup; off < kWave; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
  const float f = valid ? exp2_nonpos(ml.x - M) : 0.f;
  float fl = f * ml.y;
#pragma unroll
  for (int off = kHeadsPerGroup; off < kWave; off <<= 1) fl += __shfl_xor(fl, off);
  // sums: head h, dims d0 .. d0 + 7
  const int h = lane >> 4, d0 = 8 * (lane & 15);
  const float* src = po + rg * kTopK * kHeadsPerGroup * kDim + h * kDim + d0;
  float4 v[kTopK][2];  // every valid slot's partial, all loads in flight together
#pragma unroll
  for (int s = 0; s < kTopK; ++s) {
    const bool on = (vmask >> (4 * s)) & 1;
    const float4* p4 = reinterpret_cast<const float4*>(src + (size_t)s * kHeadsPerGroup * kDim);
    v[s][0] = on ? p4[0] : make_float4(0.f, 0.f, 0.f, 0.f);
    v[s][1] = on ? p4[1] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float acc[8] = {};
#pragma unroll
  for (int s = 0; s < kTopK; ++s) {
    const float w = __shfl(f, 4 * s + h);  // 0 for an invalid slot
    acc[0] = fmaf(w, v[s][0].x, acc[0]);
    acc[1] = fmaf(w, v[s][0].y, acc[1]);
    acc[2] = fmaf(w, v[s][0].z, acc[2]);
    acc[3] = fmaf(w, v[s][0].w, acc[3]);
    acc[4] = fmaf(w, v[s][1].x, acc[4]);
    acc[5] = fmaf(w, v[s][1].y, acc[5]);
    acc[6] = fmaf(w, v[s][1].z, acc[6]);
    acc[7] = fmaf(w, v[s][1].w, acc[7]);
  }
  const float flh = __shfl(fl, h);  // lanes 0 .. 3 hold heads 0 .. 3
  const float sc = flh > 0.f ? v_scale / flh : 0.f;
  float4* dst = reinterpret_cast<float4*>(out + rg * kHeadsPerGroup * kDim + h * kDim + d0);
  dst[0] = make_float4(acc[0] * sc, acc[1] * sc, acc[2] * sc, acc[3] * sc);
  dst[1] = make_float4(acc[4] * sc, acc[5] * sc, acc[6] * sc, acc[7] * sc);
}

}  // namespace

size_t block_major_scratch_bytes(int num_seqs, int q_len) {
  const size_t sg = (size_t)num_seqs * kGroups, E = (size_t)q_len * kTopK, rows = (size_t)num_seqs * q_len;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return al(sg * E * sizeof(int4)) + al(sg * E * 4) + al(sg * 4) +
         al(rows * kGroups * kTopK * kHeadsPerGroup * kDim * 4) + al(rows * kGroups * kTopK * kHeadsPerGroup * 8);
}

hipError_t launch_block_major_attn(const AttnArgs& a, int num_seqs, void* scratch, hipStream_t stream) {
  if (!a.kv_nvfp4 || a.q_len < 1 || a.q_len > kBmMaxQ || a.mbps > kBmMaxBlocks || !a.sel) return hipErrorInvalidValue;
  const size_t sg = (size_t)num_seqs * kGroups, E = (size_t)a.q_len * kTopK, rows = (size_t)a.rows;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  char* p = static_cast<char*>(scratch);
  int4* items = reinterpret_cast<int4*>(p);
  p += al(sg * E * sizeof(int4));
  int32_t* entries = reinterpret_cast<int32_t*>(p);
  p += al(sg * E * 4);
  int32_t* n_items = reinterpret_cast<int32_t*>(p);
  p += al(sg * 4);
  float* po = reinterpret_cast<float*>(p);
  p += al(rows * kGroups * kTopK * kHeadsPerGroup * kDim * 4);
  float2* pml = reinterpret_cast<float2*>(p);
  bm_invert_kernel<<<dim3((unsigned)sg), dim3(kInvThreads), 0, stream>>>(a.sel, a.seq_lens, a.block_table, a.q_len,
                                                                          a.mbps, items, entries, n_items);
  bm_attn_kernel<<<dim3((unsigned)(2 * device_cus())), dim3(kBmThreads), 0, stream>>>(
      items, entries, n_items, (int)sg, static_cast<const uint8_t*>(a.k), static_cast<const uint8_t*>(a.v), a.k_sf,
      a.v_sf, a.q, a.seq_lens, a.q_len, a.qk_scale_log2, po, pml);
  bm_merge_kernel<<<dim3((unsigned)((rows * kGroups + kBmWaves - 1) / kBmWaves)), dim3(kBmThreads), 0, stream>>>(
      a.sel, a.seq_lens, a.rows, a.q_len, a.mbps, po, pml, a.v_scale, a.out);
  return hipGetLastError();
}

}  // namespace msa
