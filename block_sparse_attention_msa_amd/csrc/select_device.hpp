// select_device.hpp - exact block selection of one (query row, group), run by
// a whole workgroup; shared by the stand-alone selection kernel and the
// fused attention kernel.
//
// Method ("MSA basics", vLLM MiniMax-M3.1-Flash post; "MSA mechanism details",
// MiniMax M3 x vLLM post): keep the block holding the query position
// (local_blocks = 1, init_blocks = 0) plus the best other visible blocks so
// that 16 blocks are kept; a local block that also wins top-k is not counted
// twice, so the others are the top 15 of the blocks before it.  Ties go to the
// lower block index (total order: score descending, index ascending), which
// makes the selection exact under any split of the candidates.
//
// Algorithm (A selection waves: one for tables of up to 256 blocks, else the
// waves the row needs at 1,024 keys each, but at least four, one per SIMD,
// when the workgroup has them; E <= 16 keys per lane):
//  1. wave w < A takes blocks j = 64 (A e + w) + lane (e < E; coalesced loads,
//     all issued before use, and before the row length is known) as 64-bit
//     keys (ordered score << 32 | ~j), and, for the attention, the blocks'
//     page ids from the block table;
//  2. lane l's best score over its keys in all selection waves (the blocks
//     j = l mod 64) is gathered through LDS; every active wave sorts the 64
//     lane-bests (32-bit bitonic, DPP lane moves where they exist), and their
//     15th best T0 bounds the 15th best key overall from below (15 distinct
//     blocks reach it);
//  3. keys whose score is >= T0 (every true top-15 key among them) are
//     compacted into LDS with ballots, one LDS atomic per wave; a wave whose
//     count exceeds 15 lanes x E keys (many scores tied at T0) uses its exact
//     64-bit 15th-best lane key instead, which bounds its count again;
//  4. wave 0 ranks up to 64 candidates by counting larger keys (broadcast LDS
//     reads); more are merged 49 at a time into a running top-15 with a 64-bit
//     bitonic sort;
//  5. the 15 ids plus the recent block are written in ascending order, with
//     their page ids when asked for.
// One wave issues about 40 instructions per key per lane in steps 1-3, so the
// keys are spread over a wave of each SIMD rather than held by one wave.
#pragma once

#include "msa_device.hpp"

namespace msa {

constexpr int kSelKeysPerLane = 16;                               // keys per lane of an active wave, at most
constexpr int kSelBlocksPerWave = kWave * kSelKeysPerLane;         // 1,024
constexpr int kSelWaveCap = (kTopK - 1) * kSelKeysPerLane;         // candidates per active wave, at most
constexpr int kSelMinWaves = 4;                                    // one wave per SIMD
constexpr int kSelSoloBlocks = 4 * kWave;                          // up to here one wave, no barrier

// A workgroup of NT threads selects among at most (NT / 64) x 1,024 blocks.
template <int NT>
constexpr int sel_max_blocks() { return NT / kWave * kSelBlocksPerWave; }

// The selection waves A for rows of at most cap blocks (cap <= sel_max_blocks):
// one wave up to 256 blocks (4 keys per lane cost less than the workgroup
// barrier and the exchange of lane-bests), else the waves that 1,024 keys each
// need, at least kSelMinWaves when the workgroup has them.  Wave w < A holds
// blocks 64 (A e + w) + lane.
template <int NT>
__device__ __forceinline__ int sel_waves(int cap) {
  constexpr int kWaves = NT / kWave;
  if (cap <= kSelSoloBlocks) return 1;
  const int need = (cap + kSelBlocksPerWave - 1) / kSelBlocksPerWave;
  return min(kWaves, max(need, kSelMinWaves));
}

template <int NT>
struct SelectSmem {
  static constexpr int kCandCap = kSelWaveCap * (NT / kWave) + kWave;  // at most 15 x 16 keys per active wave
  uint64_t cand[kCandCap];
  int32_t cand_page[kCandCap];
  uint32_t lane_best[NT / kWave][kWave];  // each selection wave's lane-best scores
  int32_t win[kTopK];
  int32_t win_page[kTopK];
  int count;
};

__device__ __forceinline__ uint64_t block_key(float s, int j) {
  uint32_t u = __builtin_bit_cast(uint32_t, s);
  if (u == 0x80000000u) u = 0u;  // -0 ranks equal to +0
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(~(uint32_t)j);
}
__device__ __forceinline__ int key_block(uint64_t k) { return (int)(~(uint32_t)k); }

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

// value of lane ^ J (J a power of two < 64)
template <int J>
__device__ __forceinline__ uint32_t xor_lane(uint32_t x, int lane) {
  if constexpr (J == 1) {
    return dpp_u32<0xB1>(x);                        // quad_perm [1,0,3,2]
  } else if constexpr (J == 2) {
    return dpp_u32<0x4E>(x);                        // quad_perm [2,3,0,1]
  } else if constexpr (J == 4) {
    const uint32_t up = dpp_u32<0x104>(x);          // row_shl:4, lane i reads i+4
    const uint32_t dn = dpp_u32<0x114>(x);          // row_shr:4, lane i reads i-4
    return (lane & 4) ? dn : up;
  } else if constexpr (J == 8) {
    return dpp_u32<0x128>(x);                       // row_ror:8 (= xor 8 in a row of 16)
  } else if constexpr (J == 16) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x401F);  // bit-mask swizzle: lane ^ 16
  } else {
    return (uint32_t)__shfl_xor((int)x, J);
  }
}

template <int K, int J>
__device__ __forceinline__ uint64_t bitonic_step(uint64_t v, int lane) {
  const uint32_t lo = xor_lane<J>((uint32_t)v, lane);
  const uint32_t hi = xor_lane<J>((uint32_t)(v >> 32), lane);
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  const bool lower = (lane & J) == 0;   // lower index of its pair
  const bool desc = (lane & K) == 0;    // this run sorts descending
  const bool take_max = lower == desc;
  return take_max ? (o > v ? o : v) : (o < v ? o : v);
}

// Bitonic sort of one key per lane, descending: lane 0 ends with the largest.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t v, int lane) {
  v = bitonic_step<2, 1>(v, lane);
  v = bitonic_step<4, 2>(v, lane);
  v = bitonic_step<4, 1>(v, lane);
  v = bitonic_step<8, 4>(v, lane);
  v = bitonic_step<8, 2>(v, lane);
  v = bitonic_step<8, 1>(v, lane);
  v = bitonic_step<16, 8>(v, lane);
  v = bitonic_step<16, 4>(v, lane);
  v = bitonic_step<16, 2>(v, lane);
  v = bitonic_step<16, 1>(v, lane);
  v = bitonic_step<32, 16>(v, lane);
  v = bitonic_step<32, 8>(v, lane);
  v = bitonic_step<32, 4>(v, lane);
  v = bitonic_step<32, 2>(v, lane);
  v = bitonic_step<32, 1>(v, lane);
  v = bitonic_step<64, 32>(v, lane);
  v = bitonic_step<64, 16>(v, lane);
  v = bitonic_step<64, 8>(v, lane);
  v = bitonic_step<64, 4>(v, lane);
  v = bitonic_step<64, 2>(v, lane);
  v = bitonic_step<64, 1>(v, lane);
  return v;
}

// LDS written by some lanes of a wave and read by others of the same wave.
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int K, int J>
__device__ __forceinline__ uint32_t bitonic_step32(uint32_t v, int lane) {
  const uint32_t o = xor_lane<J>(v, lane);
  const bool take_max = ((lane & J) == 0) == ((lane & K) == 0);
  return take_max ? (o > v ? o : v) : (o < v ? o : v);
}

// Bitonic sort of one 32-bit value per lane, descending.
__device__ __forceinline__ uint32_t wave_sort_desc32(uint32_t v, int lane) {
  v = bitonic_step32<2, 1>(v, lane);
  v = bitonic_step32<4, 2>(v, lane);
  v = bitonic_step32<4, 1>(v, lane);
  v = bitonic_step32<8, 4>(v, lane);
  v = bitonic_step32<8, 2>(v, lane);
  v = bitonic_step32<8, 1>(v, lane);
  v = bitonic_step32<16, 8>(v, lane);
  v = bitonic_step32<16, 4>(v, lane);
  v = bitonic_step32<16, 2>(v, lane);
  v = bitonic_step32<16, 1>(v, lane);
  v = bitonic_step32<32, 16>(v, lane);
  v = bitonic_step32<32, 8>(v, lane);
  v = bitonic_step32<32, 4>(v, lane);
  v = bitonic_step32<32, 2>(v, lane);
  v = bitonic_step32<32, 1>(v, lane);
  v = bitonic_step32<64, 32>(v, lane);
  v = bitonic_step32<64, 16>(v, lane);
  v = bitonic_step32<64, 8>(v, lane);
  v = bitonic_step32<64, 4>(v, lane);
  v = bitonic_step32<64, 2>(v, lane);
  v = bitonic_step32<64, 1>(v, lane);
  return v;
}

// Appends this wave's keys[e] >= thr (all E per lane) and their pages to
// cand[] (any order): one ballot per key slot, the popcounts prefix-summed on
// the scalar unit, one LDS atomic per wave.
template <int E, bool PAGES>
__device__ __forceinline__ void sel_append(const uint64_t (&keys)[E], const int32_t (&pages)[E], uint64_t thr,
                                           uint64_t (&ballot)[E], int total, int lane, uint64_t* cand,
                                           int32_t* cand_page, int* count, bool solo) {
  int base = 0;
  if (solo) {  // the only wave with candidates: they start at 0
    if (lane == 0) *count = total;
  } else {
    if (lane == 0) base = atomicAdd(count, total);
    base = __shfl(base, 0);
  }
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (keys[e] >= thr) {
      const int at = base + __popcll(ballot[e] & below);
      cand[at] = keys[e];
      if constexpr (PAGES) cand_page[at] = pages[e];
    }
    base += __popcll(ballot[e]);
  }
}

template <int E>
__device__ __forceinline__ int sel_ballots(const uint64_t (&keys)[E], uint64_t thr, uint64_t (&ballot)[E]) {
  int total = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    ballot[e] = __ballot(keys[e] >= thr);
    total += __popcll(ballot[e]);
  }
  return total;
}

// One wave's raw candidates: 16 block scores and block-table entries per lane.
struct SelLoads {
  float sv[kSelKeysPerLane];
  int32_t pages[kSelKeysPerLane];
};

// Issues this wave's loads of its blocks 64 (A e + w) + lane (A =
// sel_waves(cap)), clamped to the row's cap entries, so that they need not
// wait for the row length: the scores s[] and, when PAGES, the block-table
// entries (read, never followed).  Waves past A load nothing.  Entries past the
// candidates are discarded by select_blocks, so they may hold anything.
template <int NT, bool PAGES>
__device__ __forceinline__ void select_load(const float* __restrict__ s, const int32_t* __restrict__ bt_row, int cap,
                                            SelLoads& ld) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int A = sel_waves<NT>(cap);
  if (wave >= A) return;  // wave-uniform
#pragma unroll
  for (int e = 0; e < kSelKeysPerLane; ++e) {
    // keys per lane: the power of two that covers cap (select_blocks uses a
    // power of two covering the row length, never more)
    if (e > 0 && (e & (e - 1)) == 0 && kWave * A * e >= cap) break;  // wave-uniform
    const int idx = min(kWave * (A * e + wave) + lane, cap - 1);
    ld.sv[e] = s[idx];
    ld.pages[e] = PAGES ? bt_row[idx] : 0;
  }
}

// The selection proper for n >= 16 candidates (blocks 0 .. n - 1, n = r) held
// by A selection waves, with E of the loaded keys per lane in use, 64 A E >= n
// (the blocks beyond a lane's first E keys are past the row).
template <int NT, bool PAGES, int E>
__device__ __forceinline__ void select_core(const SelLoads& ld, const int32_t* __restrict__ bt_row, int r, int A,
                                            SelectSmem<NT>& sm, int32_t* out, int32_t* out_page) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int n = r;
  // waves holding candidates: with one key per lane, the first n / 64
  const int active = E == 1 ? min(A, (n + kWave - 1) / kWave) : A;
  int32_t recent_page = 0;
  if (PAGES && tid == kTopK - 1) recent_page = bt_row[r];

  // 1. E keys (and pages) per lane of the active waves, each lane's best score
  uint64_t keys[E];
  int32_t pages[E];
  uint32_t best = 0;
  if (wave < active) {  // loaded: these blocks are below cap
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = kWave * (A * e + wave) + lane;
      pages[e] = ld.pages[e];
      const uint64_t k = block_key(ld.sv[e], j);
      keys[e] = j < n ? k : 0;
      const uint32_t hi = (uint32_t)(keys[e] >> 32);
      best = hi > best ? hi : best;
    }
  }

  // 2. T0 = the 15th best of the 64 lane-best scores, lane l's best taken over
  //    its keys in every active wave (blocks j = l mod 64; the waves' bests
  //    meet in LDS), so 15 distinct blocks reach T0 and every top-15 key
  //    scores at least T0 (wave 0 always has at least 16 lanes holding keys,
  //    so T0 > 0 and absent keys, 0, never qualify).  Every active wave sorts
  //    the same 64 values.  With one active wave (solo, workgroup-uniform) no
  //    workgroup barrier is needed until the winners are written.
  const bool solo = active == 1;
  if (!solo) {
    if (wave < active) sm.lane_best[wave][lane] = best;
    if (tid == 0) sm.count = 0;
    __syncthreads();
    if (wave < active)
      for (int w = 0; w < active; ++w) best = sm.lane_best[w][lane] > best ? sm.lane_best[w][lane] : best;
  }
  uint32_t t0 = 0;
  if (wave < active) t0 = (uint32_t)__builtin_amdgcn_readlane((int)wave_sort_desc32(best, lane), kTopK - 2);

  // 3. candidates: score >= T0, or, in a wave with too many ties at T0, key >=
  //    the wave's exact 15th-best lane key
  if (wave < active) {
    uint64_t thr = (uint64_t)t0 << 32;
    uint64_t ballot[E];
    int total = sel_ballots(keys, thr, ballot);
    if (total > (kTopK - 1) * E) {  // wave-uniform
      uint64_t best64 = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) best64 = keys[e] > best64 ? keys[e] : best64;
      const uint64_t sorted = wave_sort_desc(best64, lane);
      const uint64_t tw = ((uint64_t)__shfl((uint32_t)(sorted >> 32), kTopK - 2) << 32) |
                          (uint32_t)__shfl((uint32_t)sorted, kTopK - 2);
      thr = tw > thr ? tw : thr;
      total = sel_ballots(keys, thr, ballot);
    }
    sel_append<E, PAGES>(keys, pages, thr, ballot, total, lane, sm.cand, sm.cand_page, &sm.count, solo);
  }
  if (solo)
    wave_sync_lds();  // wave 0 reads back what it wrote
  else
    __syncthreads();

  if (wave == 0) {
    // 4. the 15 best candidates -> lanes 0..14 (any order): (myj, mypage)
    const int count = sm.count;  // >= 15: every top-15 key qualifies
    int myj = 0x7fffffff;
    int32_t mypage = 0;
    if (count <= kWave) {
      const uint64_t mine = lane < count ? sm.cand[lane] : 0;
      int rank = 0;
#pragma unroll 8
      for (int i = 0; i < count; ++i) rank += sm.cand[i] > mine ? 1 : 0;
      if (lane < count && rank < kTopK - 1) {  // rank is unique: keys are distinct
        sm.win[rank] = key_block(mine);
        if constexpr (PAGES) sm.win_page[rank] = sm.cand_page[lane];
      }
      wave_sync_lds();
      if (lane < kTopK - 1) {
        myj = sm.win[lane];
        if constexpr (PAGES) mypage = sm.win_page[lane];
      }
    } else {
      // running top-15 in lanes 0..14, 49 new candidates per round
      uint64_t top = 0;
      for (int base = 0; base < count; base += kWave - (kTopK - 1)) {
        uint64_t v = 0;
        if (lane < kTopK - 1) {
          v = top;
        } else {
          const int idx = base + lane - (kTopK - 1);
          if (idx < count) v = sm.cand[idx];
        }
        top = wave_sort_desc(v, lane);
      }
      if (lane < kTopK - 1) {
        myj = key_block(top);
        if constexpr (PAGES) mypage = bt_row[myj];
      }
    }
    // 5. 15 winners ascending by block id, then the recent block
    int rank = 0;
#pragma unroll
    for (int m = 0; m < kTopK - 1; ++m) {
      const int other = __shfl(myj, m);
      rank += other < myj ? 1 : 0;
    }
    if (lane < kTopK - 1) {
      out[rank] = myj;
      if constexpr (PAGES) out_page[rank] = mypage;
    }
    if (lane == kTopK - 1) {
      out[kTopK - 1] = r;
      if constexpr (PAGES) out_page[kTopK - 1] = recent_page;
    }
  }
  __syncthreads();
}

// Selection for one (row, group) by a workgroup of NT threads; cap must not
// exceed sel_max_blocks<NT>() so that every candidate fits the selection
// waves' registers (1,024 per wave).
// ld: the wave's select_load of the row/group's scores with this cap (r < cap);
// bt_row: its block table row (read only when PAGES); r: the recent block
// (0 <= r < row length).  Writes 16 ids (ascending, -1 padded) to out[] and,
// when PAGES, their page ids to out_page[] (0 for padding), then synchronises
// the workgroup so LDS outputs are readable by every thread.  Every thread of
// the workgroup must call it.
template <int NT, bool PAGES>
__device__ void select_blocks(const SelLoads& ld, const int32_t* __restrict__ bt_row, int r, int cap,
                              SelectSmem<NT>& sm, int32_t* out, int32_t* out_page) {
  constexpr int kWaves = NT / kWave;
  static_assert(NT % kWave == 0 && kWaves >= 1, "whole waves");
  const int tid = threadIdx.x;
  if (r + 1 <= kTopK) {  // every visible block is kept
    if (tid < kTopK) {
      out[tid] = tid <= r ? tid : -1;
      if constexpr (PAGES) out_page[tid] = tid <= r ? bt_row[tid] : 0;
    }
    __syncthreads();
    return;
  }
  // candidates: blocks 0 .. r-1 (n = r >= 16); the keys per lane in use
  // follow the row length (a workgroup-uniform choice)
  const int A = sel_waves<NT>(cap);
  const int per = (r + kWave * A - 1) / (kWave * A);
  if (per <= 1)
    select_core<NT, PAGES, 1>(ld, bt_row, r, A, sm, out, out_page);
  else if (per <= 2)
    select_core<NT, PAGES, 2>(ld, bt_row, r, A, sm, out, out_page);
  else if (per <= 4)
    select_core<NT, PAGES, 4>(ld, bt_row, r, A, sm, out, out_page);
  else if (per <= 8)
    select_core<NT, PAGES, 8>(ld, bt_row, r, A, sm, out, out_page);
  else
    select_core<NT, PAGES, kSelKeysPerLane>(ld, bt_row, r, A, sm, out, out_page);
}

}  // namespace msa
