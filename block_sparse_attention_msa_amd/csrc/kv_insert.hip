// kv_insert.hip - the write side of a decode step: the new tokens' K, V and
// index keys quantised into the paged pools.
//
// Method ("What is new in M3.1" and "NVFP4 indexer DCP" of the vLLM
// MiniMax-M3.1-Flash post: the KV cache in NVFP4, E2M1 values with one E4M3
// scale per 16 elements and a tensor scale; the index cache in FP8 or NVFP4;
// "QKV GEMM + Norm + RoPE + KV-insert fusion" there: K, V and the index key
// quantised to NVFP4 and written straight into their caches; "Decode
// execution" of the MiniMax M3 x vLLM post: each step updates the cache
// state before scoring).  The pages do not print the quantiser; the one
// here, per group of 16 values x with tensor scale gs:
//   s = E4M3 nearest-even of amax|x| / (6 gs) (at most 448);
//   code_i = E2M1 nearest-even of x_i / (s gs), saturating at +-6;
// amax 0 or s == 0 stores scale 0 and codes 0.  Every step is one fp32
// operation in this order (6 gs, amax / that, s gs, x_i / that) with IEEE
// round-to-nearest-even, so the stored bytes are a function of the inputs
// alone.  FP8 index keys: E4M3 nearest-even of x / idx_scale clamped to +-448
// (sign kept on zero); bf16 pools: bf16 nearest-even of x / scale.
//
// One 128-thread workgroup per query row; a thread quantises one 16-element
// group (4 K heads x 8, 4 V heads x 8, then the index key's 8 groups), so the
// kernel reads 32 B and writes 9 B (NVFP4) per thread: a few hundred KB per
// decode step, latency-bound, nothing to tile.  NVFP4 V is stored by dim (row
// d of a page's head slab holds dim d of its 128 tokens, token 2i in the low
// nibble of byte i), so a token's 16 codes of a group go to one nibble in each
// of 16 rows, and tokens 2i, 2i + 1 share each byte.  The thread of an even
// token whose odd partner is written by the same call quantises the partner's
// group too and stores whole bytes (the partner stores only its scale); a
// token whose partner is not in the call sets its own nibble of each byte with
// an atomic AND (clear) and an atomic OR on the byte's 32-bit word, leaving the
// other nibble as it is (no other writer touches that nibble in the call).
#include "msa_device.hpp"
#include "msa_kernels.hpp"

namespace msa {
namespace {

// E4M3 code (sign 0) of the value nearest to t, 0 <= t <= 448, ties to the
// even mantissa.  Subnormals (below 2^-6) are multiples of 2^-9.
__device__ __forceinline__ uint32_t e4m3_rne_nonneg(float t) {
  if (t < 0.015625f) return (uint32_t)__builtin_rintf(t * 512.0f);  // 0..8; 8 is 2^-6 = code 0x08
  const uint32_t bits = __float_as_uint(t);
  uint32_t q = bits >> 20;                  // exponent (8 bits) and the top 3 mantissa bits
  const uint32_t rem = bits & 0xFFFFFu;     // the 20 mantissa bits rounded away
  if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;
  const int e = (int)(q >> 3) - 127;        // -6 .. 8
  return (uint32_t)(((e + 7) << 3) | (q & 7u));
}

// E2M1 code of the value nearest to y, ties to the even code, saturating at 6;
// a zero result is +0.
__device__ __forceinline__ uint32_t e2m1_rne(float y) {
  const float a = __builtin_fabsf(y);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  return (y < 0.f && c != 0u) ? (c | 8u) : c;
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t w = __float_as_uint(f);
  w += 0x7FFFu + ((w >> 16) & 1u);
  return (uint16_t)(w >> 16);
}

// 16 bf16 inputs -> fp32 (exact).
__device__ __forceinline__ void load16(const uint16_t* src, float (&x)[16]) {
  const uint4 a = *reinterpret_cast<const uint4*>(src);
  const uint4 b = *reinterpret_cast<const uint4*>(src + 8);
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    x[2 * k] = bf16lo_to_f32(w[k]);
    x[2 * k + 1] = bf16hi_to_f32(w[k]);
  }
}

// One NVFP4 group in registers: the 16 codes packed (element 2k in the low
// nibble of byte k: elements 0..7 in .x, 8..15 in .y) and the scale code.
__device__ __forceinline__ uint2 nvfp4_group(const float (&x)[16], float gs, uint32_t& scale) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i]));
  uint32_t s = 0;
  if (amax > 0.f) {
    const float denom = 6.0f * gs;
    const float t = amax / denom;
    s = e4m3_rne_nonneg(__builtin_fminf(t, 448.0f));
  }
  uint32_t lo = 0, hi = 0;
  if (s != 0u) {
    const float d = e4m3_to_f32(s) * gs;
#pragma unroll
    for (int i = 0; i < 8; ++i) lo |= e2m1_rne(x[i] / d) << (4 * i);
#pragma unroll
    for (int i = 0; i < 8; ++i) hi |= e2m1_rne(x[8 + i] / d) << (4 * i);
  }
  scale = s;
  return make_uint2(lo, hi);
}

// One NVFP4 group: 8 packed bytes (element 2k in the low nibble of byte k) + scale.
__device__ __forceinline__ void quant_nvfp4_group(const float (&x)[16], float gs, uint8_t* packed, uint8_t* scale) {
  uint32_t s;
  *reinterpret_cast<uint2*>(packed) = nvfp4_group(x, gs, s);
  *scale = (uint8_t)s;
}

// One NVFP4 V group of token tok into byte tok / 2 of the 16 dim rows starting
// at row0 (64 B each); its scale as K's.  With x_next (the group of token
// tok + 1, tok even, written by the same call) both nibbles are stored whole;
// otherwise only this token's nibble changes.
__device__ __forceinline__ void quant_nvfp4_group_v(const float (&x)[16], const float (&x_next)[16], bool both,
                                                    float gs, uint8_t* row0, int tok, uint8_t* scale) {
  uint32_t s, s_next;
  const uint2 own = nvfp4_group(x, gs, s);
  *scale = (uint8_t)s;
  const uint2 next = both ? nvfp4_group(x_next, gs, s_next) : make_uint2(0u, 0u);  // s_next: the partner stores it
  const int byte = tok >> 1, sh = 8 * (byte & 3) + 4 * (tok & 1);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t code = ((i < 8 ? own.x : own.y) >> (4 * (i & 7))) & 15u;
    uint8_t* rowi = row0 + (size_t)i * (kBlock / 2);
    if (both) {
      rowi[byte] = (uint8_t)(code | ((((i < 8 ? next.x : next.y) >> (4 * (i & 7))) & 15u) << 4));
    } else {
      uint32_t* word = reinterpret_cast<uint32_t*>(rowi + (byte & ~3));
      atomicAnd(word, ~(15u << sh));
      atomicOr(word, code << sh);
    }
  }
}

// 16 values -> 16 bf16 (x / scale, nearest-even).
__device__ __forceinline__ void store_bf16_group(const float (&x)[16], float scale, uint16_t* dst) {
  uint32_t w[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
    w[k] = (uint32_t)bf16_rne(x[2 * k] / scale) | ((uint32_t)bf16_rne(x[2 * k + 1] / scale) << 16);
  *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  *reinterpret_cast<uint4*>(dst + 8) = make_uint4(w[4], w[5], w[6], w[7]);
}

constexpr int kInsThreads = 128;

__global__ __launch_bounds__(kInsThreads) void kv_insert_kernel(const InsertArgs a) {
  const int row = blockIdx.x;
  const int b = row / a.q_len;
  const int L = a.seq_lens[b];
  if (L <= 0) return;  // padded row
  const int pos = L - a.q_len + row % a.q_len;
  const int64_t page = a.block_table[(size_t)b * a.mbps + pos / kBlock];
  const int tok = pos % kBlock;
  const int u = threadIdx.x;
  float x[16];
  if (u < 2 * kGroups * 8) {  // K (u < 32) or V: head h, group c
    const bool is_v = u >= kGroups * 8;
    const int h = (u % (kGroups * 8)) / 8, c = u % 8;
    load16((is_v ? a.v_new : a.k_new) + ((size_t)row * kGroups + h) * kDim + 16 * c, x);
    const int64_t r = (page * kGroups + h) * kBlock + tok;
    const float gs = is_v ? a.v_scale : a.k_scale;
    if (a.kv_nvfp4 && is_v) {
      // the partner token tok ^ 1 (same page) is written by this call when it is
      // the row after (tok even) or before (tok odd) in the same sequence's chunk
      const int i_row = row % a.q_len;
      const bool even = (tok & 1) == 0;
      const bool partner = even ? i_row + 1 < a.q_len : i_row > 0;
      uint8_t* row0 = a.v + ((page * kGroups + h) * kDim + 16 * c) * (kBlock / 2);
      if (partner && !even) {
        uint32_t s;
        nvfp4_group(x, gs, s);  // the even partner stores the codes
        a.v_sf[r * 8 + c] = (uint8_t)s;
      } else {
        float xn[16] = {};
        if (partner) load16(a.v_new + ((size_t)(row + 1) * kGroups + h) * kDim + 16 * c, xn);
        quant_nvfp4_group_v(x, xn, partner, gs, row0, tok, a.v_sf + r * 8 + c);
      }
    } else if (a.kv_nvfp4)
      quant_nvfp4_group(x, gs, a.k + r * (kDim / 2) + 8 * c, a.k_sf + r * 8 + c);
    else
      store_bf16_group(x, gs, reinterpret_cast<uint16_t*>(is_v ? a.v : a.k) + r * kDim + 16 * c);
  } else if (u < 2 * kGroups * 8 + 8) {  // the index key: group c
    const int c = u - 2 * kGroups * 8;
    load16(a.idx_new + (size_t)row * kDim + 16 * c, x);
    const int64_t r = page * kBlock + tok;
    if (a.idx_fmt == kIdxNvfp4) {
      quant_nvfp4_group(x, a.idx_scale, a.idx + r * (kDim / 2) + 8 * c, a.idx_sf + r * 8 + c);
    } else if (a.idx_fmt == kIdxFp8) {
      uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float y = __builtin_fmaxf(-448.0f, __builtin_fminf(448.0f, x[i] / a.idx_scale));
        const uint32_t byte = e4m3_rne_nonneg(__builtin_fabsf(y)) | (__builtin_signbitf(y) ? 0x80u : 0u);
        w[i / 4] |= byte << (8 * (i % 4));
      }
      *reinterpret_cast<uint4*>(a.idx + r * kDim + 16 * c) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      store_bf16_group(x, a.idx_scale, reinterpret_cast<uint16_t*>(a.idx) + r * kDim + 16 * c);
    }
  }
}

}  // namespace

hipError_t launch_kv_insert(const InsertArgs& a, hipStream_t stream) {
  kv_insert_kernel<<<dim3((unsigned)a.rows), dim3(kInsThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace msa
