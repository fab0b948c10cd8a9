// msa_device.hpp - gfx950 device helpers shared by the MSA kernels: exact
// format conversions on the CDNA4 conversion instructions, the bf16 dot
// product, DPP lane moves and the lane layout used by the scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msa_kernels.hpp"

namespace msa {

constexpr int kWave = 64;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

// Two OCP E4M3 bytes (HI=false: bytes 0,1 of w; HI=true: bytes 2,3) -> two
// bf16 in the same order.  Exact: E4M3 (3 mantissa bits, 2^-9..448) fits bf16.
template <bool HI>
__device__ __forceinline__ bf16x2 e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
}

// The two E2M1 nibbles of byte SEL of w (low nibble first) -> two bf16 / f32.
// Exact: E2M1 magnitudes are 0, .5, 1, 1.5, 2, 3, 4, 6.
template <int SEL>
__device__ __forceinline__ bf16x2 e2m1x2_to_bf16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL);
}
template <int SEL>
__device__ __forceinline__ f32x2 e2m1x2_to_f32x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// One OCP E4M3 byte -> f32 (exact).
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_scalef32_f32_fp8(byte, 1.0f, 0);
}

// bf16 pair -> f32 pair (exact).
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// c + a.x*b.x + a.y*b.y in fp32 (bf16 x bf16 products are exact in fp32).
__device__ __forceinline__ float dot2(bf16x2 a, bf16x2 b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

// DPP lane moves (within rows of 16 lanes).
constexpr int kDppXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowShl4 = 0x104; // lane i reads lane i+4 of its row
constexpr int kDppRowShl8 = 0x108; // lane i reads lane i+8 of its row
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Four per-lane partial dot products a[k] belong, in this lane, to groups
// (heads) k ^ (2*(lane&1)) ^ ((lane>>1)&1).  Summing over 2^LOG2 lanes that
// share a token: after the reduction, lanes whose bits 2..LOG2-1 are zero hold
// the full sum for group  2*(lane&1) + ((lane>>1)&1).  LOG2 is 3 (8 lanes per
// token) or 4 (16 lanes per token).  4 (5) DPP adds instead of 12 (16).
__device__ __forceinline__ int permuted_group(int lane, int k) { return k ^ ((lane & 1) << 1) ^ ((lane >> 1) & 1); }
__device__ __forceinline__ int lane_group(int lane) { return ((lane & 1) << 1) | ((lane >> 1) & 1); }

template <int LOG2>
__device__ __forceinline__ float reduce4_permuted(float a0, float a1, float a2, float a3) {
  a0 += dpp<kDppXor1>(a2);
  a1 += dpp<kDppXor1>(a3);
  a0 += dpp<kDppXor2>(a1);
  a0 += dpp<kDppRowShl4>(a0);
  if constexpr (LOG2 == 4) a0 += dpp<kDppRowShl8>(a0);
  return a0;
}

// 2^x on the hardware exponential (v_exp_f32), for x <= 0 (softmax weights):
// no range reduction needed; results below 2^-126 flush to 0.
__device__ __forceinline__ float exp2_nonpos(float x) { return __builtin_amdgcn_exp2f(x); }

// The scan that opens a decode step zeroes the arrival counters of the
// attention launch that follows it (n <= 64, by the launch's first
// workgroup; the kernel boundary orders these stores before the attention).
__device__ __forceinline__ void zero_step_counters(int32_t* p, int n) {
  if (p && blockIdx.x == 0 && blockIdx.y == 0 && (int)threadIdx.x < n) p[threadIdx.x] = 0;
}

__device__ __forceinline__ float wave_max_xor(float m, int from) {
  for (int off = from; off < kWave; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
  return m;
}

}  // namespace msa
