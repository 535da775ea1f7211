// Device helpers shared by the MoE-VQ kernels (gfx950, wave64).
#pragma once

#include "moe_vq_internal.h"

namespace mvq {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Sum over aligned groups of W consecutive lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// E8M0 shared exponent -> 2^(e-127) as fp32 (e = 0 gives the subnormal 2^-127, 255 NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  uint32_t bits = (e == 0) ? 0x00400000u : (e == 255 ? 0x7FC00000u : (e << 23));
  return __builtin_bit_cast(float, bits);
}

// Fill the LDS decode table (see TAB_COPIES): entry b holds sgn(b) * CB[b & 0x7F] as
// four fp16, the sign applied by flipping the fp16 sign bits (exact).
__device__ __forceinline__ void build_vq2_table(uint2* tab, const uint16_t* __restrict__ cb,
                                                int tid, int nthreads) {
  const uint2* cb2 = reinterpret_cast<const uint2*>(cb);
  for (int idx = tid; idx < 256 * TAB_COPIES; idx += nthreads) {
    const int b = idx >> 5;
    const uint2 v = cb2[b & 127];
    const uint32_t flip = (b & 128) ? 0x80008000u : 0u;
    tab[idx] = make_uint2(v.x ^ flip, v.y ^ flip);
  }
}

// LDS byte address of word byte `sel` (0..3) of `word` for this lane's table copy.
// laneoff = (lane & 31) * 8 (fits in bits 0..7).
template <int SEL>
__device__ __forceinline__ uint32_t tab_addr(uint32_t word, uint32_t laneoff) {
  return __builtin_amdgcn_perm(word, laneoff, 0x0c0c0400u + (SEL << 8));
}

__device__ __forceinline__ uint2 tab_lookup(const uint2* tab, uint32_t addr) {
  return *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(tab) + addr);
}

// Two E2M1 elements of byte SEL of `word` -> two fp16 (low nibble -> low half), exact.
template <int SEL>
__device__ __forceinline__ half2_t fp4x2_to_half2(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, SEL);
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

__device__ __forceinline__ float dot2h(half2_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(a, __builtin_bit_cast(half2_t, b), c, false);
}

__device__ __forceinline__ uint4 ldg16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

}  // namespace mvq
