// Device helpers shared by the MoE-VQ kernels (gfx950, wave64).
#pragma once

#include <type_traits>

#include "moe_vq_internal.h"

namespace mvq {

// Cross-lane reductions with DPP lane moves (VALU, no LDS traffic).  Every lane of the
// wave must be active.  Control words: quad_perm [1,0,3,2] and [2,3,0,1] exchange
// lanes 1 and 2 apart within a quad; row_half_mirror maps lane i to 7-i within each 8
// lanes and row_mirror maps i to 15-i within each 16, so after the four moves every
// lane of a 16-lane row holds the row's result.  Rows are combined through readlane.
namespace dpp {
constexpr int QUAD_XOR1 = 0xB1;
constexpr int QUAD_XOR2 = 0x4E;
constexpr int ROW_HALF_MIRROR = 0x141;
constexpr int ROW_MIRROR = 0x140;
}  // namespace dpp

template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, dpp_i32<CTRL>(__builtin_bit_cast(int, v)));
}

__device__ __forceinline__ float lane_f32(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over aligned groups of W consecutive lanes (W = 2, 4, 8, 16 or 64); every lane
// of a group receives the group's sum.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(W == 2 || W == 4 || W == 8 || W == 16 || W == 64, "group width");
  v += dpp_f32<dpp::QUAD_XOR1>(v);
  if (W >= 4) v += dpp_f32<dpp::QUAD_XOR2>(v);
  if (W >= 8) v += dpp_f32<dpp::ROW_HALF_MIRROR>(v);
  if (W >= 16) v += dpp_f32<dpp::ROW_MIRROR>(v);
  if (W == 64) v = (lane_f32(v, 0) + lane_f32(v, 16)) + (lane_f32(v, 32) + lane_f32(v, 48));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<dpp::QUAD_XOR1>(v));
  v = fmaxf(v, dpp_f32<dpp::QUAD_XOR2>(v));
  v = fmaxf(v, dpp_f32<dpp::ROW_HALF_MIRROR>(v));
  v = fmaxf(v, dpp_f32<dpp::ROW_MIRROR>(v));
  return fmaxf(fmaxf(lane_f32(v, 0), lane_f32(v, 16)), fmaxf(lane_f32(v, 32), lane_f32(v, 48)));
}

// Inclusive prefix sum over the 64 lanes: row_shr by 1, 2, 4 and 8 within each
// 16-lane row (lanes with no source in the row add 0), then the totals of the rows
// below through readlane.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
            r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// Order-preserving map of a float to uint32 (larger float -> larger key, -0 == +0;
// NaN must be excluded by the caller) and its inverse.
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f + 0.0f);  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_from_order_key(uint32_t k) {
  return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v, uint64_t old) {
  const int lo = __builtin_amdgcn_update_dpp((int)(uint32_t)old, (int)(uint32_t)v, CTRL, ROW_MASK, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp((int)(uint32_t)(old >> 32), (int)(uint32_t)(v >> 32), CTRL, ROW_MASK, 0xF, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Unsigned 64-bit maximum over the 64 lanes, returned to every lane.  After the four
// in-row moves every lane of a row holds the row maximum; row_bcast:15 then brings
// row 0 into row 1 and row 2 into row 3, row_bcast:31 brings row 1 into rows 2-3, so
// lane 63 ends with the maximum of all rows.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  uint64_t o;
  o = dpp_u64<dpp::QUAD_XOR1>(v, 0); v = o > v ? o : v;
  o = dpp_u64<dpp::QUAD_XOR2>(v, 0); v = o > v ? o : v;
  o = dpp_u64<dpp::ROW_HALF_MIRROR>(v, 0); v = o > v ? o : v;
  o = dpp_u64<dpp::ROW_MIRROR>(v, 0); v = o > v ? o : v;
  o = dpp_u64<0x142, 0xA>(v, v); v = o > v ? o : v;  // row_bcast:15 into rows 1 and 3
  o = dpp_u64<0x143, 0xC>(v, v); v = o > v ? o : v;  // row_bcast:31 into rows 2 and 3
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Exclusive block scan of four ints per thread over 1024 threads: DPP scans within
// each wave, then one over the 16 wave totals in wave 0.
__device__ inline int4 block_scan_excl4(int4 v, int4* wave_tot, int4* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int4 inc = make_int4(wave_incl_scan(v.x), wave_incl_scan(v.y), wave_incl_scan(v.z), wave_incl_scan(v.w));
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const int4 c = lane < 16 ? wave_tot[lane] : make_int4(0, 0, 0, 0);
    const int4 w = make_int4(wave_incl_scan(c.x), wave_incl_scan(c.y), wave_incl_scan(c.z), wave_incl_scan(c.w));
    if (lane < 16) wave_tot[lane] = make_int4(w.x - c.x, w.y - c.y, w.z - c.z, w.w - c.w);
    if (lane == 15) *total = w;
  }
  __syncthreads();
  const int4 b = wave_tot[wave];
  const int4 r = make_int4(b.x + inc.x - v.x, b.y + inc.y - v.y, b.z + inc.z - v.z, b.w + inc.w - v.w);
  __syncthreads();
  return r;
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
// v_ldexp_f32 of 1.0 needs no literal constants; 255 gives 2^128 = inf, and inf - inf
// is the NaN that code encodes.
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  const float v = __builtin_amdgcn_ldexpf(1.0f, (int)e - 127);
  return e == 255 ? v - v : v;
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

// Same address with the byte selector as a value (a constant once loops are unrolled).
__device__ __forceinline__ uint32_t tab_addr_sel(uint32_t word, uint32_t laneoff, uint32_t sel) {
  return __builtin_amdgcn_perm(word, laneoff, 0x0c0c0400u + (sel << 8));
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

// Exponent e with m = f * 2^e, f in [0.5, 1) (one v_frexp_exp_i32_f32; 0 for zero).
__device__ __forceinline__ int frexp_exponent(float m) { return __builtin_amdgcn_frexp_expf(m); }

// x * 2^e (one v_ldexp_f32).
__device__ __forceinline__ float ldexp2(float x, int e) { return __builtin_amdgcn_ldexpf(x, e); }

// SiLU with the hardware exponential (v_exp_f32 of x * log2(e)).
__device__ __forceinline__ float silu_fast(float g) { return g / (1.0f + __expf(-g)); }

// An expert's FC1 output from its gate and up values: silu(g) * u, or with the SwiGLU
// clamp of limit lim > 0, silu(min(g, lim)) * clamp(u, -lim, lim) (a NaN stays NaN).
__device__ __forceinline__ float swiglu(float g, float u, float lim) {
  if (lim > 0.f) {
    g = g > lim ? lim : g;
    u = u > lim ? lim : (u < -lim ? -lim : u);
  }
  return silu_fast(g) * u;
}

__device__ __forceinline__ uint4 ldg16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

// f(integral_constant<int, I>) for I = B .. N - 1, in order.
template <int B, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < N) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, N>(f);
  }
}

}  // namespace mvq
