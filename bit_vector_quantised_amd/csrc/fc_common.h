// Pieces shared by the decode-path FC kernels (vector-ALU stream/generic kernels and
// the matrix-core kernel): table fill, workspace check, token-group records.
#pragma once

#include "moe_vq_device.h"
#include "moe_vq_launch.h"

namespace mvq {

// Fill the table from one codebook entry per thread (threads 0..255 own words 0..255);
// the copy index is rotated by lane so that one ds_write_b64 instruction spreads over
// all banks.
__device__ __forceinline__ void write_table_entry(uint2* tab, uint2 cbv, int b) {
  const uint32_t flip = (b & 128) ? 0x80008000u : 0u;
  const uint2 v = make_uint2(cbv.x ^ flip, cbv.y ^ flip);
  const int rot = b & 31;
#pragma unroll
  for (int c = 0; c < TAB_COPIES; ++c) tab[b * TAB_COPIES + ((c + rot) & 31)] = v;
}

__device__ __forceinline__ uint32_t pack_half2(float lo, float hi) {
  const _Float16 l = (_Float16)lo, h = (_Float16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, l) | ((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
}

// Four VQ2 words (one dword of codes) against their 16 fp16 activations (8 dwords),
// added to p in order.  A 16-byte chunk is four such steps.
__device__ __forceinline__ float vq2_dword_dot(const uint2* tab, uint32_t wd, uint32_t laneoff,
                                               const uint32_t* xw, float p) {
  uint2 e0 = tab_lookup(tab, tab_addr<0>(wd, laneoff));
  uint2 e1 = tab_lookup(tab, tab_addr<1>(wd, laneoff));
  uint2 e2 = tab_lookup(tab, tab_addr<2>(wd, laneoff));
  uint2 e3 = tab_lookup(tab, tab_addr<3>(wd, laneoff));
  p = dot2(e0.x, xw[0], p); p = dot2(e0.y, xw[1], p);
  p = dot2(e1.x, xw[2], p); p = dot2(e1.y, xw[3], p);
  p = dot2(e2.x, xw[4], p); p = dot2(e2.y, xw[5], p);
  p = dot2(e3.x, xw[6], p); p = dot2(e3.y, xw[7], p);
  return p;
}

__device__ __forceinline__ uint32_t dword_of(const uint4& q, int i) {
  return i == 0 ? q.x : i == 1 ? q.y : i == 2 ? q.z : q.w;
}

// 16 VQ2 words of one 16-byte chunk against 64 fp16 activations (32 dwords).
__device__ __forceinline__ float vq2_chunk_dot(const uint2* tab, const uint4& q, uint32_t laneoff,
                                               const uint32_t* xw) {
  float p = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) p = vq2_dword_dot(tab, dword_of(q, i), laneoff, xw + 8 * i, p);
  return p;
}

// 32 E2M1 elements of one 16-byte chunk against 32 fp16 activations (16 dwords).
__device__ __forceinline__ float mx4_chunk_dot(const uint4& q, const uint32_t* xw) {
  float p = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t wd = i == 0 ? q.x : i == 1 ? q.y : i == 2 ? q.z : q.w;
    p = dot2h(fp4x2_to_half2<0>(wd), xw[4 * i + 0], p);
    p = dot2h(fp4x2_to_half2<1>(wd), xw[4 * i + 1], p);
    p = dot2h(fp4x2_to_half2<2>(wd), xw[4 * i + 2], p);
    p = dot2h(fp4x2_to_half2<3>(wd), xw[4 * i + 3], p);
  }
  return p;
}

// The workspace was routed for this call: shape key, counts within their bounds, the
// token-group size this kernel is built for, and (FC1) the same activations.  All header
// words are read before any is tested (one round trip, not several).  A refused call
// writes MOE_VQ_EINVAL into the status word (one lane of workgroup 0) and computes
// nothing, so moe_vq_check() reports it: nothing is skipped silently.
__device__ __forceinline__ bool ws_ok(const FcArgs& a, bool fc1, int MT) {
  const uint32_t key = a.hdr[HDR_KEY], n_active = a.hdr[HDR_N_ACTIVE];
  const uint32_t groups = a.hdr[fc1 ? HDR_GROUPS1 : HDR_GROUPS2], mt = a.hdr[fc1 ? HDR_MT1 : HDR_MT2];
  const uint32_t xlo = a.hdr[HDR_X_LO], xhi = a.hdr[HDR_X_HI], xdt = a.hdr[HDR_X_DTYPE];
  bool ok = (key == a.key) & (n_active <= (uint32_t)a.E) & (groups <= (uint32_t)a.max_groups) &
            (mt == (uint32_t)MT);
  if (fc1) ok = ok & x_matches(xlo, xhi, xdt, a.x_addr, a.x_dtype);
  if (!ok && blockIdx.x == 0 && threadIdx.x == 0) {
    a.hdr[HDR_STATUS] = MOE_VQ_EINVAL;
    a.hdr[HDR_INFO] = 0xFFFFFFFFu;
  }
  return ok;
}

// The fields of a GroupRec a tile needs, held in scalar registers (uniform per workgroup).
struct RecS {
  uint64_t slot_off;
  int32_t p0;
  int32_t mcount;
  uint32_t fmt;
  int32_t pair[MAX_MT];
};

__device__ __forceinline__ int32_t uni(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// v through an empty asm statement: the compiler cannot treat what is derived from it
// as loop-invariant.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// v copied into a new register by an instruction the compiler cannot see through.  An
// in-place cross-lane op (v_permlane32_swap) ties its operands to its results; handed a
// ring register directly, the register coalescer gives the loop-carried ring value the
// swap's registers, so the refill load lands elsewhere and the loop's back edge copies it
// back, waiting for every refill in flight.  Copying at the point of use keeps the ring
// in the registers its loads write.
__device__ __forceinline__ uint32_t reg_copy(uint32_t v) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
  return r;
}

static_assert(offsetof(GroupRec, p0) == 8 && offsetof(GroupRec, mcount) == 12 && offsetof(GroupRec, fmt) == 16 &&
              offsetof(GroupRec, pair) == 24, "GroupRec layout");

// A record's two 16-byte words as loaded, and the fields taken from them; loading two
// records before taking either lets their loads overlap.
struct RecRaw {
  int4 w0, w1, w2;
};

__device__ __forceinline__ RecRaw load_rec_raw(const GroupRec* recs, int g) {
  const int4* p = reinterpret_cast<const int4*>(recs + g);
  return RecRaw{p[0], p[1], p[2]};
}

__device__ __forceinline__ RecS rec_from_raw(const RecRaw& raw) {
  RecS r;
  r.slot_off = ((uint64_t)(uint32_t)uni(raw.w0.y) << 32) | (uint32_t)uni(raw.w0.x);
  r.p0 = uni(raw.w0.z);
  r.mcount = uni(raw.w0.w);
  r.fmt = (uint32_t)uni(raw.w1.x);
  static_assert(MAX_MT == 4, "pair indices span words 1 and 2");
  const int pw[MAX_MT] = {raw.w1.z, raw.w1.w, raw.w2.x, raw.w2.y};
#pragma unroll
  for (int j = 0; j < MAX_MT; ++j) r.pair[j] = uni(pw[j]);
  return r;
}

__device__ __forceinline__ RecS load_rec(const GroupRec* recs, int g) {
  const int4* p = reinterpret_cast<const int4*>(recs + g);
  const int4 w0 = p[0], w1 = p[1];
  RecS r;
  r.slot_off = ((uint64_t)(uint32_t)uni(w0.y) << 32) | (uint32_t)uni(w0.x);
  r.p0 = uni(w0.z);
  r.mcount = uni(w0.w);
  r.fmt = (uint32_t)uni(w1.x);
  const int* wi = reinterpret_cast<const int*>(recs + g);
#pragma unroll
  for (int j = 0; j < MAX_MT; ++j) r.pair[j] = uni(wi[6 + j]);
  return r;
}

// Same tokens (FC1: the token of every pair; FC2: the pair itself, whose h is staged).
template <int MT, bool FC1>
__device__ __forceinline__ bool same_inputs(const RecS& x, const RecS& y, int k) {
  if (x.mcount != y.mcount) return false;
  bool eq = true;
#pragma unroll
  for (int j = 0; j < MT; ++j) eq = eq && (FC1 ? (x.pair[j] / k == y.pair[j] / k) : (x.pair[j] == y.pair[j]));
  return eq;
}

}  // namespace mvq
