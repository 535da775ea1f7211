// Top-k of one token and the one-token worklist, as device functions of the routing
// kernels.
//
// Routing reading: softmax over all experts, the k largest logits (equal logits -> lower
// expert id), weights renormalised over the chosen k (Tandem-vLLM 0.2.0 announcement, "How
// it works"; vLLM-Moet README, "What we changed against official vLLM", row "MoE at
// decode": router -> FC1 -> FC2).
#pragma once

#include "moe_vq_device.h"

namespace mvq {

// Top-k of one token by one wave: sum the slice partials (in slice order), then k
// rounds of argmax (greater logit, or equal logit and lower id).  Weights are
// exp(l_i - l_max) / sum_j exp(l_j - l_max) over the chosen k, which equals the
// softmax over all experts renormalised over the chosen k.  Lane i < k returns the
// i-th chosen id in *id_out and its weight in *w_out; with WRITE it also writes ids and
// weights to the outputs.
template <int NPL, bool WRITE = true>
__device__ __forceinline__ void topk_token(const RouteArgs& a, int t, int lane, int* id_out, float* w_out = nullptr) {
  const int KSP = a.ksp;
  const int NQ = KSP / 4;                      // 16-byte partial groups per expert (0: one float)
  constexpr int QMAX = MAX_DIM / SLICE / 4;    // at most 16 slices
  constexpr int IB = NPL < 4 ? NPL : (NPL >= 16 ? 2 : 4);  // experts per lane batched
  float v[NPL];
  // every partial of a batch is loaded before any is summed: a loop over the run-time
  // slice count would wait for each load in turn
#pragma unroll
  for (int i0 = 0; i0 < NPL; i0 += IB) {
    float4 f[IB][QMAX];
#pragma unroll
    for (int ii = 0; ii < IB; ++ii) {
      const int e = lane + 64 * (i0 + ii);
      const float4* src = reinterpret_cast<const float4*>(a.logits + ((size_t)t * a.E + e) * KSP);
#pragma unroll
      for (int q = 0; q < QMAX; ++q)
        f[ii][q] = (e < a.E && q < NQ) ? src[q] : make_float4(0.f, 0.f, 0.f, 0.f);
      if (NQ == 0)  // one complete logit per expert
        f[ii][0].x = e < a.E ? a.logits[(size_t)t * a.E + e] : 0.f;
    }
#pragma unroll
    for (int ii = 0; ii < IB; ++ii) {
      const int e = lane + 64 * (i0 + ii);
      float acc = -INFINITY;
      if (e < a.E) {
        acc = 0.f;
#pragma unroll
        for (int q = 0; q < QMAX; ++q)
          if (q < NQ) { acc += f[ii][q].x; acc += f[ii][q].y; acc += f[ii][q].z; acc += f[ii][q].w; }
        if (NQ == 0) acc = f[ii][0].x;
        if (acc != acc) acc = -INFINITY;  // NaN never wins
      }
      v[i0 + ii] = acc;
    }
  }
  // Each candidate is one 64-bit key: the order-preserving logit bits above, ~id
  // below, so that the unsigned maximum is the larger logit and, among equal logits,
  // the lower id.  Key 0 (below every real key) marks a taken or missing expert.
  uint64_t key[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < a.E ? ((uint64_t)f32_order_key(v[i]) << 32) | (uint32_t)~e : 0ull;
  }
  float my_l = -INFINITY, lmax = 0.f;
  int my_id = 0;
  for (int j = 0; j < a.k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int bid = (int)~(uint32_t)best;
    const float bl = f32_from_order_key((uint32_t)(best >> 32));
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (lane + 64 * i == bid) key[i] = 0;
    if (j == 0) lmax = bl;
    if (lane == j) { my_l = bl; my_id = bid; }
  }
  const float p = (lane < a.k) ? expf(my_l - lmax) : 0.f;
  const float tot = wave_sum(p);
  if (lane < a.k) {
    const float w = p / tot;
    if (WRITE) {
      a.topk_ids[(size_t)t * a.k + lane] = my_id;
      a.topk_w[(size_t)t * a.k + lane] = w;
      a.pair_w[(size_t)t * a.k + lane] = w;
    }
    *id_out = my_id;
    if (w_out) *w_out = w;
  }
}

// The one-token worklist (k <= 64, one token group per routed pair), by one wave: the
// top-k, the k experts ordered by id, their slots checked, and -- with write -- the same
// worklist as the many-token worklist kernel (experts ascending, one pair and one group of
// each list per expert) and the header.  Lane i < k returns its pick: the expert of pair i
// (pair index p = i; E + e for the FP4 copy of e when the delta cache holds one and the
// pair's weight reaches the confidence gate), its rank among the k listed experts, its
// slot offset and format (absent when the slot is missing, misaligned or outside the
// pool).
struct OneTokenPick {
  int id, rank;
  uint64_t off;
  uint32_t fmt;
};

template <int NPL>
__device__ __forceinline__ OneTokenPick one_token_pick(const RouteArgs& ra, const WorklistArgs& a, int lane,
                                                       bool write) {
  const int k = a.k;
  // every expert's slot is read before the top-k (expert lane + 64 i in lane's entry i),
  // so that looking the chosen ones up costs shuffles, not a memory round trip after it
  moe_vq_slot pre[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    pre[i] = e < a.E ? a.slots[e] : moe_vq_slot{};
  }
  int id = 0;
  float w = 0.f;
  if (write) topk_token<NPL, true>(ra, 0, lane, &id, &w);
  else topk_token<NPL, false>(ra, 0, lane, &id, &w);
  moe_vq_slot sl{};
  {
    const int src = id & 63, hi = id >> 6;  // (every lane takes part in the shuffles)
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const uint32_t lo32 = (uint32_t)__shfl((int)(uint32_t)pre[i].byte_offset, src);
      const uint32_t hi32 = (uint32_t)__shfl((int)(uint32_t)(pre[i].byte_offset >> 32), src);
      const uint32_t fm = (uint32_t)__shfl((int)pre[i].format, src);
      if (lane < k && hi == i) {
        sl.byte_offset = ((uint64_t)hi32 << 32) | lo32;
        sl.format = fm;
      }
    }
  }
  // FP4 delta cache: the pair takes its expert's copy (listed as E + e) when the cache
  // holds one and the pair's weight reaches the confidence gate
  int v = id;
  if (a.EV > a.E) {
    moe_vq_slot d{};
    if (lane < k && w >= a.tau) d = a.delta_slots[id];
    if (d.format != MOE_VQ_FMT_ABSENT) { v = a.E + id; sl = d; }
  }
  // rank of this lane's listed expert among the k (distinct) ones, in the many-token
  // worklist's order: by expert, each copy right after its expert
  const int order = a.EV > a.E ? 2 * id + (v != id ? 1 : 0) : id;
  int rank = 0;
  for (int j = 0; j < k; ++j) rank += __shfl(order, j) < order ? 1 : 0;
  uint32_t fmt = sl.format;
  const uint64_t off = sl.byte_offset;
  uint64_t need = 0;
  if (fmt == MOE_VQ_FMT_VQ2 || fmt == MOE_VQ_FMT_MXFP4) need = slot_layout((int)fmt, a.H, a.I).total;
  const bool ok = need != 0 && (off & 255) == 0 && off <= a.pool_bytes && need <= a.pool_bytes - off;
  if (!ok) fmt = MOE_VQ_FMT_ABSENT;
  if (write) {
    int bad = (lane < k && !ok) ? v : 0x7FFFFFFF;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) bad = min(bad, __shfl_xor(bad, d));
    if (lane < k) {
      a.pair_list[rank] = lane;
      a.act_expert[rank] = v;
      a.act_start[rank] = rank;
      a.act_off[rank] = off;
      a.act_fmt[rank] = fmt;
      a.grp1[rank] = rank;
      a.grp2[rank] = rank;
      GroupRec r;
      r.slot_off = off;
      r.p0 = rank;
      r.mcount = 1;
      r.fmt = fmt;
      r.expert = v;
#pragma unroll
      for (int j = 0; j < MAX_MT; ++j) r.pair[j] = lane;
#pragma unroll
      for (int j = 0; j < 4; ++j) r.pad[j] = 0;
      a.rec1[rank] = r;
      a.rec2[rank] = r;
    }
    if (lane == 0) {
      a.act_start[k] = k;
      a.grp1[k] = k;
      a.grp2[k] = k;
      a.hdr[HDR_STATUS] = bad != 0x7FFFFFFF ? MOE_VQ_ENOTRESIDENT : MOE_VQ_OK;
      a.hdr[HDR_INFO] = (uint32_t)(bad != 0x7FFFFFFF ? bad : -1);
      a.hdr[HDR_N_ACTIVE] = k;
      a.hdr[HDR_N_PAIRS] = k;
      a.hdr[HDR_N_TOKENS] = 1;
      a.hdr[HDR_GROUPS1] = k;
      a.hdr[HDR_GROUPS2] = k;
      a.hdr[HDR_MT1] = a.MT1;
      a.hdr[HDR_MT2] = a.MT2;
      a.hdr[HDR_KEY] = a.key;
      a.hdr[HDR_X_LO] = (uint32_t)(uintptr_t)a.x;
      a.hdr[HDR_X_HI] = (uint32_t)((uint64_t)(uintptr_t)a.x >> 32);
      a.hdr[HDR_X_DTYPE] = (uint32_t)a.x_dtype;
      a.hdr[HDR_PGRID1] = 0;  // (one-token groups: the matrix-core kernels do not run)
      a.hdr[HDR_PGRID2] = 0;
    }
  }
  return OneTokenPick{v, rank, off, fmt};
}

}  // namespace mvq
