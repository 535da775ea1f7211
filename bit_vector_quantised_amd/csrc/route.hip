// Routing kernels: router product, softmax / top-k / renormalise, expert worklist.
//
// Sources: the routed experts of a DeepSeek-style MoE layer are chosen per token
// from the router logits (Tandem-vLLM 0.2.0 announcement, "How it works"; vLLM-Moet
// README, "What we changed against official vLLM", row "MoE at decode": router ->
// FC1 -> FC2).  Routing reading: softmax over all experts, the k largest logits
// (equal logits -> lower expert id), weights renormalised over the chosen k.
#include "moe_vq_launch.h"
#include "topk_common.h"

namespace mvq {

constexpr int RT_EXPERTS = 8;   // experts per router workgroup (two per wave)
constexpr int RT_TOKENS = 32;   // tokens per router workgroup

// Partial router logits over one SLICE of H for RT_EXPERTS experts and up to
// RT_TOKENS tokens; lane l covers 16 consecutive columns.  Partials are stored
// [T][E][ksp] (slice fastest, ksp = slices rounded up to 4) so the top-k stage sums
// them with 16-byte loads.  (The matrix-core router writes complete logits, ksp = 1.)
// Workgroups of expert group 0 also stage x as fp16 with a power-of-two factor per
// (token, slice): x = x_h * x_sc exactly for bf16 inputs (|x_h| < 2^15; x_sc = 0 for an
// all-zero slice).
template <bool XF32>
__global__ __launch_bounds__(256) void router_gemv_kernel(RouteArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int s = blockIdx.y;
  const int c0 = s * SLICE + lane * 16;
  const bool col_ok = c0 < a.H;  // H % 128 == 0, so a lane's 16 columns are all in or all out
  const int e0 = blockIdx.x * RT_EXPERTS + wave * 2;
  const int t0 = blockIdx.z * RT_TOKENS;
  const int t1 = min(a.T, t0 + RT_TOKENS);
  const int KSP = a.ksp;

  uint4 w[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = e0 + j;
    if (col_ok && e < a.E) {
      const uint4* p = reinterpret_cast<const uint4*>(a.router_w + (size_t)e * a.H + c0);
      w[j][0] = p[0];
      w[j][1] = p[1];
    } else {
      w[j][0] = w[j][1] = make_uint4(0, 0, 0, 0);
    }
  }
  const bool stage = (blockIdx.x == 0);

  // Tokens in batches of TB: every x load of a batch is issued before any is used, so a
  // batch waits for one memory latency, not one per token.
  constexpr int TB = XF32 ? 4 : 8;
  for (int tb = t0; tb < t1; tb += TB) {
    uint4 xv[TB][XF32 ? 4 : 2];  // a lane's 16 columns: bf16 (2 units) or fp32 (4 units)
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      const int t = tb + u;
#pragma unroll
      for (int q = 0; q < (XF32 ? 4 : 2); ++q) xv[u][q] = make_uint4(0, 0, 0, 0);
      if (col_ok && t < t1) {
        const uint4* px = XF32 ? reinterpret_cast<const uint4*>(static_cast<const float*>(a.x) + (size_t)t * a.H + c0)
                               : reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + (size_t)t * a.H + c0);
#pragma unroll
        for (int q = 0; q < (XF32 ? 4 : 2); ++q) xv[u][q] = px[q];
      }
    }
    // a lane's 16 x values of token u as fp32
    auto xval = [&](int u, float (&xf)[16]) __attribute__((always_inline)) {
      if (XF32) {
        const float* f = reinterpret_cast<const float*>(&xv[u][0]);
#pragma unroll
        for (int q = 0; q < 16; ++q) xf[q] = f[q];
      } else {
        const uint32_t* xw = reinterpret_cast<const uint32_t*>(&xv[u][0]);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          xf[2 * q] = bf16_bits_to_f32(xw[q] & 0xFFFFu);
          xf[2 * q + 1] = bf16_bits_to_f32(xw[q] >> 16);
        }
      }
    };
    float d[TB][2];
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      d[u][0] = d[u][1] = 0.f;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t* wj = reinterpret_cast<const uint32_t*>(&w[j][0]);
        if (XF32) {
          float xf[16];
          xval(u, xf);
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            d[u][j] = fmaf(bf16_bits_to_f32(wj[q] & 0xFFFFu), xf[2 * q], d[u][j]);
            d[u][j] = fmaf(bf16_bits_to_f32(wj[q] >> 16), xf[2 * q + 1], d[u][j]);
          }
        } else {
          const uint32_t* xw = reinterpret_cast<const uint32_t*>(&xv[u][0]);
#pragma unroll
          for (int q = 0; q < 8; ++q)
            d[u][j] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wj[q]),
                                                      __builtin_bit_cast(bf16x2_t, xw[q]), d[u][j], false);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      d[u][0] = wave_sum(d[u][0]);
      d[u][1] = wave_sum(d[u][1]);
    }
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      const int t = tb + u;
      if (lane == 0 && t < t1) {
        float* dst = a.logits + (size_t)t * a.E * KSP;
        if (e0 < a.E) dst[(size_t)e0 * KSP + s] = d[u][0];
        if (e0 + 1 < a.E) dst[(size_t)(e0 + 1) * KSP + s] = d[u][1];
        if (s == a.KS - 1) {  // zero the padding slices once
          for (int z = a.KS; z < KSP; ++z) {
            if (e0 < a.E) dst[(size_t)e0 * KSP + z] = 0.f;
            if (e0 + 1 < a.E) dst[(size_t)(e0 + 1) * KSP + z] = 0.f;
          }
        }
      }
    }
    if (stage) {
#pragma unroll
      for (int u = 0; u < TB; ++u) {
        const int t = tb + u;
        if (t < t1 && wave == (t & 3)) {
          float xf[16];
          xval(u, xf);
          float m = 0.f;
#pragma unroll
          for (int q = 0; q < 16; ++q) m = fmaxf(m, fabsf(xf[q]));
          m = wave_max(m);
          int ex = 0;
          if (m > 0.f && m == m) {
            int e2;
            frexpf(m, &e2);  // m < 2^e2
            ex = e2 - 15;    // |x| * 2^-ex < 2^15
          }
          if (col_ok) {
            uint32_t packed[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const _Float16 lo = (_Float16)ldexpf(xf[2 * q], -ex);
              const _Float16 hi = (_Float16)ldexpf(xf[2 * q + 1], -ex);
              packed[q] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
            }
            uint4* dst = reinterpret_cast<uint4*>(a.x_h + (size_t)t * a.H + c0);
            dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
            dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
          }
          // (an all-zero slice has factor 0, so that it never sets a common factor)
          if (lane == 0) a.x_sc[(size_t)t * a.KS + s] = m == 0.f ? 0.f : ldexpf(1.0f, ex);
        }
      }
    }
  }
}

template <int NPL>
__global__ __launch_bounds__(256) void topk_kernel(RouteArgs a) {
  asm volatile("" ::"s"(a.logits), "s"(a.pair_w));  // both argument lines at the start
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= a.T) return;
  int id;
  topk_token<NPL>(a, t, lane, &id);
}

constexpr int FUSED_TOPK_MAX_T = 16;
constexpr int PL_LDS = 2048;  // pair lists up to this length are also kept in LDS

// Single workgroup: (optionally the top-k of every token, one wave per token), then
// group the routed pairs by expert (stable: ascending pair index p = t*k + i within an
// expert), list the distinct experts in ascending id with their slot lookups, write
// the FC token-group records, and validate every selected slot.  With an FP4 delta
// cache (a.EV = 2E) a pair whose weight passes the confidence gate, and whose expert has
// a copy, is listed under the copy, expert E + e, whose slot is delta_slots[e]
// (vLLM-Moet README, "2-bit experts on vLLM v0.24.0": a delta cache and a confidence
// gate bring FP4 back where it matters).  Each copy is listed right after its expert
// (thread / counter index 2e + 1, the expert itself 2e), so that the FC kernels, which
// hand each workgroup a contiguous run of tiles in listing order, spread the copies'
// heavier tiles over the grid instead of giving them all to the last workgroups.
template <bool FUSED, int NPL>
__global__ __launch_bounds__(1024) void worklist_kernel(RouteArgs ra, WorklistArgs a) {
  __shared__ int cnt[16 * MAX_E];
  __shared__ int ids_lds[FUSED ? FUSED_TOPK_MAX_T * MAX_K : 1];
  __shared__ float w_lds[FUSED ? FUSED_TOPK_MAX_T * MAX_K : 1];
  __shared__ uint8_t has_copy[MAX_E / 2];
  __shared__ int4 wave_tot[16];
  __shared__ int4 s_total;
  __shared__ int s_bad_expert;
  __shared__ int s_bad_id;
  __shared__ int pl_lds[PL_LDS];
  // per active expert, by rank: first pair, pair count, group prefixes, slot
  __shared__ int r_start[MAX_E], r_tot[MAX_E], r_gs1[MAX_E], r_gs2[MAX_E], r_expert[MAX_E];
  __shared__ uint32_t r_fmt[MAX_E];
  __shared__ uint64_t r_off[MAX_E];
  __shared__ int r_wc1[MAX_E], r_wc2[MAX_E];  // tile-cost prefixes (the matrix-core split)
  __shared__ int4 s_cost;
  // all four scalar-cache lines of the arguments read at the start, together
  asm volatile("" ::"s"(ra.logits), "s"(a.slots), "s"(a.hdr), "s"(a.rec1));
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int E = a.E, EV = a.EV, T = a.T, k = a.k;
  const bool dc = EV > E;  // delta cache: index 2e is expert e, 2e + 1 its copy
  const int my_e = dc ? tid >> 1 : tid;
  const bool my_copy = dc && (tid & 1);
  const int my_id = my_copy ? E + my_e : my_e;  // the id the worklist reports
  // the slot of (listed) expert tid is read first, so that its latency overlaps the top-k
  moe_vq_slot sl{};
  if (tid < EV) sl = my_copy ? a.delta_slots[my_e] : a.slots[my_e];
  // counting waves: wave w takes tokens [w*C, (w+1)*C), with as many waves as tokens
  // (up to 16), so that the per-expert totals sum over no more waves than needed
  const int NWC = T < 16 ? (T > 1 ? T : 1) : 16;
  const int C = (T + NWC - 1) / NWC;
  for (int i = tid; i < NWC * EV; i += 1024) cnt[i] = 0;
  if (tid == 0) { s_bad_expert = 0x7FFFFFFF; s_bad_id = 0; }
  if (my_copy && tid < EV) has_copy[my_e] = sl.format != MOE_VQ_FMT_ABSENT;
  if (FUSED) {
    for (int t = wave; t < T; t += 16) {
      int id = 0;
      float w = 0.f;
      topk_token<NPL>(ra, t, lane, &id, &w);
      if (lane < k) { ids_lds[t * k + lane] = id; w_lds[t * k + lane] = w; }
    }
  }
  __syncthreads();
  auto id_of = [&](int p) -> int { return FUSED ? ids_lds[p] : a.topk_ids[p]; };
  // the counter index of the expert pair p (of expert e) is listed under: with the
  // cache, 2e + 1 (the copy) when the cache holds one and the pair's routing weight
  // reaches the gate, else 2e
  auto listed = [&](int p, int e) -> int {
    if (!dc) return e;
    if (!has_copy[e]) return 2 * e;
    return (FUSED ? w_lds[p] : a.pair_w[p]) >= a.tau ? 2 * e + 1 : 2 * e;
  };
  const int tb = min(T, wave * C), te = min(T, tb + C);
  for (int p = tb * k + lane; p < te * k; p += 64) {
    const int e = id_of(p);
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[wave * EV + listed(p, e)], 1);
    else s_bad_id = 1;
  }
  __syncthreads();
  int tot = 0;
  if (tid < EV)
    for (int w = 0; w < NWC; ++w) tot += cnt[w * EV + tid];
  const int g1 = (tot + a.MT1 - 1) / a.MT1;
  const int g2 = (tot + a.MT2 - 1) / a.MT2;
  const int4 sc = block_scan_excl4(make_int4(tot, tot > 0 ? 1 : 0, g1, g2), wave_tot, &s_total);
  const int start = sc.x, rank = sc.y, gs1 = sc.z, gs2 = sc.w;
  uint32_t my_fmt = MOE_VQ_FMT_ABSENT;
  if (tid < EV && tot > 0) {
    uint32_t fmt = sl.format;
    const uint64_t off = sl.byte_offset;
    uint64_t need = 0;
    if (fmt == MOE_VQ_FMT_VQ2 || fmt == MOE_VQ_FMT_MXFP4) need = slot_layout((int)fmt, a.H, a.I).total;
    const bool ok = need != 0 && (off & 255) == 0 && off <= a.pool_bytes && need <= a.pool_bytes - off;
    if (!ok) {
      fmt = MOE_VQ_FMT_ABSENT;
      atomicMin(&s_bad_expert, my_id);
    }
    a.act_expert[rank] = my_id;
    a.act_start[rank] = start;
    a.act_off[rank] = off;
    a.act_fmt[rank] = fmt;
    a.grp1[rank] = gs1;
    a.grp2[rank] = gs2;
    r_start[rank] = start; r_tot[rank] = tot; r_gs1[rank] = gs1; r_gs2[rank] = gs2;
    r_expert[rank] = my_id; r_fmt[rank] = fmt; r_off[rank] = off;
    my_fmt = fmt;
  }
  if (tid == 0) {
    const int n_active = s_total.y;
    a.act_start[n_active] = s_total.x;
    a.grp1[n_active] = s_total.z;
    a.grp2[n_active] = s_total.w;
  }
  // per-wave bases: cnt[w][e] <- start[e] + sum_{w' < w} cnt[w'][e]
  if (tid < EV) {
    int run = start;
    for (int w = 0; w < NWC; ++w) {
      const int c = cnt[w * EV + tid];
      cnt[w * EV + tid] = run;
      run += c;
    }
  }
  __syncthreads();
  // stable placement: each wave walks its tokens in order; the k experts of one token
  // are distinct, so the k lanes never collide on a counter.
  for (int t = tb; t < te; ++t) {
    if (lane < k) {
      const int p = t * k + lane;
      const int e = id_of(p);
      if ((unsigned)e < (unsigned)E) {
        const int pos = atomicAdd(&cnt[wave * EV + listed(p, e)], 1);
        a.pair_list[pos] = p;
        pl_lds[pos < PL_LDS ? pos : 0] = p;
      }
    }
  }
  __syncthreads();
  // token-group records: group g of a list belongs to the active expert of largest
  // rank whose group prefix is <= g (found by bisection over the LDS prefixes)
  const int n_act = s_total.y, G1n = s_total.z, G2n = s_total.w;
  const bool pl_in_lds = T * k <= PL_LDS;
  for (int gg = tid; gg < G1n + G2n; gg += 1024) {
    const bool one = gg < G1n;
    const int g = one ? gg : gg - G1n;
    if (g >= (one ? a.G1 : a.G2)) continue;
    const int* gs = one ? r_gs1 : r_gs2;
    const int MT = one ? a.MT1 : a.MT2;
    int lo = 0, hi = n_act - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (gs[mid] <= g) lo = mid; else hi = mid - 1;
    }
    const int gi = g - gs[lo];
    GroupRec r;
    r.slot_off = r_off[lo];
    r.p0 = r_start[lo] + gi * MT;
    r.mcount = min(MT, r_tot[lo] - gi * MT);
    r.fmt = r_fmt[lo];
    r.expert = r_expert[lo];
#pragma unroll
    for (int j = 0; j < MAX_MT; ++j) {
      const int q = r.p0 + (j < r.mcount ? j : r.mcount - 1);
      r.pair[j] = pl_in_lds ? pl_lds[q] : a.pair_list[q];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) r.pad[j] = 0;
    (one ? a.rec1 : a.rec2)[g] = r;
  }
  // The matrix-core FC kernels' tiles split over their grids by cost: boundary b of a
  // grid of n is the tile where the cost prefix reaches b / n of the total (each listed
  // expert's tiles cost part_cost(format) apiece, in listing order).  Only a step that
  // lists both formats needs it: with one format equal costs are equal counts, which the
  // kernels take by themselves when the header records no split.
  const bool listed_here = tid < EV && tot > 0;
  const bool mixed = __syncthreads_or(listed_here && my_fmt == MOE_VQ_FMT_MXFP4) &&
                     __syncthreads_or(listed_here && my_fmt == MOE_VQ_FMT_VQ2);
  const int pgrid1 = mixed ? a.grid1 : 0, pgrid2 = mixed ? a.grid2 : 0;
  if (mixed && (pgrid1 > 0 || pgrid2 > 0)) {
    const int wt = listed_here ? part_cost(my_fmt) : 0;
    const int4 cs = block_scan_excl4(make_int4(g1 * a.rb1 * wt, g2 * a.rb2 * wt, 0, 0), wave_tot, &s_cost);
    if (tid < EV && tot > 0) { r_wc1[rank] = cs.x; r_wc2[rank] = cs.y; }
    __syncthreads();
    auto split = [&](int grid, int rb, const int* wc, const int* gs, int G, int C, int32_t* out) {
      for (int b = tid; b <= grid; b += 1024) {
        // floor(b C / grid): exact in double (b C < 2^53, and a quotient that is not an
        // integer lies at least 1 / grid from one)
        const int target = (int)floor((double)b * (double)C / (double)grid);
        int tile = 0;
        if (n_act > 0) {
          int lo = 0, hi = n_act - 1;  // the last listed expert whose prefix is <= target
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (wc[mid] <= target) lo = mid; else hi = mid - 1;
          }
          const int w = part_cost(r_fmt[lo]);
          const int nt = ((lo + 1 < n_act ? gs[lo + 1] : G) - gs[lo]) * rb;
          const int in = (target - wc[lo] + w - 1) / w;
          tile = gs[lo] * rb + (in < nt ? in : nt);
        }
        out[b] = tile;
      }
    };
    if (pgrid1 > 0) split(pgrid1, a.rb1, r_wc1, r_gs1, G1n, s_cost.x, a.part1);
    if (pgrid2 > 0) split(pgrid2, a.rb2, r_wc2, r_gs2, G2n, s_cost.y, a.part2);
  }
  if (tid == 0) {
    uint32_t status = MOE_VQ_OK;
    int info = -1;
    if (s_bad_expert != 0x7FFFFFFF) { status = MOE_VQ_ENOTRESIDENT; info = s_bad_expert; }
    if (s_bad_id) { status = MOE_VQ_EINVAL; }
    a.hdr[HDR_STATUS] = status;
    a.hdr[HDR_INFO] = (uint32_t)info;
    a.hdr[HDR_N_ACTIVE] = s_total.y;
    a.hdr[HDR_N_PAIRS] = s_total.x;
    a.hdr[HDR_N_TOKENS] = T;
    a.hdr[HDR_GROUPS1] = s_total.z;
    a.hdr[HDR_GROUPS2] = s_total.w;
    a.hdr[HDR_MT1] = a.MT1;
    a.hdr[HDR_MT2] = a.MT2;
    a.hdr[HDR_KEY] = a.key;
    a.hdr[HDR_X_LO] = (uint32_t)(uintptr_t)a.x;
    a.hdr[HDR_X_HI] = (uint32_t)((uint64_t)(uintptr_t)a.x >> 32);
    a.hdr[HDR_X_DTYPE] = (uint32_t)a.x_dtype;
    a.hdr[HDR_PGRID1] = (uint32_t)pgrid1;
    a.hdr[HDR_PGRID2] = (uint32_t)pgrid2;
  }
}

// ---------------------------------------------------------------------------------------
// Many tokens: the router product on the matrix cores, and the fp16 staging of x
// ---------------------------------------------------------------------------------------

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float rf32x4_t __attribute__((ext_vector_type(4)));

constexpr int RM_TOKENS = 64;   // tokens per workgroup (16 per wave)
constexpr int RM_EXPERTS = 64;  // experts per workgroup (4 blocks of 16)
constexpr int RM_MIN_T = 64;    // from this many bf16 tokens on, the matrix-core router

// logits[t][e] = sum_h W_r[e][h] x[t][h] for bf16 x with v_mfma_f32_16x16x32_bf16 (bf16
// products are exact in fp32; fp32 accumulation).  Wave w of a workgroup takes tokens
// 16w..16w+15 of its 64 and all 64 of its experts; both operands are read straight from
// global memory, 16 bytes per lane and step (A: token row, B: expert row).  Rows past T
// or E re-read the last row and are not written.
__global__ __launch_bounds__(256) void router_mfma_kernel(RouteArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i16 = lane & 15, kq = lane >> 4;
  const int t0 = blockIdx.x * RM_TOKENS + wave * 16;
  const int e0 = blockIdx.y * RM_EXPERTS;
  const int H = a.H;
  const uint16_t* xr = static_cast<const uint16_t*>(a.x) + (size_t)min(t0 + i16, a.T - 1) * H + 8 * kq;
  const uint16_t* wr[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) wr[nb] = a.router_w + (size_t)min(e0 + nb * 16 + i16, a.E - 1) * H + 8 * kq;
  rf32x4_t acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = rf32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < H; k += 128) {
    bf16x8_t af[4], bf[4][4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      af[s] = *reinterpret_cast<const bf16x8_t*>(xr + k + 32 * s);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) bf[s][nb] = *reinterpret_cast<const bf16x8_t*>(wr[nb] + k + 32 * s);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s], bf[s][nb], acc[nb], 0, 0, 0);
  }
  // D: lane holds expert column i16 and token rows 4*kq + 0..3 of each block
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + 4 * kq + r, e = e0 + nb * 16 + i16;
      if (t < a.T && e < a.E) a.logits[(size_t)t * a.E + e] = acc[nb][r];
    }
}

// x as fp16 with one power-of-two factor per (token, 1024-column slice), for the
// decode-path FC kernels (exact for bf16 x): one wave per (token, slice), 16 columns
// per lane.
template <bool XF32>
__device__ __forceinline__ void stage_x_row(const RouteArgs& a, int t, int s, int lane) {
  const int c0 = s * SLICE + lane * 16;
  const bool col_ok = c0 < a.H;
  float xf[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) xf[q] = 0.f;
  if (col_ok) {
    if (XF32) {
      const float4* px = reinterpret_cast<const float4*>(static_cast<const float*>(a.x) + (size_t)t * a.H + c0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = px[q];
        xf[4 * q] = v.x; xf[4 * q + 1] = v.y; xf[4 * q + 2] = v.z; xf[4 * q + 3] = v.w;
      }
    } else {
      const uint4* px = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + (size_t)t * a.H + c0);
      const uint4 xv[2] = {px[0], px[1]};
      const uint32_t* xw = reinterpret_cast<const uint32_t*>(xv);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        xf[2 * q] = bf16_bits_to_f32(xw[q] & 0xFFFFu);
        xf[2 * q + 1] = bf16_bits_to_f32(xw[q] >> 16);
      }
    }
  }
  float m = 0.f;
#pragma unroll
  for (int q = 0; q < 16; ++q) m = fmaxf(m, fabsf(xf[q]));
  m = wave_max(m);
  int ex = 0;
  if (m > 0.f && m == m) ex = frexp_exponent(m) - 15;  // |x| * 2^-ex < 2^15
  if (col_ok) {
    uint32_t packed[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const _Float16 lo = (_Float16)ldexp2(xf[2 * q], -ex), hi = (_Float16)ldexp2(xf[2 * q + 1], -ex);
      packed[q] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    uint4* dst = reinterpret_cast<uint4*>(a.x_h + (size_t)t * a.H + c0);
    dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  }
  // (an all-zero slice has factor 0, so that it never sets a common factor)
  if (lane == 0) a.x_sc[(size_t)t * a.KS + s] = m == 0.f ? 0.f : ldexp2(1.0f, ex);
}

template <bool XF32>
__global__ __launch_bounds__(64) void stage_x_kernel(RouteArgs a) {
  stage_x_row<XF32>(a, blockIdx.x, blockIdx.y, threadIdx.x);
}

// Fewer tokens than the matrix-core router takes (bf16 x): the product split over K as the
// GEMV router splits it, on the matrix cores.  Workgroup (expert block of RS_EXPERTS,
// slice of 1024 columns); wave w takes 256 columns of the slice for every token block of
// 16.  Eight experts per workgroup rather than the matrix op's 16 columns: twice the
// workgroups (224 for 256 experts and H = 7168), each reading half the weights, so that
// more compute units share the router's read.  Its
// loads (weights and x) are all issued before the first matrix op, so a workgroup waits
// for one memory latency.  The four waves' sums meet in LDS in a fixed order, and the
// slice's partial logit goes where the GEMV router puts it ([T][E][ksp]).  The workgroups
// of a slice also stage its x as fp16 for the FC kernels.
constexpr int RS_EXPERTS = 8;  // experts per workgroup: the matrix op's other 8 columns are zeros
constexpr int RS_MAX_T = 64;  // token blocks of 16, at most four

__global__ __launch_bounds__(256) void router_mfma_small_kernel(RouteArgs a) {
  __shared__ float red[4][RS_MAX_T / 16][16][17];
  // the argument lines and the grid size (a hidden argument) read at the start together
  asm volatile("" ::"s"(a.x_h), "s"(a.pair_w), "s"(gridDim.x));
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i16 = lane & 15, kq = lane >> 4;
  const int e0 = blockIdx.x * RS_EXPERTS, s = blockIdx.y;
  const int T = a.T, H = a.H, MB = (T + 15) / 16;
  const int c0 = s * SLICE + wave * 256 + 8 * kq;  // + 32 j: 8 columns, all in or all out (H % 128 == 0)
  const uint16_t* xb = static_cast<const uint16_t*>(a.x);
  const bool col_ok = i16 < RS_EXPERTS;  // matrix-op columns past the workgroup's experts stay zero
  const uint16_t* wr = a.router_w + (size_t)min(e0 + (col_ok ? i16 : 0), a.E - 1) * H;
  const bf16x8_t zero = bf16x8_t{};
  bf16x8_t bfr[8], afr[RS_MAX_T / 16][8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = c0 + 32 * j;
    bfr[j] = (col_ok && c < H) ? *reinterpret_cast<const bf16x8_t*>(wr + c) : zero;
  }
#pragma unroll
  for (int mb = 0; mb < RS_MAX_T / 16; ++mb) {
    const uint16_t* xr = xb + (size_t)min(mb * 16 + i16, T - 1) * H;  // rows past T re-read the last
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = c0 + 32 * j;
      afr[mb][j] = (mb < MB && c < H) ? *reinterpret_cast<const bf16x8_t*>(xr + c) : zero;
    }
  }
  // D: lane holds expert column i16 and token rows 4 kq + 0..3 of each token block
#pragma unroll
  for (int mb = 0; mb < RS_MAX_T / 16; ++mb) {
    if (mb < MB) {
      rf32x4_t acc = rf32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[mb][j], bfr[j], acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][mb][4 * kq + r][i16] = acc[r];
    }
  }
  __syncthreads();
  const int KSP = a.ksp;
  for (int o = tid; o < MB * 256; o += 256) {
    const int mb = o >> 8, row = (o >> 4) & 15, col = o & 15;
    const int t = mb * 16 + row, e = e0 + col;
    if (t < T && col < RS_EXPERTS && e < a.E) {
      const float v = ((red[0][mb][row][col] + red[1][mb][row][col]) + red[2][mb][row][col]) + red[3][mb][row][col];
      float* dst = a.logits + ((size_t)t * a.E + e) * KSP;
      dst[s] = v;
      if (s == a.KS - 1)
        for (int z = a.KS; z < KSP; ++z) dst[z] = 0.f;  // the padding slices
    }
  }
  // the slice's staging, spread over the workgroups of the slice: at most one token per
  // wave up to 4 * E / RS_EXPERTS tokens (each token is a memory round trip)
  for (int t = blockIdx.x * 4 + wave; t < T; t += gridDim.x * 4) stage_x_row<false>(a, t, s, lane);
}

// One-token step (k <= 64, one token group per routed pair): one wave does the top-k,
// orders the k experts by id, checks their slots and writes the same worklist as
// worklist_kernel, with a few memory round trips instead of a 1024-thread workgroup's phases.
template <int NPL>
__global__ __launch_bounds__(64) void worklist_one_kernel(RouteArgs ra, WorklistArgs a) {
  // The two argument structs span four scalar-cache lines; all are read here, at the
  // start, rather than each first where it is used (after the top-k), behind a miss.
  asm volatile("" ::"s"(ra.logits), "s"(a.slots), "s"(a.hdr), "s"(a.rec1));
  (void)one_token_pick<NPL>(ra, a, threadIdx.x, true);
}

template <int NPL>
static void launch_topk_worklist(const RouteArgs& ra, const WorklistArgs& wa, hipStream_t st) {
  if (ra.T == 1 && ra.k <= 64 && wa.MT1 == 1 && wa.MT2 == 1 && wa.G1 >= ra.k && wa.G2 >= ra.k) {
    worklist_one_kernel<NPL><<<1, 64, 0, st>>>(ra, wa);
  } else if (ra.T <= FUSED_TOPK_MAX_T) {
    worklist_kernel<true, NPL><<<1, 1024, 0, st>>>(ra, wa);
  } else {
    topk_kernel<NPL><<<(ra.T + 3) / 4, 256, 0, st>>>(ra);
    worklist_kernel<false, NPL><<<1, 1024, 0, st>>>(ra, wa);
  }
}

hipError_t launch_route(const RouteArgs& ra, int x_dtype, const WorklistArgs& wa, hipStream_t st) {
  (void)hipGetLastError();  // start from a clean error state: report only our own launches
  if (x_dtype == MOE_VQ_BF16 && ra.T >= RM_MIN_T) {
    RouteArgs rm = ra;
    rm.ksp = 1;
    stage_x_kernel<false><<<dim3(rm.T, rm.KS), 64, 0, st>>>(rm);
    router_mfma_kernel<<<dim3((rm.T + RM_TOKENS - 1) / RM_TOKENS, (rm.E + RM_EXPERTS - 1) / RM_EXPERTS), 256, 0, st>>>(rm);
    const int npl = (rm.E + 63) / 64;
    if (npl <= 1) launch_topk_worklist<1>(rm, wa, st);
    else if (npl <= 2) launch_topk_worklist<2>(rm, wa, st);
    else if (npl <= 4) launch_topk_worklist<4>(rm, wa, st);
    else if (npl <= 8) launch_topk_worklist<8>(rm, wa, st);
    else launch_topk_worklist<16>(rm, wa, st);
    return hipGetLastError();
  }
  dim3 g1((ra.E + RT_EXPERTS - 1) / RT_EXPERTS, ra.KS, (ra.T + RT_TOKENS - 1) / RT_TOKENS);
  if (x_dtype == MOE_VQ_BF16 && ra.T >= 1 && ra.T <= RS_MAX_T)
    router_mfma_small_kernel<<<dim3((ra.E + RS_EXPERTS - 1) / RS_EXPERTS, ra.KS), 256, 0, st>>>(ra);
  else if (x_dtype == MOE_VQ_F32)
    router_gemv_kernel<true><<<g1, 256, 0, st>>>(ra);
  else
    router_gemv_kernel<false><<<g1, 256, 0, st>>>(ra);
  const int npl = (ra.E + 63) / 64;
  if (npl <= 1) launch_topk_worklist<1>(ra, wa, st);
  else if (npl <= 2) launch_topk_worklist<2>(ra, wa, st);
  else if (npl <= 4) launch_topk_worklist<4>(ra, wa, st);
  else if (npl <= 8) launch_topk_worklist<8>(ra, wa, st);
  else launch_topk_worklist<16>(ra, wa, st);
  return hipGetLastError();
}

}  // namespace mvq
