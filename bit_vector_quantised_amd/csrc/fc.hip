// Decode-path expert kernels: FC1 (gate/up) with SiLU*up fused, and FC2 (down) with
// the weighted combine.  Expert weights stream from HBM as VQ2 words or MXFP4
// nibbles with 16-byte loads, are decoded in registers (VQ2 through the signed
// codebook table in LDS, MXFP4 with the gfx950 FP4->FP16 convert) and reduced with
// v_dot2_f32_f16 into fp32 accumulators, then across the lanes of a row with
// butterfly shuffles.
//
// Sources: the routed experts are 2-bit vector codes decoded on the fly (Tandem-vLLM
// 0.2.0 announcement, "How it works"; vLLM-Moet README, "2-bit experts on vLLM
// v0.24.0": sign-symmetric codebook); FC1 then FC2 per expert with no padding of
// experts to a fixed row count (vLLM-Moet README, "What we changed against official
// vLLM", row "MoE at decode"); silu*up fused into the routed-expert GEMV (vLLM-Moet
// README, "Qwen3.8-Flash-Next-FP8 on 4x RTX PRO 6000"); the 52 most-routed experts
// kept in FP4 (Tandem-vLLM announcement, "Quality vs the official FP4 checkpoint").
//
// Work decomposition.  The worklist lists the distinct selected experts; the tokens
// of one expert are cut into groups of at most MT tokens, each described by one
// GroupRec.  A tile is (token group, block of rows).  LPR lanes share one row (lane
// `sub` takes 16-byte chunks sub, sub+LPR, ...), every decoded chunk is applied to all
// tokens of the group, so each code byte is read from HBM once per token group.
//
// Two kernels:
//  * fc_stream_kernel (K = 1024, 2048 or 7168): a persistent grid; each
//    workgroup walks a contiguous run of tiles with two register buffers, issuing the
//    next tile's 14 x 16-byte loads per lane before decoding the current tile, so the
//    code stream stays in flight while the LDS lookups run.  The decode table and the
//    staged activations are built once and restaged only when the token group changes.
//  * fc_generic_kernel (any K multiple of 128): a persistent grid that prefetches one
//    chunk ahead; used for the shapes the tile kernel does not cover.
#include "fc_common.h"

#include <type_traits>

namespace mvq {

constexpr int LB_VQ = 14;   // 16-byte code loads in flight per lane (VQ2 tiles)
constexpr int LB_MX = 14;   // same budget for MXFP4 tiles (twice the bytes per weight)

// -------------------------------------------------------------------------------------
// fc_stream_kernel: K = 1024 * CPL, LPR = 16, persistent and software-pipelined
// -------------------------------------------------------------------------------------

template <int CPL, int MT, bool FC1>
struct TileGeom {
  static constexpr int NM = FC1 ? 2 : 1;
  static constexpr int RPL_RAW = FC1 ? LB_VQ / (2 * CPL) : LB_VQ / CPL;
  // a token group of MT > 1 holds NM * RPL * MT accumulators: fewer rows per lane
  static constexpr int RPL_CAP = MT > 1 ? 4 : (CPL == 1 ? 8 / NM : 16);
  static constexpr int RPL = RPL_RAW < 1 ? 1 : (RPL_RAW > RPL_CAP ? RPL_CAP : RPL_RAW);  // rows per lane
  static constexpr int ROWS = 16 * RPL;                              // rows per tile
  static constexpr int MXC = 2 * CPL;                                // MXFP4 chunks per lane per row
  static constexpr int RPP_MX_RAW = LB_MX / (NM * MXC);
  static constexpr int RPP_MX = RPP_MX_RAW < 1 ? 1 : (RPP_MX_RAW > RPL ? RPL : RPP_MX_RAW);
};

// The code words and scales one lane reads for one VQ2 tile.
template <int CPL, int MT, bool FC1>
struct VqBuf {
  uint4 q[TileGeom<CPL, MT, FC1>::RPL][TileGeom<CPL, MT, FC1>::NM][CPL];
  uint32_t s[TileGeom<CPL, MT, FC1>::RPL][TileGeom<CPL, MT, FC1>::NM][CPL];
};

// The loads of one (row, chunk) of a VQ2 tile: both matrices' 16 code bytes and scale.
template <int CPL, int MT, bool FC1>
__device__ __forceinline__ void issue_vq_chunk(VqBuf<CPL, MT, FC1>& b, const FcArgs& a, const RecS& r, int rb,
                                               int NROWS, int wave, int rg, int sub, int rr, int j) {
  using G = TileGeom<CPL, MT, FC1>;
  constexpr int K = 1024 * CPL;
  const uint8_t* slot = a.pool + r.slot_off;
  const uint8_t* qb0 = slot + (FC1 ? a.vq2.q_gate : a.vq2.q_down);
  const uint8_t* qb1 = slot + a.vq2.q_up;
  const uint8_t* sb0 = slot + (FC1 ? a.vq2.s_gate : a.vq2.s_down);
  const uint8_t* sb1 = slot + a.vq2.s_up;
  const int n = min(rb * G::ROWS + rr * 16 + wave * 4 + rg, NROWS - 1);
  const uint32_t qo = (uint32_t)n * (K / 4) + (uint32_t)sub * 16;
  const uint32_t so = (uint32_t)n * (K / 64) + (uint32_t)(sub >> 1) * 2;
#pragma unroll
  for (int m = 0; m < G::NM; ++m) {
    b.q[rr][m][j] = *reinterpret_cast<const uint4*>((m == 0 ? qb0 : qb1) + qo + j * 256);
    b.s[rr][m][j] = *reinterpret_cast<const uint16_t*>((m == 0 ? sb0 : sb1) + so + j * 16);
  }
}

template <int CPL, int MT, bool FC1>
__device__ __forceinline__ void issue_vq(VqBuf<CPL, MT, FC1>& b, const FcArgs& a, const RecS& r, int rb,
                                         int NROWS, int wave, int rg, int sub) {
  using G = TileGeom<CPL, MT, FC1>;
  constexpr int K = 1024 * CPL;
  // uniform matrix bases + one 32-bit per-lane row offset; the chunk offset j*256 (and
  // the scale offset j*16) is an immediate of the load instruction
  const uint8_t* slot = a.pool + r.slot_off;
  const uint8_t* qb0 = slot + (FC1 ? a.vq2.q_gate : a.vq2.q_down);
  const uint8_t* qb1 = slot + a.vq2.q_up;
  const uint8_t* sb0 = slot + (FC1 ? a.vq2.s_gate : a.vq2.s_down);
  const uint8_t* sb1 = slot + a.vq2.s_up;
#pragma unroll
  for (int rr = 0; rr < G::RPL; ++rr) {
    // rows past the end (ragged shapes only) re-read the last row; finish() drops them
    const int n = min(rb * G::ROWS + rr * 16 + wave * 4 + rg, NROWS - 1);
    const uint32_t qo = (uint32_t)n * (K / 4) + (uint32_t)sub * 16;
    const uint32_t so = (uint32_t)n * (K / 64) + (uint32_t)(sub >> 1) * 2;
#pragma unroll
    for (int j = 0; j < CPL; ++j)
#pragma unroll
      for (int m = 0; m < G::NM; ++m) {
        b.q[rr][m][j] = *reinterpret_cast<const uint4*>((m == 0 ? qb0 : qb1) + qo + j * 256);
        b.s[rr][m][j] = *reinterpret_cast<const uint16_t*>((m == 0 ? sb0 : sb1) + so + j * 16);
      }
  }
}

template <int CPL, int MT, bool FC1>
__global__ __launch_bounds__(FC_THREADS, 2) void fc_stream_kernel(FcArgs a) {
  using G = TileGeom<CPL, MT, FC1>;
  constexpr int NM = G::NM, RPL = G::RPL, ROWS = G::ROWS;
  constexpr int K = 1024 * CPL;
  constexpr int KS = CPL;  // activation slices
  constexpr int XT = (K / 64) * XCHUNK_UNITS;  // padded 16-byte units per token
  __shared__ uint2 tab[256 * TAB_COPIES];
  __shared__ uint4 xs[MT * XT];
  __shared__ float xsc[MT * KS];
  __shared__ float red[4][MT * KS];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rg = lane >> 4, sub = lane & 15;
  const uint32_t laneoff = (uint32_t)(lane & 31) << 3;
  const int NROWS = FC1 ? a.I : a.H;
  const int RB = (NROWS + ROWS - 1) / ROWS;

  const uint2 cbv = reinterpret_cast<const uint2*>(a.codebook)[tid & 127];
  // The kernel arguments span five scalar-cache lines; the activation pointers' line and
  // the grid size (a hidden argument) are read here, with the header, rather than first
  // where they are used, behind a miss.
  asm volatile("" ::"s"(FC1 ? a.x_h : (const uint16_t*)a.h_in), "s"(gridDim.x));
  if (!ws_ok(a, FC1, MT)) return;
  const int n_tiles = (int)a.hdr[FC1 ? HDR_GROUPS1 : HDR_GROUPS2] * RB;
  // a contiguous run of tiles per workgroup: consecutive tiles share the token group
  const int t_begin = (int)(((long)blockIdx.x * n_tiles) / gridDim.x);
  const int t_end = (int)(((long)(blockIdx.x + 1) * n_tiles) / gridDim.x);
  if (t_begin >= t_end) return;

  // Stage the activations of record r into LDS (FC1: fp16 x of its tokens; FC2: h of
  // its pairs scaled to fp16 with one power-of-two factor per 1024-column slice), in two
  // halves: the loads, then (after the caller has issued the tile's code loads, so that
  // waiting for the activations does not wait for the codes too) the LDS stores.
  // 16-byte units of one token per thread (K / 8 units over FC_THREADS threads)
  constexpr int XU = FC1 ? (K / 8 + FC_THREADS - 1) / FC_THREADS : 1;
  struct StageRegs {
    uint4 xv[FC1 ? MT : 1][XU];
    float scv[FC1 ? MT : 1];
    float4 hv[FC1 ? 1 : MT * KS];
  };
  auto stage_load = [&](const RecS& r) __attribute__((always_inline)) -> StageRegs {
    StageRegs g;
    // staging runs once per token group: its per-lane addresses are recomputed here
    // rather than hoisted out of the tile loop and held in registers across it
    const int tid = opaque(threadIdx.x);
    if (FC1) {
      // the token loop is unrolled so that every pair index is read with a constant
      // index (a per-lane index would put the record in scratch memory)
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        const bool live = j < r.mcount;
        const size_t tok = live ? (size_t)(r.pair[j] / a.k) : 0;
        const uint4* src = reinterpret_cast<const uint4*>(a.x_h + tok * K);
#pragma unroll
        for (int i = 0; i < XU; ++i) {
          const int o = tid + i * FC_THREADS;
          g.xv[j][i] = (live && o < K / 8) ? src[o] : make_uint4(0, 0, 0, 0);
        }
        g.scv[j] = (live && tid < KS) ? a.x_sc[tok * KS + tid] : 1.f;
      }
    } else {
#pragma unroll
      for (int j = 0; j < MT; ++j)
#pragma unroll
        for (int s = 0; s < KS; ++s)
          g.hv[j * KS + s] = j < r.mcount ? reinterpret_cast<const float4*>(a.h_in + (size_t)r.pair[j] * K)[s * 256 + tid]
                                          : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    return g;
  };
  auto stage_store = [&](const StageRegs& g) __attribute__((always_inline)) {
    const int tid = opaque(threadIdx.x);
    const int wave = tid >> 6, lane = tid & 63;
    if (FC1) {
#pragma unroll
      for (int j = 0; j < MT; ++j) {
#pragma unroll
        for (int i = 0; i < XU; ++i) {
          const int o = tid + i * FC_THREADS;
          if (o < K / 8) xs[j * XT + x_unit(o)] = g.xv[j][i];
        }
        if (tid < KS) xsc[j * KS + tid] = g.scv[j];
      }
    } else {
#pragma unroll
      for (int js = 0; js < MT * KS; ++js) {
        const float4 v = g.hv[js];
        float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
        m = wave_max(m);
        if (lane == 0) red[wave][js] = m;
      }
      __syncthreads();
#pragma unroll
      for (int js = 0; js < MT * KS; ++js) {
        const float m = fmaxf(fmaxf(red[0][js], red[1][js]), fmaxf(red[2][js], red[3][js]));
        int ex = 0;
        if (m > 0.f && m == m) ex = frexp_exponent(m) - 15;
        const float4 v = g.hv[js];
        const int j = js / KS, s = js % KS;
        const uint2 pk = make_uint2(pack_half2(ldexp2(v.x, -ex), ldexp2(v.y, -ex)),
                                    pack_half2(ldexp2(v.z, -ex), ldexp2(v.w, -ex)));
        const int u = (s * SLICE + 4 * tid) / 8;  // 16-byte unit within the token
        reinterpret_cast<uint2*>(xs)[(j * XT + x_unit(u)) * 2 + (tid & 1)] = pk;
        if (tid == 0) xsc[js] = ldexp2(1.0f, ex);
      }
    }
  };

  // One tile's outputs from its accumulators (16 lanes of a row reduced first).
  auto finish = [&](float (&acc)[NM][RPL][MT], const RecS& r, int rb) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[m][rr][t] = group_sum<16>(acc[m][rr][t]);
#pragma unroll
    for (int rr = 0; rr < RPL; ++rr) {
      const int n = rb * ROWS + rr * 16 + wave * 4 + rg;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        if (((rr * MT + t) & 15) == sub && t < r.mcount && n < NROWS) {
          const int p = r.pair[t];
          if (FC1) {
            const float gv = acc[0][rr][t], uv = acc[NM - 1][rr][t];
            a.out[(size_t)p * a.I + n] = swiglu(gv, uv, a.lim);
          } else {
            a.out[(size_t)p * a.H + n] = a.pair_w[p] * acc[0][rr][t];
          }
        }
      }
    }
  };

  // VQ2 tile from a filled buffer.  With PF, the next tile's loads (record rn2, row
  // block rbn, into nb) are issued one (row, chunk) at a time, each after the same
  // (row, chunk) of this tile has been decoded: issuing a whole tile at once holds the
  // wave until the memory pipeline has taken every load, which at one or two tiles per
  // workgroup left the decode waiting until nearly all the data had arrived.  The two
  // forms are separate code so that each keeps exact load counts in its waits.
  auto compute_vq = [&](const VqBuf<CPL, MT, FC1>& b, const RecS& r, int rb, auto pf, VqBuf<CPL, MT, FC1>& nb,
                        const RecS& rn2, int rbn) __attribute__((always_inline)) {
    constexpr bool PF = decltype(pf)::value;
    // one base register plus immediate offsets for the factor reads (constant
    // addresses would each be held in a register across the tile loop)
    const float* xscb = xsc + opaque(0);
    float acc[NM][RPL][MT];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[m][rr][t] = 0.f;
#pragma unroll
    for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = sub + 16 * j;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          if (t < r.mcount) {
            // the chunk's 64 activations are read 16 at a time, each shared by the
            // NM matrices, which keeps 8 registers (not 32) of activations live
            const uint4* xp = xs + t * XT + c * XCHUNK_UNITS;
            float pr[NM];
#pragma unroll
            for (int m = 0; m < NM; ++m) pr[m] = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint4 xr[2] = {xp[2 * i], xp[2 * i + 1]};
              const uint32_t* xw = reinterpret_cast<const uint32_t*>(xr);
#pragma unroll
              for (int m = 0; m < NM; ++m) pr[m] = vq2_dword_dot(tab, dword_of(b.q[rr][m][j], i), laneoff, xw, pr[m]);
            }
            const float f = xscb[t * KS + j];
#pragma unroll
            for (int m = 0; m < NM; ++m)
              acc[m][rr][t] = fmaf(f16_bits_to_f32(b.s[rr][m][j]) * f, pr[m], acc[m][rr][t]);
          }
        }
        if constexpr (PF) issue_vq_chunk(nb, a, rn2, rbn, NROWS, wave, rg, sub, rr, j);
      }
    finish(acc, r, rb);
  };

  // MXFP4 tile (loads and compute, not pipelined), or an absent expert (zeros).  The
  // tile's (row, matrix) units of MXC 16-byte loads are processed UPP at a time.
  auto compute_mx = [&](const RecS& r, int rb) __attribute__((always_inline)) {
    const float* xscb = xsc + opaque(0);
    constexpr int MXC = G::MXC;
    constexpr int NU = RPL * NM;                                   // units per tile
    constexpr int UPP_RAW = LB_MX / MXC;
    constexpr int UPP = UPP_RAW < 1 ? 1 : (UPP_RAW > NU ? NU : UPP_RAW);
    float acc[NM][RPL][MT];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[m][rr][t] = 0.f;
    if (r.fmt == MOE_VQ_FMT_MXFP4) {
      const uint8_t* slot = a.pool + r.slot_off;
      const uint8_t* qb0 = slot + (FC1 ? a.mx4.q_gate : a.mx4.q_down);
      const uint8_t* qb1 = slot + a.mx4.q_up;
      const uint8_t* sb0 = slot + (FC1 ? a.mx4.s_gate : a.mx4.s_down);
      const uint8_t* sb1 = slot + a.mx4.s_up;
#pragma unroll
      for (int u0 = 0; u0 < NU; u0 += UPP) {
        uint4 qm[UPP][MXC];
        uint32_t em[UPP][MXC];
#pragma unroll
        for (int uu = 0; uu < UPP; ++uu) {
          const int u = u0 + uu, rr = u / NM, m = u % NM;
          const int n = min(rb * ROWS + rr * 16 + wave * 4 + rg, NROWS - 1);
          const uint32_t qo = (uint32_t)n * (K / 2) + (uint32_t)sub * 16;
          const uint32_t eo = (uint32_t)n * (K / 32) + (uint32_t)sub;
#pragma unroll
          for (int j = 0; j < MXC; ++j) {
            if (u < NU) {
              qm[uu][j] = *reinterpret_cast<const uint4*>((m == 0 ? qb0 : qb1) + qo + j * 256);
              em[uu][j] = ((m == 0 ? sb0 : sb1) + eo)[j * 16];
            } else {
              qm[uu][j] = make_uint4(0, 0, 0, 0);
              em[uu][j] = 127;
            }
          }
        }
#pragma unroll
        for (int uu = 0; uu < UPP; ++uu) {
          const int u = u0 + uu, rr = u / NM, m = u % NM;
          if (u >= NU) break;
#pragma unroll
          for (int j = 0; j < MXC; ++j) {
            const int c = sub + 16 * j;
#pragma unroll
            for (int t = 0; t < MT; ++t) {
              if (t < r.mcount) {
                const uint4* xp = xs + t * XT + (c >> 1) * XCHUNK_UNITS + (c & 1) * 4;
                uint4 xr[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) xr[i] = xp[i];
                const uint32_t* xw = reinterpret_cast<const uint32_t*>(xr);
                const float f = xscb[t * KS + (c >> 5)];
                const float pr = mx4_chunk_dot(qm[uu][j], xw);
                acc[m][rr][t] = fmaf(e8m0_to_f32(em[uu][j]) * f, pr, acc[m][rr][t]);
              }
            }
          }
        }
      }
    }
    // (an absent expert keeps acc at zero: its outputs are written as 0 and the
    //  worklist has recorded MOE_VQ_ENOTRESIDENT in the status word)
    finish(acc, r, rb);
  };

  // ---- prologue: first tile's record, its code loads, activations and the table
  int t = t_begin;
  const RecRaw raw_c = load_rec_raw(a.rec, t / RB);
  const RecRaw raw_n = load_rec_raw(a.rec, (t + 1 < t_end ? t + 1 : t) / RB);
  RecS rc = rec_from_raw(raw_c);
  RecS rn = rec_from_raw(raw_n);
  VqBuf<CPL, MT, FC1> A, B;
  {
    const StageRegs g = stage_load(rc);
    if (rc.fmt == MOE_VQ_FMT_VQ2) issue_vq(A, a, rc, t % RB, NROWS, wave, rg, sub);
    write_table_entry(tab, cbv, tid);
    stage_store(g);
  }
  __syncthreads();

  // ---- steady state: the next tile's loads are in flight while this tile decodes.
  // `pending` says whether the other buffer already holds the next tile's loads.
  auto step = [&](VqBuf<CPL, MT, FC1>& cur, VqBuf<CPL, MT, FC1>& nxt) __attribute__((always_inline)) -> bool {
    const int tn = t + 1;
    const bool more = tn < t_end;
    const bool same = more && same_inputs<MT, FC1>(rn, rc, a.k);
    // prefetch only between VQ2 tiles of the same token group (an MXFP4 tile uses the
    // register budget of both buffers itself)
    const bool prefetch = more && same && rn.fmt == MOE_VQ_FMT_VQ2 && rc.fmt == MOE_VQ_FMT_VQ2;
    const RecS rnn = (tn + 1 < t_end) ? load_rec(a.rec, (tn + 1) / RB) : rn;
    if (prefetch) compute_vq(cur, rc, t % RB, std::true_type{}, nxt, rn, tn % RB);
    else if (rc.fmt == MOE_VQ_FMT_VQ2) compute_vq(cur, rc, t % RB, std::false_type{}, nxt, rn, tn % RB);
    else compute_mx(rc, t % RB);
    if (!more) return false;
    if (!same) {
      const StageRegs g = stage_load(rn);
      if (rn.fmt == MOE_VQ_FMT_VQ2) issue_vq(nxt, a, rn, tn % RB, NROWS, wave, rg, sub);
      __syncthreads();  // every wave is done with the staged activations
      stage_store(g);
      __syncthreads();
    } else if (!prefetch && rn.fmt == MOE_VQ_FMT_VQ2) {
      issue_vq(nxt, a, rn, tn % RB, NROWS, wave, rg, sub);
    }
    rc = rn;
    rn = rnn;
    t = tn;
    return true;
  };
  for (;;) {
    if (!step(A, B)) break;
    if (!step(B, A)) break;
  }
}

// -------------------------------------------------------------------------------------
// fc_generic_kernel: any K multiple of 128, persistent grid
// -------------------------------------------------------------------------------------

constexpr int RPL_GEN = 2;

int gen_lanes_per_row(int K) {
  const int nchunk = K / 64;
  if (nchunk % 16 == 0) return 16;
  if (nchunk % 8 == 0) return 8;
  if (nchunk % 4 == 0) return 4;
  return 2;
}

template <int LPR, int MT, bool FC1>
__global__ __launch_bounds__(FC_THREADS) void fc_generic_kernel(FcArgs a) {
  __shared__ uint2 tab[256 * TAB_COPIES];
  extern __shared__ uint4 dyn[];
  constexpr int NM = FC1 ? 2 : 1;
  constexpr int RPL = RPL_GEN;
  constexpr int RG = 64 / LPR;
  constexpr int ROWS = (FC_THREADS / 64) * RG * RPL;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rg = lane / LPR, sub = lane % LPR;
  const uint32_t laneoff = (uint32_t)(lane & 31) << 3;
  const int K = FC1 ? a.H : a.I;
  const int NROWS = FC1 ? a.I : a.H;
  const int KS = n_slices(K);
  const int XT = (int)fc_x_units(K);
  uint4* xs = dyn;
  float* xsc = reinterpret_cast<float*>(dyn + (size_t)MT * XT);

  const uint2 cbv = reinterpret_cast<const uint2*>(a.codebook)[tid & 127];
  if (!ws_ok(a, FC1, MT)) return;
  const int n_groups = (int)a.hdr[FC1 ? HDR_GROUPS1 : HDR_GROUPS2];
  const int RB = (NROWS + ROWS - 1) / ROWS;
  const int n_tiles = n_groups * RB;
  write_table_entry(tab, cbv, tid);

  int cur_g = -1;
  for (int tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int g = tile / RB, rb = tile % RB;
    const GroupRec rec = a.rec[g];
    const int p0 = rec.p0, mcount = rec.mcount;
    const uint32_t fmt = rec.fmt;
    const uint8_t* slot = a.pool + rec.slot_off;

    if (g != cur_g) {
      __syncthreads();
      if (FC1) {
        for (int j = 0; j < mcount; ++j) {
          const int t = a.pair_list[p0 + j] / a.k;
          const uint4* src = reinterpret_cast<const uint4*>(a.x_h + (size_t)t * K);
          for (int i = tid; i < K / 8; i += FC_THREADS) xs[j * XT + x_unit(i)] = src[i];
          for (int i = tid; i < KS; i += FC_THREADS) xsc[j * KS + i] = a.x_sc[(size_t)t * KS + i];
        }
      } else {
        for (int js = wave; js < mcount * KS; js += FC_THREADS / 64) {
          const int j = js / KS, s = js % KS;
          const int p = a.pair_list[p0 + j];
          const int c0 = s * SLICE + lane * 16;
          float v[16];
          float m = 0.f;
          if (c0 < K) {
            const float4* src = reinterpret_cast<const float4*>(a.h_in + (size_t)p * K + c0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float4 f = src[q];
              v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
            }
#pragma unroll
            for (int q = 0; q < 16; ++q) m = fmaxf(m, fabsf(v[q]));
          }
          m = wave_max(m);
          int ex = 0;
          if (m > 0.f && m == m) ex = frexp_exponent(m) - 15;
          if (c0 < K) {
            uint32_t pk[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) pk[q] = pack_half2(ldexp2(v[2 * q], -ex), ldexp2(v[2 * q + 1], -ex));
            xs[j * XT + x_unit(c0 / 8)] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
            xs[j * XT + x_unit(c0 / 8 + 1)] = make_uint4(pk[4], pk[5], pk[6], pk[7]);
          }
          if (lane == 0) xsc[j * KS + s] = ldexp2(1.0f, ex);
        }
      }
      __syncthreads();
      cur_g = g;
    }

    const int nbase = rb * ROWS + (wave * RG + rg) * RPL;
    int nrow[RPL];
    bool rok[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r) { nrow[r] = nbase + r; rok[r] = nrow[r] < NROWS; }
    float acc[NM][RPL][MT];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int r = 0; r < RPL; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[m][r][t] = 0.f;

    if (fmt == MOE_VQ_FMT_VQ2) {
      const uint8_t* qb[2] = {slot + (FC1 ? a.vq2.q_gate : a.vq2.q_down), slot + a.vq2.q_up};
      const uint16_t* sb[2] = {reinterpret_cast<const uint16_t*>(slot + (FC1 ? a.vq2.s_gate : a.vq2.s_down)),
                               reinterpret_cast<const uint16_t*>(slot + a.vq2.s_up)};
      const int cpl = (K / 64) / LPR;
      for (int j = 0; j < cpl; ++j) {
        const int c = sub + LPR * j;
        uint4 q[NM][RPL];
        uint32_t sc[NM][RPL];
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int r = 0; r < RPL; ++r) {
            q[m][r] = rok[r] ? ldg16(qb[m] + (size_t)nrow[r] * (K / 4) + c * 16) : make_uint4(0, 0, 0, 0);
            sc[m][r] = rok[r] ? sb[m][(size_t)nrow[r] * (K / 128) + (c >> 1)] : 0u;
          }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          if (t < mcount) {
            const uint4* xp = xs + t * XT + c * XCHUNK_UNITS;
            uint4 xr[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) xr[i] = xp[i];
            const uint32_t* xw = reinterpret_cast<const uint32_t*>(xr);
            const float f = xsc[t * KS + (c >> 4)];
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
              for (int r = 0; r < RPL; ++r)
                acc[m][r][t] = fmaf(f16_bits_to_f32(sc[m][r]) * f, vq2_chunk_dot(tab, q[m][r], laneoff, xw), acc[m][r][t]);
          }
        }
      }
    } else if (fmt == MOE_VQ_FMT_MXFP4) {
      const uint8_t* qb[2] = {slot + (FC1 ? a.mx4.q_gate : a.mx4.q_down), slot + a.mx4.q_up};
      const uint8_t* sb[2] = {slot + (FC1 ? a.mx4.s_gate : a.mx4.s_down), slot + a.mx4.s_up};
      const int cpl = (K / 32) / LPR;
      for (int j = 0; j < cpl; ++j) {
        const int c = sub + LPR * j;
        uint4 q[NM][RPL];
        uint32_t se[NM][RPL];
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int r = 0; r < RPL; ++r) {
            q[m][r] = rok[r] ? ldg16(qb[m] + (size_t)nrow[r] * (K / 2) + c * 16) : make_uint4(0, 0, 0, 0);
            se[m][r] = rok[r] ? sb[m][(size_t)nrow[r] * (K / 32) + c] : 127u;
          }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          if (t < mcount) {
            const uint4* xp = xs + t * XT + (c >> 1) * XCHUNK_UNITS + (c & 1) * 4;
            uint4 xr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) xr[i] = xp[i];
            const uint32_t* xw = reinterpret_cast<const uint32_t*>(xr);
            const float f = xsc[t * KS + (c >> 5)];
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
              for (int r = 0; r < RPL; ++r)
                acc[m][r][t] = fmaf(e8m0_to_f32(se[m][r]) * f, mx4_chunk_dot(q[m][r], xw), acc[m][r][t]);
          }
        }
      }
    }

#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int r = 0; r < RPL; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[m][r][t] = group_sum<LPR>(acc[m][r][t]);
#pragma unroll
    for (int r = 0; r < RPL; ++r)
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        if (((r + RPL * t) % LPR) == sub && t < mcount && rok[r]) {
          const int p = a.pair_list[p0 + t];
          if (FC1) {
            const float gv = acc[0][r][t], uv = acc[NM - 1][r][t];
            a.out[(size_t)p * a.I + nrow[r]] = swiglu(gv, uv, a.lim);
          } else {
            a.out[(size_t)p * a.H + nrow[r]] = a.pair_w[p] * acc[0][r][t];
          }
        }
      }
  }
}

// y[t][n] = sum_{i<k} o_buf[t*k + i][n] in pair order (deterministic), added to y's value
// when accumulate is set (the shared expert).  Pairs whose expert was not resident hold
// zeros (their FC2 tiles still write them).
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o_buf, float* __restrict__ y,
                                                      int T, int H, int k, int accumulate) {
  const size_t n4 = (size_t)T * H / 4;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    const size_t t = (i * 4) / H, n = (i * 4) % H;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (accumulate) acc = *reinterpret_cast<const float4*>(y + t * H + n);
    for (int j = 0; j < k; ++j) {
      const float4 v = *reinterpret_cast<const float4*>(o_buf + (t * k + j) * H + n);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    *reinterpret_cast<float4*>(y + t * H + n) = acc;
  }
}

// -------------------------------------------------------------------------------------
// Host launchers
// -------------------------------------------------------------------------------------

template <bool FC1>
static hipError_t launch_stream(const FcArgs& a, int K, int MT, int max_groups, int n_cu, hipStream_t st,
                                bool* done) {
  *done = false;
  if (K % 1024 != 0) return hipSuccess;
  const int cpl = K / 1024;
  const int nrows = FC1 ? a.I : a.H;
  const size_t lds = fc_lds_bytes(MT, K);
  int per_cu = (int)(LDS_LIMIT / lds);
  per_cu = per_cu < 1 ? 1 : (per_cu > 2 ? 2 : per_cu);
  // FC2 at K = 7168 with one token per group needs more registers than a wave of
  // this kernel has (it would spill to scratch memory, whose set-up costs more per
  // launch than the kernel's own run): the generic kernel takes that shape.
#define MVQ_STREAM_CASE(C, M)                                                                \
  if constexpr (FC1 || C != 7 || M != 1)                                                     \
  if (cpl == C && MT == M) {                                                                 \
    constexpr int ROWS = TileGeom<C, M, FC1>::ROWS;                                           \
    const long tiles = (long)max_groups * ((nrows + ROWS - 1) / ROWS);                      \
    long grid = (long)n_cu * per_cu;                                                         \
    if (tiles < grid) grid = tiles;                                                          \
    *done = true;                                                                            \
    if (grid <= 0) return hipSuccess;                                                        \
    launch_fc_kernel(fc_stream_kernel<C, M, FC1>, (unsigned)grid, FC_THREADS, 0, st, a);      \
    return hipGetLastError();                                                                \
  }
  MVQ_STREAM_CASE(1, 1) MVQ_STREAM_CASE(2, 1) MVQ_STREAM_CASE(7, 1)
  MVQ_STREAM_CASE(1, 4) MVQ_STREAM_CASE(2, 4) MVQ_STREAM_CASE(7, 4)
#undef MVQ_STREAM_CASE
  return hipSuccess;
}

template <bool FC1>
static hipError_t launch_generic(const FcArgs& a, int K, int MT, int max_groups, int n_cu, hipStream_t st) {
  const int lpr = gen_lanes_per_row(K);
  const int nrows = FC1 ? a.I : a.H;
  const int rows = (FC_THREADS / 64) * (64 / lpr) * RPL_GEN;
  const long tiles = (long)max_groups * ((nrows + rows - 1) / rows);
  const size_t lds = fc_lds_bytes(MT, K);
  int per_cu = (int)(LDS_LIMIT / lds);
  per_cu = per_cu < 1 ? 1 : (per_cu > 4 ? 4 : per_cu);
  long grid = (long)n_cu * per_cu;
  if (tiles < grid) grid = tiles;
  if (grid < 1) grid = 1;
  const size_t dyn = (size_t)MT * fc_x_units(K) * 16 + (size_t)MT * n_slices(K) * 4;
  // The dynamic-LDS limit is raised once per kernel instance to the largest size any
  // call can ask for (idempotent, so a racing second call is harmless).
#define MVQ_GEN_CASE(L, M)                                                                   \
  if (lpr == L && MT == M) {                                                                 \
    auto kern = fc_generic_kernel<L, M, FC1>;                                                \
    static bool attr_set = false;                                                            \
    if (!attr_set) {                                                                         \
      hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, \
                                         LDS_LIMIT - TAB_BYTES - 256);                      \
      if (e != hipSuccess) return e;                                                         \
      attr_set = true;                                                                       \
    }                                                                                        \
    launch_fc_kernel(kern, (unsigned)grid, FC_THREADS, (uint32_t)dyn, st, a);                \
    return hipGetLastError();                                                                \
  }
  MVQ_GEN_CASE(16, 1) MVQ_GEN_CASE(16, 2) MVQ_GEN_CASE(16, 4)
  MVQ_GEN_CASE(8, 1) MVQ_GEN_CASE(8, 2) MVQ_GEN_CASE(8, 4)
  MVQ_GEN_CASE(4, 1) MVQ_GEN_CASE(4, 2) MVQ_GEN_CASE(4, 4)
  MVQ_GEN_CASE(2, 1) MVQ_GEN_CASE(2, 2) MVQ_GEN_CASE(2, 4)
#undef MVQ_GEN_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_fc1(const FcArgs& a, int MT, int max_groups, int n_cu, hipStream_t st) {
  (void)hipGetLastError();  // start from a clean error state: report only our own launches
  bool done = false;
  hipError_t e = launch_mfma<true>(a, a.H, MT, max_groups, n_cu, st, &done);
  if (e != hipSuccess || done) return e;
  e = launch_stream<true>(a, a.H, MT, max_groups, n_cu, st, &done);
  if (e != hipSuccess || done) return e;
  return launch_generic<true>(a, a.H, MT, max_groups, n_cu, st);
}

hipError_t launch_fc2(const FcArgs& a, int MT, int max_groups, int n_cu, hipStream_t st) {
  (void)hipGetLastError();  // start from a clean error state: report only our own launches
  bool done = false;
  hipError_t e = launch_fc2_single(a, MT, st, &done);  // one token: writes y itself
  if (e != hipSuccess || done) return e;
  e = launch_mfma<false>(a, a.I, MT, max_groups, n_cu, st, &done);
  if (e == hipSuccess && !done) e = launch_stream<false>(a, a.I, MT, max_groups, n_cu, st, &done);
  if (e == hipSuccess && !done) e = launch_generic<false>(a, a.I, MT, max_groups, n_cu, st);
  if (e != hipSuccess) return e;
  const size_t n4 = (size_t)a.T * a.H / 4;
  const int blocks = (int)((n4 + 255) / 256 < 4096 ? (n4 + 255) / 256 : 4096);
  launch_combine(a.out, a.y, a.T, a.H, a.k, a.accumulate, blocks, st);
  return hipGetLastError();
}

void launch_combine(const float* o_buf, float* y, int T, int H, int k, int accumulate, int blocks, hipStream_t st) {
  combine_kernel<<<blocks, 256, 0, st>>>(o_buf, y, T, H, k, accumulate);
}

}  // namespace mvq
