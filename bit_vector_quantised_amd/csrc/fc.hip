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
//  * fc_tile_kernel (K a multiple of 1024, K <= 8192): one workgroup per tile.  The
//    workgroup first issues the codebook load, its staging loads and ALL code/scale
//    loads of its rows, then builds the LDS table while the code stream is in flight
//    and consumes the loads in issue order (vmcnt is in order), so every wave keeps
//    ~14 x 16 B per lane in flight from its first cycle.
//  * fc_generic_kernel (any K multiple of 128): a persistent grid that prefetches one
//    chunk ahead; used for the shapes the tile kernel does not cover.
#include "moe_vq_device.h"
#include "moe_vq_launch.h"

namespace mvq {

constexpr int LB_VQ = 14;   // 16-byte code loads in flight per lane (VQ2 tiles)
constexpr int LB_MX = 14;   // same budget for MXFP4 tiles (twice the bytes per weight)

// -------------------------------------------------------------------------------------
// Shared pieces
// -------------------------------------------------------------------------------------

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

__device__ __forceinline__ bool ws_ok(const FcArgs& a, bool fc1, int MT) {
  return a.hdr[HDR_KEY] == a.key && a.hdr[HDR_N_ACTIVE] <= (uint32_t)a.E &&
         a.hdr[fc1 ? HDR_GROUPS1 : HDR_GROUPS2] <= (uint32_t)a.max_groups &&
         a.hdr[fc1 ? HDR_MT1 : HDR_MT2] == (uint32_t)MT;
}

// 16 VQ2 words of one 16-byte chunk against 64 fp16 activations (32 dwords).
__device__ __forceinline__ float vq2_chunk_dot(const uint2* tab, const uint4& q, uint32_t laneoff,
                                               const uint32_t* xw) {
  float p = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t wd = i == 0 ? q.x : i == 1 ? q.y : i == 2 ? q.z : q.w;
    uint2 e0 = tab_lookup(tab, tab_addr<0>(wd, laneoff));
    uint2 e1 = tab_lookup(tab, tab_addr<1>(wd, laneoff));
    uint2 e2 = tab_lookup(tab, tab_addr<2>(wd, laneoff));
    uint2 e3 = tab_lookup(tab, tab_addr<3>(wd, laneoff));
    p = dot2(e0.x, xw[8 * i + 0], p); p = dot2(e0.y, xw[8 * i + 1], p);
    p = dot2(e1.x, xw[8 * i + 2], p); p = dot2(e1.y, xw[8 * i + 3], p);
    p = dot2(e2.x, xw[8 * i + 4], p); p = dot2(e2.y, xw[8 * i + 5], p);
    p = dot2(e3.x, xw[8 * i + 6], p); p = dot2(e3.y, xw[8 * i + 7], p);
  }
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

// -------------------------------------------------------------------------------------
// fc_tile_kernel: K = 1024 * CPL, LPR = 16, one workgroup per (group, row block)
// -------------------------------------------------------------------------------------

template <int CPL, bool FC1>
struct TileGeom {
  static constexpr int NM = FC1 ? 2 : 1;
  static constexpr int RPL_RAW = FC1 ? LB_VQ / (2 * CPL) : LB_VQ / CPL;
  static constexpr int RPL = RPL_RAW < 1 ? 1 : RPL_RAW;           // rows per lane
  static constexpr int ROWS = 16 * RPL;                              // rows per tile
  static constexpr int MXC = 2 * CPL;                                // MXFP4 chunks per lane per row
  static constexpr int RPP_MX_RAW = LB_MX / (NM * MXC);
  static constexpr int RPP_MX = RPP_MX_RAW < 1 ? 1 : (RPP_MX_RAW > RPL ? RPL : RPP_MX_RAW);
};

template <int CPL, int MT, bool FC1>
__global__ __launch_bounds__(FC_THREADS, 2) void fc_tile_kernel(FcArgs a) {
  using G = TileGeom<CPL, FC1>;
  constexpr int NM = G::NM, RPL = G::RPL, ROWS = G::ROWS;
  constexpr int K = 1024 * CPL;
  constexpr int KS = CPL;  // activation slices
  __shared__ uint2 tab[256 * TAB_COPIES];
  __shared__ uint4 xs[MT * K / 8];
  __shared__ float xsc[MT * KS];
  __shared__ float red[4][MT * KS];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rg = lane >> 4, sub = lane & 15;
  const uint32_t laneoff = (uint32_t)(lane & 31) << 3;
  const int NROWS = FC1 ? a.I : a.H;
  const int RB = (NROWS + ROWS - 1) / ROWS;
  const int g = blockIdx.x / RB, rb = blockIdx.x % RB;

  // (1) loads that do not depend on the worklist contents
  const uint2 cbv = reinterpret_cast<const uint2*>(a.codebook)[tid & 127];
  if (!ws_ok(a, FC1, MT)) return;
  const int n_groups = (int)a.hdr[FC1 ? HDR_GROUPS1 : HDR_GROUPS2];
  if (g >= n_groups) return;
  const GroupRec rec = a.rec[g];
  const int mcount = rec.mcount;
  const uint32_t fmt = rec.fmt;
  const uint8_t* slot = a.pool + rec.slot_off;

  // (2) staging loads: FC1 reads the fp16 activations of the group's tokens, FC2 the
  // fp32 h of its pairs (thread tid covers columns 4*tid..4*tid+3 of every slice)
  int pair[MT];
#pragma unroll
  for (int j = 0; j < MT; ++j) pair[j] = a.pair_list[rec.p0 + (j < mcount ? j : 0)];
  constexpr int XV = FC1 ? (MT * K / 8 + FC_THREADS - 1) / FC_THREADS : 1;
  uint4 xv[XV];
  float4 hv[FC1 ? 1 : MT * KS];
  float scv = 1.f;
  if (FC1) {
#pragma unroll
    for (int i = 0; i < XV; ++i) {
      const int idx = tid + i * FC_THREADS;
      const int j = idx / (K / 8), o = idx % (K / 8);
      if (idx < MT * K / 8 && j < mcount)
        xv[i] = reinterpret_cast<const uint4*>(a.x_h + (size_t)(pair[j] / a.k) * K)[o];
      else
        xv[i] = make_uint4(0, 0, 0, 0);
    }
    if (tid < MT * KS) {
      const int j = tid / KS, s = tid % KS;
      scv = j < mcount ? a.x_sc[(size_t)(pair[j] / a.k) * KS + s] : 1.f;
    }
  } else {
#pragma unroll
    for (int j = 0; j < MT; ++j)
#pragma unroll
      for (int s = 0; s < KS; ++s)
        hv[j * KS + s] = j < mcount ? reinterpret_cast<const float4*>(a.h_in + (size_t)pair[j] * K)[s * 256 + tid]
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
  }

  // (3) row coordinates and the code/scale loads of the first pass
  int nrow[RPL];
  bool rok[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    nrow[r] = rb * ROWS + r * 16 + wave * 4 + rg;
    rok[r] = nrow[r] < NROWS;
  }
  float acc[NM][RPL][MT];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int r = 0; r < RPL; ++r)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[m][r][t] = 0.f;

  const bool is_vq = fmt == MOE_VQ_FMT_VQ2;
  const bool is_mx = fmt == MOE_VQ_FMT_MXFP4;
  uint4 q[RPL][NM][CPL];
  uint32_t sq[RPL][NM][CPL];
  if (is_vq) {
    const uint8_t* qb0 = slot + (FC1 ? a.vq2.q_gate : a.vq2.q_down);
    const uint8_t* qb1 = slot + a.vq2.q_up;
    const uint16_t* sb0 = reinterpret_cast<const uint16_t*>(slot + (FC1 ? a.vq2.s_gate : a.vq2.s_down));
    const uint16_t* sb1 = reinterpret_cast<const uint16_t*>(slot + a.vq2.s_up);
#pragma unroll
    for (int r = 0; r < RPL; ++r)
#pragma unroll
      for (int j = 0; j < CPL; ++j)
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          const int c = sub + 16 * j;
          if (rok[r]) {
            q[r][m][j] = ldg16((m == 0 ? qb0 : qb1) + (size_t)nrow[r] * (K / 4) + c * 16);
            sq[r][m][j] = (m == 0 ? sb0 : sb1)[(size_t)nrow[r] * (K / 128) + (c >> 1)];
          } else {
            q[r][m][j] = make_uint4(0, 0, 0, 0);
            sq[r][m][j] = 0;
          }
        }
  }

  // (4) LDS: decode table and staged activations
  write_table_entry(tab, cbv, tid);
  if (FC1) {
#pragma unroll
    for (int i = 0; i < XV; ++i) {
      const int idx = tid + i * FC_THREADS;
      if (idx < MT * K / 8) xs[idx] = xv[i];
    }
    if (tid < MT * KS) xsc[tid] = scv;
  } else {
    // one power-of-two factor per (pair, 1024-column slice): block-wide max first
#pragma unroll
    for (int js = 0; js < MT * KS; ++js) {
      const float4 v = hv[js];
      float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
      m = wave_max(m);
      if (lane == 0) red[wave][js] = m;
    }
    __syncthreads();
#pragma unroll
    for (int js = 0; js < MT * KS; ++js) {
      const float m = fmaxf(fmaxf(red[0][js], red[1][js]), fmaxf(red[2][js], red[3][js]));
      int ex = 0;
      if (m > 0.f && m == m) { int e2; frexpf(m, &e2); ex = e2 - 15; }
      const float4 v = hv[js];
      const int j = js / KS, s = js % KS;
      uint2 pk = make_uint2(pack_half2(ldexpf(v.x, -ex), ldexpf(v.y, -ex)), pack_half2(ldexpf(v.z, -ex), ldexpf(v.w, -ex)));
      reinterpret_cast<uint2*>(xs)[(j * K + s * SLICE) / 4 + tid] = pk;
      if (tid == 0) xsc[js] = ldexpf(1.0f, ex);
    }
  }
  __syncthreads();

  // (5) compute, consuming the loads in issue order
  if (is_vq) {
#pragma unroll
    for (int r = 0; r < RPL; ++r)
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = sub + 16 * j;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          if (t < mcount) {
            const uint4* xp = xs + t * (K / 8) + c * 8;
            uint4 xr[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) xr[i] = xp[i];
            const uint32_t* xw = reinterpret_cast<const uint32_t*>(xr);
            const float f = xsc[t * KS + j];
#pragma unroll
            for (int m = 0; m < NM; ++m) {
              const float p = vq2_chunk_dot(tab, q[r][m][j], laneoff, xw);
              acc[m][r][t] = fmaf(f16_bits_to_f32(sq[r][m][j]) * f, p, acc[m][r][t]);
            }
          }
        }
      }
  } else if (is_mx) {
    constexpr int MXC = G::MXC, RPP = G::RPP_MX;
    const uint8_t* qb0 = slot + (FC1 ? a.mx4.q_gate : a.mx4.q_down);
    const uint8_t* qb1 = slot + a.mx4.q_up;
    const uint8_t* sb0 = slot + (FC1 ? a.mx4.s_gate : a.mx4.s_down);
    const uint8_t* sb1 = slot + a.mx4.s_up;
#pragma unroll
    for (int r0 = 0; r0 < RPL; r0 += RPP) {
      uint4 qm[RPP][NM][MXC];
      uint32_t em[RPP][NM][MXC];
#pragma unroll
      for (int rr = 0; rr < RPP; ++rr)
#pragma unroll
        for (int j = 0; j < MXC; ++j)
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            const int r = r0 + rr;
            const int c = sub + 16 * j;
            if (r < RPL && rok[r < RPL ? r : 0]) {
              const int n = nrow[r < RPL ? r : 0];
              qm[rr][m][j] = ldg16((m == 0 ? qb0 : qb1) + (size_t)n * (K / 2) + c * 16);
              em[rr][m][j] = (m == 0 ? sb0 : sb1)[(size_t)n * (K / 32) + c];
            } else {
              qm[rr][m][j] = make_uint4(0, 0, 0, 0);
              em[rr][m][j] = 127;
            }
          }
#pragma unroll
      for (int rr = 0; rr < RPP; ++rr) {
        if (r0 + rr >= RPL) break;
#pragma unroll
        for (int j = 0; j < MXC; ++j) {
          const int c = sub + 16 * j;
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            if (t < mcount) {
              const uint4* xp = xs + t * (K / 8) + c * 4;
              uint4 xr[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) xr[i] = xp[i];
              const uint32_t* xw = reinterpret_cast<const uint32_t*>(xr);
              const float f = xsc[t * KS + (c >> 5)];
#pragma unroll
              for (int m = 0; m < NM; ++m) {
                const float p = mx4_chunk_dot(qm[rr][m][j], xw);
                acc[m][r0 + rr][t] = fmaf(e8m0_to_f32(em[rr][m][j]) * f, p, acc[m][r0 + rr][t]);
              }
            }
          }
        }
      }
    }
  }
  // (an absent expert leaves acc at zero: h / pair outputs are written as 0 and the
  //  worklist has recorded MOE_VQ_ENOTRESIDENT in the status word)

  // (6) reduce the 16 lanes of each row and write
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int r = 0; r < RPL; ++r)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[m][r][t] = group_sum<16>(acc[m][r][t]);
#pragma unroll
  for (int r = 0; r < RPL; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (((r * MT + t) & 15) == sub && t < mcount && rok[r]) {
        const int p = pair[t];
        if (FC1) {
          const float gv = acc[0][r][t], uv = acc[NM - 1][r][t];
          a.out[(size_t)p * a.I + nrow[r]] = gv / (1.0f + expf(-gv)) * uv;
        } else {
          a.out[(size_t)p * a.H + nrow[r]] = a.pair_w[p] * acc[0][r][t];
        }
      }
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
  uint4* xs = dyn;
  float* xsc = reinterpret_cast<float*>(dyn + (size_t)MT * (K / 8));

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
          for (int i = tid; i < K / 8; i += FC_THREADS) xs[j * (K / 8) + i] = src[i];
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
          if (m > 0.f && m == m) { int e2; frexpf(m, &e2); ex = e2 - 15; }
          if (c0 < K) {
            uint32_t pk[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) pk[q] = pack_half2(ldexpf(v[2 * q], -ex), ldexpf(v[2 * q + 1], -ex));
            uint4* dst = xs + j * (K / 8) + c0 / 8;
            dst[0] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
            dst[1] = make_uint4(pk[4], pk[5], pk[6], pk[7]);
          }
          if (lane == 0) xsc[j * KS + s] = ldexpf(1.0f, ex);
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
            const uint4* xp = xs + t * (K / 8) + c * 8;
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
            const uint4* xp = xs + t * (K / 8) + c * 4;
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
            a.out[(size_t)p * a.I + nrow[r]] = gv / (1.0f + expf(-gv)) * uv;
          } else {
            a.out[(size_t)p * a.H + nrow[r]] = a.pair_w[p] * acc[0][r][t];
          }
        }
      }
  }
}

// y[t][n] = sum_{i<k} o_buf[t*k + i][n] in pair order (deterministic).  Pairs whose
// expert was not resident hold zeros (their FC2 tiles still write them).
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o_buf, float* __restrict__ y,
                                                      int T, int H, int k) {
  const size_t n4 = (size_t)T * H / 4;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    const size_t t = (i * 4) / H, n = (i * 4) % H;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
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
static hipError_t launch_tile(const FcArgs& a, int K, int MT, int max_groups, hipStream_t st, bool* done) {
  *done = false;
  if (K % 1024 != 0) return hipSuccess;
  const int cpl = K / 1024;
  const int nrows = FC1 ? a.I : a.H;
#define MVQ_TILE_CASE(C, M)                                                                  \
  if (cpl == C && MT == M) {                                                                 \
    constexpr int ROWS = TileGeom<C, FC1>::ROWS;                                             \
    const long grid = (long)max_groups * ((nrows + ROWS - 1) / ROWS);                       \
    *done = true;                                                                            \
    if (grid <= 0) return hipSuccess;                                                        \
    fc_tile_kernel<C, M, FC1><<<(unsigned)grid, FC_THREADS, 0, st>>>(a);                     \
    return hipGetLastError();                                                                \
  }
  MVQ_TILE_CASE(1, 1) MVQ_TILE_CASE(2, 1) MVQ_TILE_CASE(4, 1) MVQ_TILE_CASE(7, 1) MVQ_TILE_CASE(8, 1)
  MVQ_TILE_CASE(1, 4) MVQ_TILE_CASE(2, 4) MVQ_TILE_CASE(4, 4) MVQ_TILE_CASE(7, 4)
#undef MVQ_TILE_CASE
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
  const size_t dyn = (size_t)MT * K * 2 + (size_t)MT * n_slices(K) * 4;
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
    kern<<<(unsigned)grid, FC_THREADS, dyn, st>>>(a);                                        \
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
  hipError_t e = launch_tile<true>(a, a.H, MT, max_groups, st, &done);
  if (e != hipSuccess || done) return e;
  return launch_generic<true>(a, a.H, MT, max_groups, n_cu, st);
}

hipError_t launch_fc2(const FcArgs& a, int MT, int max_groups, int n_cu, hipStream_t st) {
  (void)hipGetLastError();  // start from a clean error state: report only our own launches
  bool done = false;
  hipError_t e = launch_tile<false>(a, a.I, MT, max_groups, st, &done);
  if (e == hipSuccess && !done) e = launch_generic<false>(a, a.I, MT, max_groups, n_cu, st);
  if (e != hipSuccess) return e;
  const size_t n4 = (size_t)a.T * a.H / 4;
  const int blocks = (int)((n4 + 255) / 256 < 4096 ? (n4 + 255) / 256 : 4096);
  combine_kernel<<<blocks, 256, 0, st>>>(a.out, a.y, a.T, a.H, a.k);
  return hipGetLastError();
}

}  // namespace mvq
