// Prefill form of the routed-expert step: the tokens of each expert are grouped into
// tiles of PF_BM tokens, and FC1 (gate/up, SiLU*up fused) and FC2 (down, routing weight
// fused) run as grouped matrix-core GEMMs (v_mfma_f32_16x16x32_f16) over expert weights
// decoded in registers.  The per-pair FC2 outputs are summed per token by the decode
// path's combine kernel.
//
// Sources: the routed experts are 2-bit vector codes with a sign-symmetric codebook,
// decoded on the fly (Tandem-vLLM 0.2.0 announcement, "How it works"; vLLM-Moet README,
// "2-bit experts on vLLM v0.24.0"); tokens are grouped per expert with no padding of an
// expert to a fixed row count and no padding rows written back (vLLM-Moet README, "What
// we changed against official vLLM", rows "MoE at decode" and "prefill").
//
// Operands.  A (activations) is fp16: x with one power-of-two factor per token (exact
// for bf16 values no smaller than 2^-24 of the token's largest), h with one per pair.
// B (weights) is decoded per lane: a VQ2 word through the LDS table of signed codebook
// vectors, times its group scale in fp16 (one rounding, relative error <= 2^-11); MXFP4
// bytes with the gfx950 FP4->FP16 convert, scaled by 2^(e - e_row) where e_row is the
// largest E8M0 exponent of the weight row, and 2^(e_row - 127) multiplies the row's fp32
// outputs: converted values are at most 6 in magnitude for any exponent, and exact while
// e >= e_row - 23.  The contraction index is permuted the same way in A and B: within a
// 128-wide scale group, lanes 16q..16q+15 hold k = 32q + 8s + (0..7) at MFMA step s, so
// one lane's codes for a group are contiguous (8 VQ2 bytes or 16 MXFP4 bytes).
//
// MFMA lane layout (16x16x32): A lane l holds row l%16, k = 8(l/16)+0..7; B lane l holds
// column l%16, the same k; D lane l holds column l%16, rows 4(l/16)+0..3.
#include <type_traits>

#include "moe_vq_device.h"
#include "moe_vq_launch.h"

namespace mvq {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int PF_THREADS = 256;
// The prefill table keeps 16 copies of the 256 signed codebook vectors (32 KiB): lookups
// are a small part of this kernel's LDS traffic, and the smaller table lets two
// workgroups share a CU.  Lane l reads copy l & 15 at byte b * 128 + (l & 15) * 8.
constexpr int PF_COPIES = 16;
constexpr int PF_AROW = PF_KG + 8;  // fp16 per staged row: 272 B, so 16 rows hit 16 bank groups

template <bool FC1>
struct PfGeom {
  static constexpr int NM = FC1 ? 2 : 1;                 // matrices (gate, up) or (down)
  static constexpr int NB = FC1 ? 2 : 4;                 // 16-row blocks per wave per matrix
  static constexpr int BN = (PF_THREADS / 64) * NB * 16;  // rows per tile
  static_assert(BN == (FC1 ? 128 : 256), "tile rows");
};

// The workspace was routed for this call (shape key, count of active experts, the same
// activations).  A refused call writes MOE_VQ_EINVAL into the status word (one lane of
// workgroup 0 of each kernel) and computes nothing, so moe_vq_check() reports it.
__device__ __forceinline__ bool pf_ws_ok(const PrefillArgs& a) {
  const uint32_t key = a.hdr[HDR_KEY], n_active = a.hdr[HDR_N_ACTIVE];
  const uint32_t xlo = a.hdr[HDR_X_LO], xhi = a.hdr[HDR_X_HI], xdt = a.hdr[HDR_X_DTYPE];
  const bool ok = (key == a.key) & (n_active <= (uint32_t)a.E) &
                  x_matches(xlo, xhi, xdt, (uint64_t)(uintptr_t)a.x, a.x_dtype);
  if (!ok && blockIdx.x == 0 && threadIdx.x == 0) {
    a.hdr[HDR_STATUS] = MOE_VQ_EINVAL;
    a.hdr[HDR_INFO] = 0xFFFFFFFFu;
  }
  return ok;
}

// ---------------------------------------------------------------------------------------
// x -> fp16 with one power-of-two factor per token; zero the per-pair max |h|
// ---------------------------------------------------------------------------------------

template <bool XF32>
__global__ __launch_bounds__(PF_THREADS) void prefill_stage_kernel(PrefillArgs a) {
  __shared__ float red[PF_THREADS / 64];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H;
  auto load8 = [&](int c, float* v) {
    if (XF32) {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.x) + (size_t)t * H + c);
      const float4 u = p[0], w = p[1];
      v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w; v[4] = w.x; v[5] = w.y; v[6] = w.z; v[7] = w.w;
    } else {
      const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + (size_t)t * H + c);
      const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[2 * q] = bf16_bits_to_f32(wd[q] & 0xFFFFu);
        v[2 * q + 1] = bf16_bits_to_f32(wd[q] >> 16);
      }
    }
  };
  float m = 0.f;
  for (int c = tid * 8; c < H; c += PF_THREADS * 8) {
    float v[8];
    load8(c, v);
#pragma unroll
    for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(v[q]));
  }
  m = wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  int ex = 0;
  if (m > 0.f && m == m) ex = frexp_exponent(m) - 15;  // |x| * 2^-ex < 2^15
  for (int c = tid * 8; c < H; c += PF_THREADS * 8) {
    float v[8];
    load8(c, v);
    uint4 o;
    uint32_t* ow = reinterpret_cast<uint32_t*>(&o);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const _Float16 lo = (_Float16)ldexp2(v[2 * q], -ex), hi = (_Float16)ldexp2(v[2 * q + 1], -ex);
      ow[q] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    *reinterpret_cast<uint4*>(a.x16 + (size_t)t * H + c) = o;
  }
  if (tid == 0) a.x16_e[t] = ex;
  if (tid < a.k) a.hmax[(size_t)t * a.k + tid] = 0u;
}

// ---------------------------------------------------------------------------------------
// Token-tile prefix over the active experts (one workgroup)
// ---------------------------------------------------------------------------------------

__global__ __launch_bounds__(1024) void prefill_setup_kernel(PrefillArgs a) {
  __shared__ int4 wave_tot[16];
  __shared__ int4 s_total;
  const int tid = threadIdx.x;
  if (!pf_ws_ok(a)) return;
  const int n_act = (int)a.hdr[HDR_N_ACTIVE];
  const int m = tid < n_act ? a.act_start[tid + 1] - a.act_start[tid] : 0;
  const int c = (m + PF_BM - 1) / PF_BM;
  const int4 sc = block_scan_excl4(make_int4(c, 0, 0, 0), wave_tot, &s_total);
  if (tid < n_act) a.mt_pre[tid] = sc.x;
  if (tid == 0) a.mt_pre[n_act] = s_total.x;
}

// ---------------------------------------------------------------------------------------
// Grouped GEMM tile: PF_BM tokens of one expert x BN rows
// ---------------------------------------------------------------------------------------

// Codes one lane needs for one (matrix, row block) and one scale group.
struct PfCodes {
  uint4 q;      // VQ2: 8 bytes in q.x, q.y; MXFP4: 16 bytes
  uint32_t s;   // VQ2: fp16 scale bits; MXFP4: E8M0 byte
};

template <int FMT>
__device__ __forceinline__ PfCodes pf_load_codes(const uint8_t* qb, const uint8_t* sb, int n, int K, int g, int kq) {
  PfCodes c;
  if (FMT == MOE_VQ_FMT_VQ2) {
    const uint2 v = *reinterpret_cast<const uint2*>(qb + (size_t)n * (K / 4) + g * 32 + kq * 8);
    c.q = make_uint4(v.x, v.y, 0u, 0u);
    c.s = *reinterpret_cast<const uint16_t*>(sb + ((size_t)n * (K / 128) + g) * 2);
  } else if (FMT == MOE_VQ_FMT_MXFP4) {
    c.q = *reinterpret_cast<const uint4*>(qb + (size_t)n * (K / 2) + g * 64 + kq * 16);
    c.s = sb[(size_t)n * (K / 32) + g * 4 + kq];
  } else {
    c.q = make_uint4(0u, 0u, 0u, 0u);
    c.s = 0u;
  }
  return c;
}

// B fragment (8 fp16 for k = 32q + 8s + 0..7) of step s.  erow: MXFP4 row exponent.
template <int FMT, int S>
__device__ __forceinline__ half8_t pf_decode(const uint2* tab, const PfCodes& c, uint32_t laneoff, int erow) {
  half8_t b;
  if (FMT == MOE_VQ_FMT_VQ2) {
    const uint32_t wd = (S < 2) ? c.q.x : c.q.y;
    // v_perm puts the code byte above the doubled lane offset; halving gives the address
    const uint2 e0 = tab_lookup(tab, tab_addr<(2 * S) & 3>(wd, laneoff) >> 1);
    const uint2 e1 = tab_lookup(tab, tab_addr<(2 * S + 1) & 3>(wd, laneoff) >> 1);
    const half2_t sc = __builtin_bit_cast(half2_t, (c.s & 0xFFFFu) * 0x10001u);
    const half2_t p0 = __builtin_bit_cast(half2_t, e0.x) * sc, p1 = __builtin_bit_cast(half2_t, e0.y) * sc;
    const half2_t p2 = __builtin_bit_cast(half2_t, e1.x) * sc, p3 = __builtin_bit_cast(half2_t, e1.y) * sc;
    b[0] = p0[0]; b[1] = p0[1]; b[2] = p1[0]; b[3] = p1[1];
    b[4] = p2[0]; b[5] = p2[1]; b[6] = p3[0]; b[7] = p3[1];
  } else if (FMT == MOE_VQ_FMT_MXFP4) {
    const uint32_t wd = S == 0 ? c.q.x : S == 1 ? c.q.y : S == 2 ? c.q.z : c.q.w;
    const float sc = ldexp2(1.0f, (int)c.s - erow);  // 2^(e - e_row), in (0, 1]
    const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, sc, 0);
    const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, sc, 1);
    const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, sc, 2);
    const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, sc, 3);
    b[0] = p0[0]; b[1] = p0[1]; b[2] = p1[0]; b[3] = p1[1];
    b[4] = p2[0]; b[5] = p2[1]; b[6] = p3[0]; b[7] = p3[1];
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) b[q] = (_Float16)0.f;
  }
  return b;
}

template <bool FC1>
struct PfTile {
  int p_lo, mcnt, nt;
  uint32_t fmt;
  uint64_t off;
};

// Main loop of one tile for one weight format.  rowf receives the factor of each of the
// lane's output rows (MXFP4: 2^(e_row - 127); VQ2: 1).  NMB: the 16-token blocks of the
// tile that hold tokens; the rest are neither staged, read nor multiplied (an expert's
// last tile often holds a few tokens: with about 130 tokens per expert, tiles of 64, 64
// and 2).
template <bool FC1, int FMT, int NMB>
__device__ __forceinline__ void pf_tile(const PrefillArgs& a, const PfTile<FC1>& tl, const uint2* tab,
                                        _Float16 (*As)[PF_BM * PF_AROW], f32x4_t (&acc)[PfGeom<FC1>::NM][PfGeom<FC1>::NB][4],
                                        const int* s_pair, const float* s_fac,
                                        float (&rowf)[PfGeom<FC1>::NM][PfGeom<FC1>::NB]) {
  using G = PfGeom<FC1>;
  constexpr int NM = G::NM, NB = G::NB, BN = G::BN;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i16 = lane & 15, kq = lane >> 4;
  const uint32_t laneoff = (uint32_t)(lane & 15) << 4;  // doubled: see PF_COPIES
  const int K = FC1 ? a.H : a.I;
  const int NROWS = FC1 ? a.I : a.H;
  const int NG = K / PF_KG;
  const SlotLayout& SL = FMT == MOE_VQ_FMT_MXFP4 ? a.mx4 : a.vq2;
  const uint8_t* slot = a.pool + tl.off;
  const uint8_t* qb[NM];
  const uint8_t* sb[NM];
  qb[0] = slot + (FC1 ? SL.q_gate : SL.q_down);
  sb[0] = slot + (FC1 ? SL.s_gate : SL.s_down);
  if (NM > 1) { qb[NM - 1] = slot + SL.q_up; sb[NM - 1] = slot + SL.s_up; }
  int rows[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)  // rows past the end re-read the last row; the epilogue drops them
    rows[nb] = min(tl.nt * BN + wave * NB * 16 + nb * 16 + i16, NROWS - 1);
  // MXFP4: the largest E8M0 exponent of each of the lane's rows.  The four lanes of a row
  // (kq = 0..3) read every fourth dword of its K/32 exponent bytes, eight dwords per row
  // and pass, every load of a pass issued before any is used.
  int erow[NM][NB];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      erow[m][nb] = 0;
      rowf[m][nb] = 1.0f;
    }
  if (FMT == MOE_VQ_FMT_MXFP4) {
    const int nd = K / 128;  // dwords of E8M0 bytes per row
    uint32_t mx[NM][NB];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) mx[m][nb] = 0u;
    for (int d0 = kq; d0 < nd; d0 += 32) {
      uint32_t w[NM][NB][8];
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint32_t* er = reinterpret_cast<const uint32_t*>(sb[m] + (size_t)rows[nb] * (K / 32));
#pragma unroll
          for (int i = 0; i < 8; ++i) w[m][nb][i] = d0 + 4 * i < nd ? er[d0 + 4 * i] : 0u;
        }
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t v = w[m][nb][i];
            mx[m][nb] = max(mx[m][nb], max(max(v & 0xFFu, (v >> 8) & 0xFFu), max((v >> 16) & 0xFFu, v >> 24)));
          }
    }
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        int e = (int)mx[m][nb];
        e = max(e, __shfl_xor(e, 16));
        e = max(e, __shfl_xor(e, 32));
        erow[m][nb] = e;
        rowf[m][nb] = e8m0_to_f32((uint32_t)e);
      }
  }

  // staging: thread tid stages 32 consecutive k of token row tid/4 (FC1: fp16 x; FC2:
  // the bf16 h that FC1 wrote, scaled by the pair's power-of-two factor into fp16)
  //
  // Every global load of the main loop is issued on every path: a load skipped on some
  // path (a guard on the group index, or a row past the tile's tokens) makes the compiler
  // count the loads in flight as on the shortest path, i.e. wait at the top of each group
  // for the loads just issued for two groups ahead.  Group indices past the end are
  // clamped (the loads re-read the last group), rows past the tile's tokens read the
  // tile's first row and are stored as zeros.
  const int srow = tid >> 2, skq = (tid & 3) * 32;
  const int sp = s_pair[srow];                 // -1 past the tile's tokens
  const int sp_ld = sp >= 0 ? sp : s_pair[0];  // (a tile holds at least one token)
  const bool stage = srow < NMB * 16;          // (one wave stages 16 rows: uniform per wave)
  constexpr int AV = 4;                        // 16-byte loads per thread per group
  auto a_load = [&](int g, uint4 (&v)[AV]) __attribute__((always_inline)) {
    const uint4* src = FC1 ? reinterpret_cast<const uint4*>(a.x16 + (size_t)(sp_ld / a.k) * K + g * PF_KG + skq)
                           : reinterpret_cast<const uint4*>(a.h + (size_t)sp_ld * K + g * PF_KG + skq);
#pragma unroll
    for (int i = 0; i < AV; ++i) v[i] = src[i];
  };
  auto a_store = [&](int buf, const uint4 (&v)[AV]) __attribute__((always_inline)) {
    if (!stage) return;
    uint4* dst = reinterpret_cast<uint4*>(&As[buf][srow * PF_AROW + skq]);
    const uint32_t keep = sp >= 0 ? 0xFFFFFFFFu : 0u;  // (a mask, not a select of operands)
    if (FC1) {
#pragma unroll
      for (int i = 0; i < AV; ++i) dst[i] = make_uint4(v[i].x & keep, v[i].y & keep, v[i].z & keep, v[i].w & keep);
    } else {
      // bf16 h -> fp16 with the pair's power-of-two factor
      const float f = s_fac[srow];
#pragma unroll
      for (int i = 0; i < AV; ++i) {
        const uint32_t* w = reinterpret_cast<const uint32_t*>(&v[i]);
        uint32_t ow[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float x0 = bf16_bits_to_f32(w[q] & 0xFFFFu) * f, x1 = bf16_bits_to_f32(w[q] >> 16) * f;
          ow[q] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x0) |
                  ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x1) << 16);
        }
        dst[i] = make_uint4(ow[0] & keep, ow[1] & keep, ow[2] & keep, ow[3] & keep);
      }
    }
  };

  // Codes and activations are loaded two groups ahead of their use: register set
  // g % 3 holds group g.  The loop is unrolled by three so the sets rotate by name and
  // no register holding an in-flight load is ever copied (a copy would wait for it).
  PfCodes cs0[NM][NB], cs1[NM][NB], cs2[NM][NB];
  uint4 as0[AV], as1[AV], as2[AV];
  auto codes_load = [&](int g, PfCodes (&c)[NM][NB]) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) c[m][nb] = pf_load_codes<FMT>(qb[m], sb[m], rows[nb], K, g, kq);
  };
  codes_load(0, cs0);
  codes_load(min(1, NG - 1), cs1);
  a_load(0, as0);
  a_load(min(1, NG - 1), as1);
  a_store(0, as0);
  __syncthreads();

  // group g: issue group g + 2, multiply group g, stage group g + 1's activations (after
  // the last group that store goes to the buffer no group reads again)
  auto body = [&](int g, const PfCodes (&cur)[NM][NB], PfCodes (&c_ahead)[NM][NB], const uint4 (&a_next)[AV],
                  uint4 (&a_ahead)[AV]) __attribute__((always_inline)) {
    const int ga = min(g + 2, NG - 1);
    codes_load(ga, c_ahead);
    a_load(ga, a_ahead);
    const _Float16* Ab = As[g & 1];
    if constexpr (FMT == MOE_VQ_FMT_VQ2) {
      // The group's B fragments j = (S, m, nb) in order.  Fragment j's two table lookups
      // are issued LA fragments ahead of its products, and step S + 1's A fragments two
      // fragments before the step starts, so that the LDS round trips run under earlier
      // fragments' MFMAs (scheduling barriers keep that order).
      constexpr int NF = NM * NB, J = 4 * NF, LA = 2;
      uint2 lk[J + LA][2];
      half8_t af[2][4];
      auto issue = [&](auto J_) __attribute__((always_inline)) {
        constexpr int j = decltype(J_)::value;
        if constexpr (j < J) {
          constexpr int S = j / NF, m = (j % NF) / NB, nb = j % NB;
          const uint32_t wd = S < 2 ? cur[m][nb].q.x : cur[m][nb].q.y;
          lk[j][0] = tab_lookup(tab, tab_addr<(2 * S) & 3>(wd, laneoff) >> 1);
          lk[j][1] = tab_lookup(tab, tab_addr<(2 * S + 1) & 3>(wd, laneoff) >> 1);
        }
      };
      auto a_frag = [&](auto S_) __attribute__((always_inline)) {
        constexpr int S = decltype(S_)::value;
        if constexpr (S < 4) {
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb)
            af[S & 1][mb] = *reinterpret_cast<const half8_t*>(&Ab[(mb * 16 + i16) * PF_AROW + 32 * kq + 8 * S]);
        }
      };
      a_frag(std::integral_constant<int, 0>{});
      static_for<0, LA>(issue);
      static_for<0, J>([&](auto J_) __attribute__((always_inline)) {
        constexpr int j = decltype(J_)::value;
        constexpr int S = j / NF, f = j % NF, m = f / NB, nb = f % NB;
        issue(std::integral_constant<int, j + LA>{});
        if constexpr (f == (NF > 2 ? NF - 2 : 0)) a_frag(std::integral_constant<int, S + 1>{});
        const half2_t sc = __builtin_bit_cast(half2_t, (cur[m][nb].s & 0xFFFFu) * 0x10001u);
        const uint2 e0 = lk[j][0], e1 = lk[j][1];
        const half2_t p0 = __builtin_bit_cast(half2_t, e0.x) * sc, p1 = __builtin_bit_cast(half2_t, e0.y) * sc;
        const half2_t p2 = __builtin_bit_cast(half2_t, e1.x) * sc, p3 = __builtin_bit_cast(half2_t, e1.y) * sc;
        half8_t bf;
        bf[0] = p0[0]; bf[1] = p0[1]; bf[2] = p1[0]; bf[3] = p1[1];
        bf[4] = p2[0]; bf[5] = p2[1]; bf[6] = p3[0]; bf[7] = p3[1];
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
          acc[m][nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[S & 1][mb], bf, acc[m][nb][mb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      });
      a_store((g + 1) & 1, a_next);
      __syncthreads();
      return;
    }
    auto step = [&](auto S_) __attribute__((always_inline)) {
      constexpr int S = decltype(S_)::value;
      half8_t af[NMB];
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
        af[mb] = *reinterpret_cast<const half8_t*>(&Ab[(mb * 16 + i16) * PF_AROW + 32 * kq + 8 * S]);
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const half8_t bf = pf_decode<FMT, S>(tab, cur[m][nb], laneoff, erow[m][nb]);
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb)
            acc[m][nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mb], bf, acc[m][nb][mb], 0, 0, 0);
        }
    };
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 3>{});
    a_store((g + 1) & 1, a_next);
    __syncthreads();
  };
  // three groups per iteration with no guard inside (see above), then the one or two left
  int g = 0;
  for (; g + 3 <= NG; g += 3) {
    body(g, cs0, cs2, as1, as2);
    body(g + 1, cs1, cs0, as2, as0);
    body(g + 2, cs2, cs1, as0, as1);
  }
  if (g < NG) body(g, cs0, cs2, as1, as2);
  if (g + 1 < NG) body(g + 1, cs1, cs0, as2, as0);
}

template <bool FC1>
__global__ __launch_bounds__(PF_THREADS, 2) void prefill_fc_kernel(PrefillArgs a) {
  using G = PfGeom<FC1>;
  constexpr int NM = G::NM, NB = G::NB, BN = G::BN;
  __shared__ uint2 tab[256 * PF_COPIES];
  __shared__ __align__(16) _Float16 As[2][PF_BM * PF_AROW];
  __shared__ int s_pair[PF_BM];
  __shared__ float s_fac[PF_BM];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i16 = lane & 15, kq = lane >> 4;
  if (!pf_ws_ok(a)) return;
  const int NROWS = FC1 ? a.I : a.H;
  const int NT = (NROWS + BN - 1) / BN;
  const int n_act = (int)a.hdr[HDR_N_ACTIVE];
  // XCD-aware order: workgroups go to the 8 XCDs round-robin (block b to XCD b % 8),
  // each with its own L2.  XCD x takes the x-th eighth of the logical tiles (token tile
  // major, row tile minor, experts in order), so the row tiles that share one token
  // tile's activations, and the token tiles that share one expert's codes, run together
  // on one XCD and read those bytes into one L2 instead of eight.
  const int n_valid = a.mt_pre[n_act] * NT;
  const int per = (n_valid + 7) / 8;
  const int jx = blockIdx.x >> 3;
  if (jx >= per) return;
  const int L = (blockIdx.x & 7) * per + jx;
  if (L >= n_valid) return;
  // active expert of this logical tile: the last rank whose tiles start at or before it
  // (an expert's tiles are the logical tiles mt_pre[e] * NT .. mt_pre[e + 1] * NT - 1)
  int lo = 0, hi = n_act - 1;
  {
    const int mtl = L / NT;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.mt_pre[mid] <= mtl) lo = mid; else hi = mid - 1;
    }
  }
  // within the expert, row tile major: its token tiles that share one row tile's codes
  // run next to each other
  const int ce = a.mt_pre[lo + 1] - a.mt_pre[lo];
  const int li = L - a.mt_pre[lo] * NT;
  const int mt = a.mt_pre[lo] + li % ce;
  PfTile<FC1> tl;
  tl.nt = li / ce;
  tl.p_lo = a.act_start[lo] + (mt - a.mt_pre[lo]) * PF_BM;
  tl.mcnt = min(PF_BM, a.act_start[lo + 1] - tl.p_lo);
  tl.fmt = a.act_fmt[lo];
  tl.off = a.act_off[lo];

  {
    const uint2* cb2 = reinterpret_cast<const uint2*>(a.codebook);
    for (int idx = tid; idx < 256 * PF_COPIES; idx += PF_THREADS) {
      const int b = idx / PF_COPIES;
      const uint2 v = cb2[b & 127];
      const uint32_t flip = (b & 128) ? 0x80008000u : 0u;
      tab[idx] = make_uint2(v.x ^ flip, v.y ^ flip);
    }
  }
  if (tid < PF_BM) {
    const int p = tid < tl.mcnt ? a.pair_list[tl.p_lo + tid] : -1;
    s_pair[tid] = p;
    float f = 1.f;
    if (!FC1 && p >= 0) {
      const float hm = __builtin_bit_cast(float, a.hmax[p]);
      const int ex = (hm > 0.f && hm == hm) ? frexp_exponent(hm) - 15 : 0;
      f = ldexp2(1.0f, -ex);
    }
    s_fac[tid] = f;
  }
  __syncthreads();

  f32x4_t acc[NM][NB][4];
  float rowf[NM][NB];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      rowf[m][nb] = 1.0f;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[m][nb][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  // (an absent expert keeps zeros; the worklist has set MOE_VQ_ENOTRESIDENT)
  auto run = [&](auto NMB_) __attribute__((always_inline)) {
    constexpr int NMB = decltype(NMB_)::value;
    if (tl.fmt == MOE_VQ_FMT_VQ2) pf_tile<FC1, MOE_VQ_FMT_VQ2, NMB>(a, tl, tab, As, acc, s_pair, s_fac, rowf);
    else if (tl.fmt == MOE_VQ_FMT_MXFP4) pf_tile<FC1, MOE_VQ_FMT_MXFP4, NMB>(a, tl, tab, As, acc, s_pair, s_fac, rowf);
  };
  switch ((tl.mcnt + 15) >> 4) {  // (a tile holds 1 .. PF_BM tokens)
    case 1: run(std::integral_constant<int, 1>{}); break;
    case 2: run(std::integral_constant<int, 2>{}); break;
    case 3: run(std::integral_constant<int, 3>{}); break;
    default: run(std::integral_constant<int, 4>{}); break;
  }

  // epilogue: D lane holds column i16 (output row) and token rows 4*kq + 0..3 of each block
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = mb * 16 + 4 * kq + r;
      const int p = s_pair[row];
      float hm = 0.f;
      if (p >= 0) {
        if (FC1) {
          const float f = ldexp2(1.0f, a.x16_e[p / a.k]);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const int n = tl.nt * BN + wave * NB * 16 + nb * 16 + i16;
            const float gv = acc[0][nb][mb][r] * (f * rowf[0][nb]), uv = acc[1][nb][mb][r] * (f * rowf[1][nb]);
            const float h = swiglu(gv, uv, a.lim);
            if (n < NROWS) {
              a.h[(size_t)p * a.I + n] = f32_to_bf16_rne(h);
              hm = fmaxf(hm, fabsf(h));
            }
          }
        } else {
          const float f = a.pair_w[p] / s_fac[row];
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const int n = tl.nt * BN + wave * NB * 16 + nb * 16 + i16;
            if (n < NROWS) a.o_buf[(size_t)p * a.H + n] = acc[0][nb][mb][r] * (f * rowf[0][nb]);
          }
        }
      }
      if (FC1) {
        // the 16 lanes of one token row are one DPP row: reduce, then one atomic per row
        hm = fmaxf(hm, dpp_f32<dpp::QUAD_XOR1>(hm));
        hm = fmaxf(hm, dpp_f32<dpp::QUAD_XOR2>(hm));
        hm = fmaxf(hm, dpp_f32<dpp::ROW_HALF_MIRROR>(hm));
        hm = fmaxf(hm, dpp_f32<dpp::ROW_MIRROR>(hm));
        if (i16 == 0 && p >= 0) atomicMax(&a.hmax[p], __builtin_bit_cast(uint32_t, hm));
      }
    }
}

// ---------------------------------------------------------------------------------------
// Host launcher
// ---------------------------------------------------------------------------------------

hipError_t launch_prefill(const PrefillArgs& a, int x_dtype, hipStream_t st) {
  (void)hipGetLastError();  // start from a clean error state: report only our own launches
  if (x_dtype == MOE_VQ_F32) prefill_stage_kernel<true><<<a.T, PF_THREADS, 0, st>>>(a);
  else prefill_stage_kernel<false><<<a.T, PF_THREADS, 0, st>>>(a);
  prefill_setup_kernel<<<1, 1024, 0, st>>>(a);
  const long mt_max = pf_max_mtiles(a.T, a.k, a.E);
  // (rounded up to whole rounds of the 8 XCDs: the kernel maps block b to XCD b % 8)
  const long g1 = (mt_max * ((a.I + pf_rows_per_tile(true) - 1) / pf_rows_per_tile(true)) + 7) & ~7L;
  const long g2 = (mt_max * ((a.H + pf_rows_per_tile(false) - 1) / pf_rows_per_tile(false)) + 7) & ~7L;
  if (g1 > 0x7FFFFFFF || g2 > 0x7FFFFFFF) return hipErrorInvalidValue;
  prefill_fc_kernel<true><<<(unsigned)g1, PF_THREADS, 0, st>>>(a);
  prefill_fc_kernel<false><<<(unsigned)g2, PF_THREADS, 0, st>>>(a);
  const size_t n4 = (size_t)a.T * a.H / 4;
  const int blocks = (int)((n4 + 255) / 256 < 4096 ? (n4 + 255) / 256 : 4096);
  launch_combine(a.o_buf, a.y, a.T, a.H, a.k, 0, blocks, st);
  return hipGetLastError();
}

}  // namespace mvq
