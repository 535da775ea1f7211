// Decode-path FC1 (gate/up, SiLU*up fused) and FC2 (down, routing weight fused) on the
// matrix cores, for token groups of MT <= 4 tokens of one expert.
//
// Sources: the routed experts are 2-bit vector codes with a sign-symmetric codebook,
// decoded on the fly (Tandem-vLLM 0.2.0 announcement, "How it works"; vLLM-Moet README,
// "2-bit experts on vLLM v0.24.0"); FC1 then FC2 per expert with no padding of an
// expert to a fixed row count (vLLM-Moet README, "What we changed against official
// vLLM", row "MoE at decode"); silu*up fused into the expert product (vLLM-Moet README,
// "Qwen3.8-Flash-Next-FP8 on 4x RTX PRO 6000").
//
// The product of a group of at most 4 tokens with one expert matrix is a GEMV-like
// problem bound by the code stream.  It runs on v_mfma_f32_16x16x32_f16 anyway,
// because there the contraction over k happens inside the matrix core.  That removes
// the per-row cross-lane sums, and only the lanes that carry a real token read
// activations from LDS.  The 12 or 15 padding token rows cost matrix-core cycles only,
// and those are idle in this kernel.
//
// B operand: a lane's 8 code bytes of one 128-wide scale group are 8 table lookups of
// signed codebook vectors, which are exact fp16 values.  The group scale multiplies the
// group's partial product afterwards in fp32, so no weight is rounded.  The contraction
// index is permuted identically in A and B: within a group, lanes 16q..16q+15 hold
// k = 32q + 8s + (0..7) at MFMA step s.
//
// A operand: the staged activations, fp16 with one power-of-two factor per (token, 1024
// columns) (exact for bf16 x); the factor also multiplies the group's product.
//
// Work: a tile is (token group, 16 * NB rows); the eight waves of a workgroup take the
// eight parts of K, and their partial sums meet in LDS at the end of the tile.  Each
// wave keeps its whole part of the next tile's codes in flight: the register ring
// slot of a (group, matrix, row block) is reloaded with the next tile's codes right
// after this tile has consumed it.
#include <type_traits>

#include "fc_common.h"

namespace mvq {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int MF_WAVES = 8;                 // waves per workgroup; each takes 1/8 of K
constexpr int MF_THREADS = 64 * MF_WAVES;

template <int CPL, bool FC1>
struct MfGeom {
  static constexpr int K = 1024 * CPL;
  static constexpr int NM = FC1 ? 2 : 1;
  static constexpr int NGQ = CPL;      // 128-wide scale groups in a wave's eighth of K
  // 16-row blocks per tile: enough (group, matrix, block) ring slots per wave to keep
  // 14-16 loads of 512 bytes in flight
  static constexpr int NB = CPL >= 4 ? (FC1 ? 1 : 2) : (FC1 ? 8 / CPL : 16 / CPL);
  static constexpr int ROWS = 16 * NB;
  static constexpr int KS = CPL;       // activation slices of 1024 columns
  // MXFP4 tiles load MXG groups per pass: the largest divisor of NGQ whose codes fit in
  // about 80 registers next to the (live) VQ2 ring
  static constexpr int mxg() {
    int best = 1;
    for (int d = 1; d <= NGQ; ++d)
      if (NGQ % d == 0 && d * NM * NB * 5 <= 80) best = d;
    return best;
  }
  static constexpr int MXG = mxg();
};

// VQ2 codes one lane holds for one (group, matrix, row block): 8 code bytes and the
// group's fp16 scale bits.
struct MfCode {
  uint2 q;
  uint32_t s;
};

// MXFP4 codes of one (group, matrix, row block): 16 bytes (32 weights, one E8M0 block).
struct MfMx {
  uint4 q;
  uint32_t e;
};

size_t mf_lds_bytes(int MT, int K, bool fc1) {
  const int cpl = K / 1024;
  const int nm = fc1 ? 2 : 1;
  const int nb = cpl >= 4 ? (fc1 ? 1 : 2) : (fc1 ? 8 / cpl : 16 / cpl);
  const size_t b = (size_t)TAB_BYTES + (size_t)MT * K * 2 + (size_t)MT * cpl * 4 +
                   (size_t)2 * MF_WAVES * nm * nb * 16 * MT * 4 + (size_t)MF_WAVES * MT * cpl * 4;
  return (b + 511) & ~(size_t)511;
}

template <int CPL, int MT, bool FC1>
__global__ __launch_bounds__(MF_THREADS, 1) void fc_mfma_kernel(FcArgs a) {
  using G = MfGeom<CPL, FC1>;
  constexpr int K = G::K, NM = G::NM, NB = G::NB, ROWS = G::ROWS, NGQ = G::NGQ, KS = G::KS;
  __shared__ uint2 tab[256 * TAB_COPIES];
  __shared__ __align__(16) _Float16 xs[MT * K];
  __shared__ float xsc[MT * KS];
  __shared__ float red[2][MF_WAVES][NM][NB][16][MT];
  __shared__ float smax[MF_WAVES][MT * KS];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i16 = lane & 15, kq = lane >> 4;
  const uint32_t laneoff = (uint32_t)(lane & 31) << 3;
  const int NROWS = FC1 ? a.I : a.H;
  const int RB = (NROWS + ROWS - 1) / ROWS;
  const int g0 = uni(wave) * NGQ;  // first scale group of this wave's eighth of K

  const uint2 cbv = reinterpret_cast<const uint2*>(a.codebook)[tid & 127];
  if (!ws_ok(a, FC1, MT)) return;
  const int n_tiles = (int)a.hdr[FC1 ? HDR_GROUPS1 : HDR_GROUPS2] * RB;
  const int t_begin = (int)(((long)blockIdx.x * n_tiles) / gridDim.x);
  const int t_end = (int)(((long)(blockIdx.x + 1) * n_tiles) / gridDim.x);
  if (t_begin >= t_end) return;

  // Stage the activations of record r (FC1: fp16 x of its tokens; FC2: h of its pairs,
  // scaled to fp16 with one power-of-two factor per 1024-column slice).
  auto stage = [&](const RecS& r) __attribute__((always_inline)) {
    const int t0 = opaque(threadIdx.x);
    const int w0 = t0 >> 6, l0 = t0 & 63;
    if (FC1) {
      constexpr int XU = (K / 8 + MF_THREADS - 1) / MF_THREADS;
      uint4 xv[MT][XU];
      float scv[MT];
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        const bool live = j < r.mcount;
        const size_t tok = live ? (size_t)(r.pair[j] / a.k) : 0;
        const uint4* src = reinterpret_cast<const uint4*>(a.x_h + tok * K);
#pragma unroll
        for (int i = 0; i < XU; ++i) {
          const int o = t0 + i * MF_THREADS;
          xv[j][i] = (live && o < K / 8) ? src[o] : make_uint4(0u, 0u, 0u, 0u);
        }
        scv[j] = (live && t0 < KS) ? a.x_sc[tok * KS + t0] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < MT; ++j) {
#pragma unroll
        for (int i = 0; i < XU; ++i) {
          const int o = t0 + i * MF_THREADS;
          if (o < K / 8) reinterpret_cast<uint4*>(xs + j * K)[o] = xv[j][i];
        }
        if (t0 < KS) xsc[j * KS + t0] = scv[j];
      }
    } else {
      // one slice of 1024 columns is 512 threads x 2 values
      float2 hv[MT * KS];
#pragma unroll
      for (int j = 0; j < MT; ++j)
#pragma unroll
        for (int s = 0; s < KS; ++s)
          hv[j * KS + s] = j < r.mcount
                               ? reinterpret_cast<const float2*>(a.h_in + (size_t)r.pair[j] * K)[s * 512 + t0]
                               : make_float2(0.f, 0.f);
#pragma unroll
      for (int js = 0; js < MT * KS; ++js) {
        const float2 v = hv[js];
        float m = fmaxf(fabsf(v.x), fabsf(v.y));
        m = wave_max(m);
        if (l0 == 0) smax[w0][js] = m;
      }
      __syncthreads();
#pragma unroll
      for (int js = 0; js < MT * KS; ++js) {
        float m = smax[0][js];
#pragma unroll
        for (int w = 1; w < MF_WAVES; ++w) m = fmaxf(m, smax[w][js]);
        int ex = 0;
        if (m > 0.f && m == m) ex = frexp_exponent(m) - 15;
        const float2 v = hv[js];
        const int j = js / KS, s = js % KS;
        reinterpret_cast<uint32_t*>(xs + j * K + s * SLICE)[t0] = pack_half2(ldexp2(v.x, -ex), ldexp2(v.y, -ex));
        if (t0 == 0) xsc[js] = j < r.mcount ? ldexp2(1.0f, ex) : 0.f;
      }
    }
  };

  // Addresses of one tile's VQ2 codes: uniform matrix bases, one 32-bit offset per lane
  // and row block (row, first group of the wave's part of K, lane's 8 bytes); the group
  // offset gi*32 (gi*2 for the scales) is the load instruction's immediate.
  struct MfAddr {
    const uint8_t* qb[NM];
    const uint8_t* sb[NM];
    uint32_t qo[NB], so[NB];
  };
  auto vq_addr = [&](const RecS& r, int rb) __attribute__((always_inline)) -> MfAddr {
    MfAddr d;
    const uint8_t* slot = a.pool + r.slot_off;
    d.qb[0] = slot + (FC1 ? a.vq2.q_gate : a.vq2.q_down);
    d.sb[0] = slot + (FC1 ? a.vq2.s_gate : a.vq2.s_down);
    if (NM > 1) { d.qb[NM - 1] = slot + a.vq2.q_up; d.sb[NM - 1] = slot + a.vq2.s_up; }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      // rows past the end (ragged shapes only) re-read the last row; the epilogue drops them
      const uint32_t n = (uint32_t)min(rb * ROWS + nb * 16 + i16, NROWS - 1);
      d.qo[nb] = n * (uint32_t)(K / 4) + (uint32_t)(g0 * 32 + kq * 8);
      d.so[nb] = (n * (uint32_t)(K / 128) + (uint32_t)g0) * 2u;
    }
    return d;
  };
  auto vq_load = [&](const MfAddr& d, int gi, int m, int nb) __attribute__((always_inline)) -> MfCode {
    MfCode c;
    c.q = *reinterpret_cast<const uint2*>(d.qb[m] + d.qo[nb] + gi * 32);
    c.s = *reinterpret_cast<const uint16_t*>(d.sb[m] + d.so[nb] + gi * 2);
    return c;
  };

  // A fragments of group g.  Rows of the product are independent, so the lanes of the
  // padding token rows (i16 >= MT) read a real row too: their results are never used
  // (their factors are 0 and the epilogue writes rows < MT only), and the reads need no
  // branch.
  const _Float16* xrow = xs + (i16 % MT) * K + 32 * kq;
  auto a_frags = [&](int g, half8_t (&af)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 4; ++s) af[s] = *reinterpret_cast<const half8_t*>(xrow + g * 128 + 8 * s);
  };
  // per-lane factor of D row r (token 4*kq + r) for activation slice sl; 0 for the
  // padding rows
  const bool real_rows = kq == 0;
  auto x_factors = [&](int sl, float (&fx)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = xsc[(r < MT ? r : MT - 1) * KS + sl];
      fx[r] = (real_rows && r < MT) ? v : 0.f;
    }
  };

  f32x4_t acc[NM][NB];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[m][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };

  // VQ2 tile: consume the ring, refilling each slot with the next tile's codes
  MfCode ring[NGQ][NM][NB];
  auto compute_vq = [&](bool refill, const RecS& rn, int rbn) __attribute__((always_inline)) {
    const MfAddr dn = vq_addr(rn, rbn);
#pragma unroll
    for (int gi = 0; gi < NGQ; ++gi) {
      const int g = g0 + gi;
      half8_t af[4];
      a_frags(g, af);
      float fx[4];
      x_factors(g >> 3, fx);
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          // the slot is consumed (lookups, scale) before its refill is issued, so the
          // refill can land in the same registers: no copies of in-flight loads at
          // the loop edge (a copy would wait for the load)
          const MfCode c = ring[gi][m][nb];
          half8_t bfr[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const uint32_t wd = s < 2 ? c.q.x : c.q.y;
            const uint2 e0 = tab_lookup(tab, tab_addr_sel(wd, laneoff, (2 * s) & 3));
            const uint2 e1 = tab_lookup(tab, tab_addr_sel(wd, laneoff, (2 * s + 1) & 3));
            bfr[s] = __builtin_bit_cast(half8_t, make_uint4(e0.x, e0.y, e1.x, e1.y));
          }
          const float sc = f16_bits_to_f32(c.s);
          if (refill) ring[gi][m][nb] = vq_load(dn, gi, m, nb);
          f32x4_t tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 4; ++s) tmp = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[s], bfr[s], tmp, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[m][nb][r] = fmaf(sc * fx[r], tmp[r], acc[m][nb][r]);
        }
    }
  };

  // MXFP4 tile (not pipelined): MXG groups of the wave's part of K per pass
  auto compute_mx = [&](const RecS& r, int rb) __attribute__((always_inline)) {
    const uint8_t* slot = a.pool + r.slot_off;
#pragma unroll
    for (int h = 0; h < NGQ / G::MXG; ++h) {
      constexpr int NH = G::MXG;
      MfMx mx[NH][NM][NB];
#pragma unroll
      for (int j = 0; j < NH; ++j)
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const uint8_t* qb = slot + (m == 0 ? (FC1 ? a.mx4.q_gate : a.mx4.q_down) : a.mx4.q_up);
            const uint8_t* sb = slot + (m == 0 ? (FC1 ? a.mx4.s_gate : a.mx4.s_down) : a.mx4.s_up);
            const uint32_t n = (uint32_t)min(rb * ROWS + nb * 16 + i16, NROWS - 1);
            const int g = g0 + h * NH + j;
            mx[j][m][nb].q = *reinterpret_cast<const uint4*>(qb + n * (uint32_t)(K / 2) + (uint32_t)(g * 64 + kq * 16));
            mx[j][m][nb].e = sb[n * (uint32_t)(K / 32) + (uint32_t)(g * 4 + kq)];
          }
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        const int g = g0 + h * NH + j;
        half8_t af[4];
        a_frags(g, af);
        float fx[4];
        x_factors(g >> 3, fx);
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const float es = e8m0_to_f32(mx[j][m][nb].e);
            f32x4_t tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const uint32_t wd = s == 0 ? mx[j][m][nb].q.x : s == 1 ? mx[j][m][nb].q.y
                                : s == 2 ? mx[j][m][nb].q.z : mx[j][m][nb].q.w;
              const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, es, 0);
              const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, es, 1);
              const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, es, 2);
              const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, es, 3);
              const half8_t b = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
              tmp = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[s], b, tmp, 0, 0, 0);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[m][nb][q] = fmaf(fx[q], tmp[q], acc[m][nb][q]);
          }
      }
    }
  };

  // End of a tile: the eight waves' partial sums meet in LDS, then the outputs.
  auto finish = [&](const RecS& r, int rb, int buf) __attribute__((always_inline)) {
    if (kq == 0) {
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int q = 0; q < MT; ++q) red[buf][wave][m][nb][i16][q] = acc[m][nb][q];
    }
    __syncthreads();
    if (tid < NB * 16) {
      const int nb = tid >> 4, i = tid & 15;
      const int n = rb * ROWS + nb * 16 + i;
#pragma unroll
      for (int q = 0; q < MT; ++q) {
        if (q < r.mcount && n < NROWS) {
          float v[NM];
#pragma unroll
          for (int m = 0; m < NM; ++m)
          {
            float sum = red[buf][0][m][nb][i][q];
#pragma unroll
            for (int w = 1; w < MF_WAVES; ++w) sum += red[buf][w][m][nb][i][q];
            v[m] = sum;
          }
          const int p = r.pair[q];
          if (FC1) a.out[(size_t)p * a.I + n] = silu_fast(v[0]) * v[NM - 1];
          else a.out[(size_t)p * a.H + n] = a.pair_w[p] * v[0];
        }
      }
    }
  };

  // Loads of a whole ring for tile (r, rb), in the order the refills use (group,
  // matrix, row block); the scheduling barriers keep that order, so that the count of
  // loads in flight after each slot is the same whichever way the loop is entered.
  auto ring_load = [&](const RecS& r, int rb) __attribute__((always_inline)) {
    const MfAddr d = vq_addr(r, rb);
#pragma unroll
    for (int gi = 0; gi < NGQ; ++gi)
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          ring[gi][m][nb] = vq_load(d, gi, m, nb);
          __builtin_amdgcn_sched_barrier(0);
        }
  };

  // ---- prologue.  Records are read one tile ahead of their use (rn is needed for the
  // refill addresses while this tile decodes; reading it later would wait for loads
  // issued after it).
  int t = t_begin;
  RecS rc = load_rec(a.rec, t / RB);
  RecS rn = (t + 1 < t_end) ? load_rec(a.rec, (t + 1) / RB) : rc;
  stage(rc);  // staging loads are issued before the code loads
  if (rc.fmt == MOE_VQ_FMT_VQ2) ring_load(rc, t % RB);
  if (tid < 256) write_table_entry(tab, cbv, tid);
  __syncthreads();

  int buf = 0;
  for (;;) {
    const int tn = t + 1;
    const bool more = tn < t_end;
    const RecS rnn = (tn + 1 < t_end) ? load_rec(a.rec, (tn + 1) / RB) : rn;
    const bool next_vq = more && rn.fmt == MOE_VQ_FMT_VQ2;
    zero_acc();
    if (rc.fmt == MOE_VQ_FMT_VQ2) {
      compute_vq(next_vq, rn, tn % RB);  // refills the ring with tile tn's codes
    } else {
      if (rc.fmt == MOE_VQ_FMT_MXFP4) compute_mx(rc, t % RB);
      // (an absent expert keeps zeros; the worklist has recorded MOE_VQ_ENOTRESIDENT)
      if (next_vq) ring_load(rn, tn % RB);
    }
    finish(rc, t % RB, buf);
    if (!more) break;
    if (!same_inputs<MT, FC1>(rn, rc, a.k)) {
      __syncthreads();  // every wave is done with the staged activations
      stage(rn);
      __syncthreads();
    }
    rc = rn;
    rn = rnn;
    t = tn;
    buf ^= 1;
  }
}

// ---------------------------------------------------------------------------------------
// Host launcher
// ---------------------------------------------------------------------------------------

template <bool FC1>
hipError_t launch_mfma(const FcArgs& a, int K, int MT, int max_groups, int n_cu, hipStream_t st, bool* done) {
  *done = false;
  // token groups of 4; single tokens take the vector-ALU stream kernel
  if (K % 1024 != 0 || MT != 4) return hipSuccess;
  const int cpl = K / 1024;
  const int nrows = FC1 ? a.I : a.H;
  const size_t lds = mf_lds_bytes(MT, K, FC1);
  if (lds > (size_t)LDS_LIMIT) return hipSuccess;
  const int per_cu = 1;  // 8 waves of up to 256 registers fill a CU
#define MVQ_MFMA_CASE(C, M)                                                                  \
  if (cpl == C && MT == M) {                                                                 \
    constexpr int ROWS = MfGeom<C, FC1>::ROWS;                                               \
    const long tiles = (long)max_groups * ((nrows + ROWS - 1) / ROWS);                      \
    long grid = (long)n_cu * per_cu;                                                         \
    if (tiles < grid) grid = tiles;                                                          \
    *done = true;                                                                            \
    if (grid <= 0) return hipSuccess;                                                        \
    fc_mfma_kernel<C, M, FC1><<<(unsigned)grid, MF_THREADS, 0, st>>>(a);                     \
    return hipGetLastError();                                                                \
  }
  MVQ_MFMA_CASE(1, 4) MVQ_MFMA_CASE(2, 4) MVQ_MFMA_CASE(7, 4)
#undef MVQ_MFMA_CASE
  return hipSuccess;
}

template hipError_t launch_mfma<true>(const FcArgs&, int, int, int, int, hipStream_t, bool*);
template hipError_t launch_mfma<false>(const FcArgs&, int, int, int, int, hipStream_t, bool*);

}  // namespace mvq
