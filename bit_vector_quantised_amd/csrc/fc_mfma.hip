// Decode-path FC1 (gate/up, SiLU*up fused) and FC2 (down, routing weight fused) on the
// matrix cores, for token groups of up to MF_MT = 16 tokens of one expert.
//
// Sources: the routed experts are 2-bit vector codes with a sign-symmetric codebook,
// decoded on the fly (Tandem-vLLM 0.2.0 announcement, "How it works"; vLLM-Moet README,
// "2-bit experts on vLLM v0.24.0"); FC1 then FC2 per expert with no padding of an
// expert to a fixed row count (vLLM-Moet README, "What we changed against official
// vLLM", row "MoE at decode"); silu*up fused into the expert product (vLLM-Moet README,
// "Qwen3.8-Flash-Next-FP8 on 4x RTX PRO 6000").
//
// The product of a group of at most 16 tokens with one expert matrix is a GEMV-like
// problem bound by the code stream.  It runs on v_mfma_f32_16x16x32_f16: the 16 rows of
// the A operand are the group's tokens, so each expert is read once per 16 tokens (the
// Zipf-skewed batches give some experts many tokens), and the contraction over k
// happens inside the matrix core, with no per-row cross-lane sums.
//
// A operand: held in registers for the whole token group, never in LDS, so that the
// only LDS traffic of the inner loop is the codebook lookups.  Each wave holds its part
// of K of the group's activations in fp16 with one power-of-two factor per token (FC1:
// the staged x, brought to a common factor over the part, exact for bf16 x) or per pair
// (FC2: fp32 h rounded to fp16).  The factor multiplies the wave's partial sums once
// per tile, so a scale group costs four fp32 FMAs beyond its matrix ops; FC2's routing
// weight multiplies each pair's output in fp32.
//
// MXFP4 B operand: a lane's 32 weights of a group are one E8M0 block.  The four blocks of
// a 128-wide group (held by the four lanes of a row) share one product, so each block is
// converted to fp16 with 2^(e - e_max), e_max the largest of the four exponents, and
// 2^(e_max - 127) multiplies the group's fp32 sum.  The converted values are at most 6 in
// magnitude (no overflow for any exponent) and exact while e >= e_max - 23; elements of a
// block more than 23 binades below its group's largest are rounded (each is below
// 2^-22 of that block's unit).
//
// B operand: a lane's code bytes of one 128-wide scale group are table lookups of signed
// codebook vectors, which are exact fp16 values.  The group scale multiplies the group's
// partial product afterwards in fp32, so no weight is rounded.  Codes arrive as 16-byte
// loads that cover two scale groups (16 rows x 64 bytes per instruction); one
// v_permlane32_swap per dword pair regroups them so that every lane holds 8 code bytes
// of each group.  The contraction index is permuted identically in A and B: within a
// group, lanes 16q..16q+15 hold k = 32 p(q) + 8s + (0..7) at MFMA step s, with
// p = (0, 2, 1, 3).
//
// Work: a tile is (token group, 16 * NB rows); the W waves of a workgroup take the W
// parts of K, and their partial sums meet in LDS at the end of the tile.  Each
// wave keeps its whole part of the next tile's codes in flight: the register ring slot
// of a (group pair, matrix, row block) is reloaded with the next tile's codes right
// after this tile has consumed it.
#include <type_traits>

#include "fc_common.h"

namespace mvq {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Waves per workgroup; each takes 1/W of K and holds its part of the A fragments in
// registers.  W = 8: two waves per SIMD with 256 registers each (at K = 7168 the A
// fragments of 7 groups take 112).  One wave per SIMD (W = 4, 512 registers) measured
// slower: two waves per SIMD hide each other's LDS and load latency.
template <int CPL, bool FC1>
constexpr int mf_waves() { return 8; }

template <int CPL, bool FC1>
struct MfGeom {
  static constexpr int W = mf_waves<CPL, FC1>();
  static constexpr int THREADS = 64 * W;
  static constexpr int K = 1024 * CPL;
  static constexpr int NM = FC1 ? 2 : 1;
  static constexpr int NGQ = 8 * CPL / W;  // 128-wide scale groups in a wave's part of K
  static constexpr int KS = CPL;           // activation slices of 1024 columns (FC1 factors)
  static constexpr int NPAIR = NGQ / 2;  // groups read two at a time (16-byte loads)
  static constexpr bool ODD = (NGQ & 1) != 0;  // the last group is read alone (8 bytes)
  // 16-row blocks per tile: ring slots per wave for several KB of codes in flight (a
  // tile's time is mostly load latency, so more bytes per tile is more throughput); FC1
  // at most 4 blocks with eight waves (registers), at most 8 (matrix, block) pairs so the
  // partial sums fit in LDS
  static constexpr int NB_RULE = CPL >= 4 ? (FC1 ? 1 : 2) : (FC1 ? 8 / CPL : 16 / CPL);
  static constexpr int NB_CAP = W == 8 ? (FC1 ? 4 : 8) : 8 / NM;
  static constexpr int NB = NB_RULE < NB_CAP ? NB_RULE : NB_CAP;
  static constexpr int ROWS = 16 * NB;
  static_assert(ROWS == mf_tile_rows(CPL, FC1), "the worklist's tile split assumes this tile height");
  static constexpr int QS = ROWS + 1;  // LDS stride of one token's partial sums
  static constexpr int RED = W * NM * MF_MT * QS;  // floats per reduction buffer
  static constexpr int NBUF = (size_t)TAB_BYTES + 2 * (size_t)RED * 4 <= (size_t)150 * 1024 ? 2 : 1;
  // MXFP4 groups beyond the ring's load in passes of up to MXG groups: as many as fit in
  // about 40 registers (80 with one wave per SIMD)
  // (30 with two waves per SIMD, where the A fragments take 112 of 256)
  static constexpr int mxg() {
    const int budget = W == 4 ? 80 : 40;
    int best = 1;
    for (int d = 1; d <= NGQ; ++d)
      if (d * NM * NB * 5 <= budget) best = d;
    return best;
  }
  static constexpr int MXG = mxg();
  // VQ2 scales staged through LDS (SST): a tile's scale rows are contiguous per matrix,
  // so the workgroup reads them with one 16-byte load per thread instead of one 4-byte
  // load per lane and group pair (16 rows per instruction: half of the memory requests
  // for 3 % of the bytes).  Measured faster for FC2 and the small-K kernels, slightly
  // slower for FC1 at K = 7168, which keeps its scales in the ring.  Bytes per row, LDS
  // row stride (an odd number of dwords: the 16 rows a wave reads at once fall in
  // distinct banks), 16-byte chunks per row, chunks per tile, bytes per buffer.
  static constexpr bool SST = !(FC1 && CPL >= 4);
  static constexpr int SROWB = K / 64;
  static constexpr int SRS = SROWB + 4;
  static constexpr int SCH = SROWB / 16;
  static constexpr int SCHUNKS = NM * ROWS * SCH;
  static constexpr int SCB = NM * ROWS * SRS;
  static_assert(!SST || SCHUNKS <= THREADS, "one 16-byte chunk of scales per thread");
};

// VQ2 codes one lane holds for one (group pair, matrix, row block): 16 code bytes (8 of
// each group once swapped) and, where the scales are not staged through LDS (RS), the
// two groups' fp16 scale bits.  Pairs start at an even group, so the two scales are one
// aligned dword.
template <bool RS>
struct MfPair {
  uint4 q;
  uint32_t s;  // scale bits: low half the first group, high half the second
};
template <>
struct MfPair<false> {
  uint4 q;
};

// The same for a group read alone.
template <bool RS>
struct MfOne {
  uint2 q;
  uint32_t s;
};
template <>
struct MfOne<false> {
  uint2 q;
};

// MXFP4 codes of one (group, matrix, row block): 16 bytes (32 weights, one E8M0 block).
struct MfMx {
  uint4 q;
  uint32_t e;
};

template <int CPL, bool FC1>
__global__ __launch_bounds__((MfGeom<CPL, FC1>::THREADS), 1) void fc_mfma_kernel(FcArgs a) {
  using G = MfGeom<CPL, FC1>;
  constexpr int MF_WAVES = G::W, MF_THREADS = G::THREADS;
  constexpr int K = G::K, NM = G::NM, NB = G::NB, ROWS = G::ROWS, NGQ = G::NGQ, KS = G::KS;
  constexpr int NPAIR = G::NPAIR, QS = G::QS, RED = G::RED, NBUF = G::NBUF;
  constexpr bool ODD = G::ODD;
  constexpr bool SST = G::SST;
  constexpr int SROWB = G::SROWB, SRS = G::SRS, SCH = G::SCH, SCHUNKS = G::SCHUNKS, SCB = G::SCB;
  using Pair = MfPair<!SST>;
  using One = MfOne<!SST>;
  // LDS, in one array so that the decode table starts at address 0: a lookup's address
  // is then the v_perm result itself (past 64 KB it would need an add per lookup, the
  // immediate offset of a ds_read being 16 bits).  Then the per-wave partial sums, and
  // the pair of each token row of the current and the next token group: the outputs'
  // rows, read from LDS rather than from global memory at the end of every tile (a load
  // there would wait for every older load, i.e. for the ring in flight).  Last (SST),
  // the VQ2 scales of the current and the next tile.
  constexpr int LDS_SC = TAB_BYTES + NBUF * RED * 4 + 2 * MF_MT * 4 * (FC1 ? 1 : 2);
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_SC + (SST ? 2 * SCB : 0)];
  uint2* const tab = reinterpret_cast<uint2*>(lds);
  float* const red = reinterpret_cast<float*>(lds + TAB_BYTES);
  int (*const s_pair)[MF_MT] = reinterpret_cast<int (*)[MF_MT]>(lds + TAB_BYTES + NBUF * RED * 4);
  // FC2: the routing weight of each token row, next to its pair
  float (*const s_w)[MF_MT] = reinterpret_cast<float (*)[MF_MT]>(lds + TAB_BYTES + NBUF * RED * 4 + 2 * MF_MT * 4);
  uint8_t* const sc_lds = lds + LDS_SC;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i16 = lane & 15, kq = lane >> 4;
  const int pq = ((kq & 1) << 1) | (kq >> 1);  // k-part of the group held by this lane
  const uint32_t laneoff = (uint32_t)(lane & 31) << 3;
  const int NROWS = FC1 ? a.I : a.H;
  const int RB = (NROWS + ROWS - 1) / ROWS;
  const int g0 = uni(wave) * NGQ;  // first scale group of this wave's part of K
  const int sl0 = g0 >> 3;         // its first 1024-column slice (FC1 factors)
  // Register slot gi of the wave's groups: slots 0 .. 2*NPAIR-1 are the pairs, starting
  // at the first even group; slot NGQ-1 (odd NGQ) is the group read alone, the first
  // group when g0 is odd, else the last.
  const int gpair = g0 + (g0 & 1);
  const int gone = (g0 & 1) ? g0 : g0 + NGQ - 1;
  auto gid = [&](int gi) __attribute__((always_inline)) -> int { return (ODD && gi == NGQ - 1) ? gone : gpair + gi; };

  const uint2 cbv = reinterpret_cast<const uint2*>(a.codebook)[tid & 127];
  // The kernel arguments span five scalar-cache lines: the activation and output
  // pointers', the MXFP4 offsets' and the grid size's are read here with the header.
  asm volatile("" ::"s"(FC1 ? a.x_h : (const uint16_t*)a.h_in), "s"(a.mx4.s_down), "s"(gridDim.x));
  // The workgroup's tiles: the worklist's split by cost when it was made for this grid
  // (read together with the header), else an equal share of the tile count.
  int pb = 0, pe = 0;
  if (a.part) { pb = a.part[blockIdx.x]; pe = a.part[blockIdx.x + 1]; }
  if (!ws_ok(a, FC1, MF_MT)) return;
  const int n_tiles = (int)a.hdr[FC1 ? HDR_GROUPS1 : HDR_GROUPS2] * RB;
  const bool split = a.part && a.hdr[FC1 ? HDR_PGRID1 : HDR_PGRID2] == gridDim.x;
  const int t_begin = split ? pb : (int)(((long)blockIdx.x * n_tiles) / gridDim.x);
  const int t_end = split ? min(pe, n_tiles) : (int)(((long)(blockIdx.x + 1) * n_tiles) / gridDim.x);
  if (t_begin >= t_end) return;

  // ---- activations of the current token group, in registers
  half8_t A[NGQ][4];                            // A fragments, group gi, step s
  float fw[4];                                  // factor of D row 4 kq + r (0 past the group)
  float4 A32[FC1 ? 1 : NGQ][8];                 // FC2: the next group's h, as loaded

  // Per-lane pair of A row i16 for group record r; padding rows repeat the last real one.
  struct Tok {
    int arow;
  };
  auto tok_load = [&](const RecS& r) __attribute__((always_inline)) -> Tok {
    Tok t;
    t.arow = a.pair_list[r.p0 + min(i16, r.mcount - 1)];
    return t;
  };
  // Issue the loads of a token group's activations (FC1: the staged fp16 x and its
  // slice factors; FC2: fp32 h), converted by convert_x / convert_h.
  // The token rows of the next group are loaded at the top of a tile and used after it:
  // arithmetic on them next to their load would wait there for every older load, i.e.
  // for the ring in flight.  This fence keeps their first use where it is written.
  auto tok_fence = [&](const Tok& t_in) __attribute__((always_inline)) -> Tok {
    Tok t;
    t.arow = opaque(t_in.arow);
    return t;
  };
  float hw = 0.f;  // FC2: routing weight of the pair of A row i16 (kept in LDS for the output)
  // FC1: slice factors of A row i16's token for the (at most two) 1024-column slices
  // the wave's groups touch
  float xs[2];
  auto act_load = [&](const Tok& t, const RecS& r) __attribute__((always_inline)) {
    (void)r;
    if (FC1) {
      const int tokA = t.arow / a.k;
      const uint16_t* xr = a.x_h + (size_t)tokA * K + 32 * pq;
#pragma unroll
      for (int gi = 0; gi < NGQ; ++gi)
#pragma unroll
        for (int s = 0; s < 4; ++s) A[gi][s] = *reinterpret_cast<const half8_t*>(xr + gid(gi) * 128 + 8 * s);
#pragma unroll
      for (int j = 0; j < 2; ++j) xs[j] = a.x_sc[(size_t)tokA * KS + min(sl0 + j, KS - 1)];
    } else {
      hw = a.pair_w[t.arow];
      const float* hr = a.h_in + (size_t)t.arow * K + 32 * pq;
#pragma unroll
      for (int gi = 0; gi < NGQ; ++gi)
#pragma unroll
        for (int i = 0; i < 8; ++i) A32[FC1 ? 0 : gi][i] = *reinterpret_cast<const float4*>(hr + gid(gi) * 128 + 4 * i);
    }
  };
  // D row 4 kq + r takes the factor f of A row 4 kq + r (0 past the group's tokens)
  auto row_factors = [&](float f, const RecS& r) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float v = __shfl(f, 4 * kq + q);
      fw[q] = 4 * kq + q < r.mcount ? v : 0.f;
    }
  };
  // FC1: the staged x has one power-of-two factor per (token, 1024-column slice), 0 for
  // an all-zero slice.  The wave's part takes the largest factor F of the slices it
  // touches, and the A fragments of a slice with factor f are multiplied by f / F (a
  // power of two, at most 1), exactly unless a result falls below fp16's normal range
  // with bits to lose: for bf16 x, values more than 2^32 below the largest of their
  // part.
  auto convert_x = [&](const RecS& r) __attribute__((always_inline)) {
    if (FC1) {
      const bool two = ((g0 + NGQ - 1) >> 3) > sl0;  // uniform: the part spans two slices
      const float F = two ? fmaxf(xs[0], xs[1]) : xs[0];
      const int eF = frexp_exponent(F);
      _Float16 rs[2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        rs[j] = xs[j] > 0.f ? (_Float16)ldexp2(1.0f, frexp_exponent(xs[j]) - eF) : (_Float16)0.f;
#pragma unroll
      for (int gi = 0; gi < NGQ; ++gi) {
        const int j = (gid(gi) >> 3) - sl0;  // uniform
        const _Float16 m = j == 0 ? rs[0] : rs[1];
        const half8_t mv = {m, m, m, m, m, m, m, m};
#pragma unroll
        for (int s = 0; s < 4; ++s) A[gi][s] = A[gi][s] * mv;
      }
      row_factors(F, r);
    }
  };
  // FC2: fp32 h -> fp16 A fragments with one power-of-two factor per (pair, wave part).
  auto convert_h = [&](const RecS& r) __attribute__((always_inline)) {
    if (!FC1) {
      float m = 0.f;
#pragma unroll
      for (int gi = 0; gi < NGQ; ++gi)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float4 u = A32[FC1 ? 0 : gi][i];
          m = fmaxf(m, fmaxf(fmaxf(fabsf(u.x), fabsf(u.y)), fmaxf(fabsf(u.z), fabsf(u.w))));
        }
      // the largest |h| of the row's part (the four lanes of the row hold a quarter
      // each), scaled below 2^15
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      int ex = 0;
      if (m > 0.f && m < INFINITY) ex = frexp_exponent(m) - 15;
      row_factors(ldexp2(1.0f, ex), r);
#pragma unroll
      for (int gi = 0; gi < NGQ; ++gi)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float4 u = A32[FC1 ? 0 : gi][2 * s], w = A32[FC1 ? 0 : gi][2 * s + 1];
          A[gi][s] = half8_t{(_Float16)ldexp2(u.x, -ex), (_Float16)ldexp2(u.y, -ex), (_Float16)ldexp2(u.z, -ex),
                             (_Float16)ldexp2(u.w, -ex), (_Float16)ldexp2(w.x, -ex), (_Float16)ldexp2(w.y, -ex),
                             (_Float16)ldexp2(w.z, -ex), (_Float16)ldexp2(w.w, -ex)};
        }
    }
  };

  // Addresses of one tile's codes in the ring's shape: uniform matrix bases, 32-bit
  // per-lane row offsets per row block, and per-slot immediates.  Both formats put slot
  // pi's 16 bytes per lane 64 bytes further along the row and its scale dword 4 bytes
  // further: VQ2 pair slot pi is groups gpair + 2pi, gpair + 2pi + 1 (16 bytes at the
  // lane's quarter of the pair's 64); an MXFP4 slot pi is group gpair + pi (16 bytes of
  // the lane's k-part p(q), and the dword of the group's four E8M0 bytes).
  struct MfAddr {
    const uint8_t* qb[NM];
    const uint8_t* sb[NM];
    uint32_t qo[NB], so[NB];  // per row block: slot 0's code and scale offsets
    uint32_t dq0, ds0;        // subtracted: back to the row start (lane part of the codes)
    uint32_t dq1, ds1;        // added for the lone group (wrapping 32-bit deltas)
  };
  // VQ2 lone group, relative to slot 0's offsets: (gone*32 + pq*8) - (gpair*32 + kq*16)
  const uint32_t lone_dq = (uint32_t)(gone * 32 + pq * 8) - (uint32_t)(gpair * 32 + kq * 16);
  const uint32_t lone_ds = (uint32_t)(gone * 2) - (uint32_t)(gpair * 2);
  auto vq_addr = [&](const RecS& r, int rb) __attribute__((always_inline)) -> MfAddr {
    MfAddr d;
    const bool mx = r.fmt == MOE_VQ_FMT_MXFP4;
    const SlotLayout& L = mx ? a.mx4 : a.vq2;
    const uint8_t* slot = a.pool + r.slot_off;
    d.qb[0] = slot + (FC1 ? L.q_gate : L.q_down);
    d.sb[0] = slot + (FC1 ? L.s_gate : L.s_down);
    if (NM > 1) { d.qb[NM - 1] = slot + L.q_up; d.sb[NM - 1] = slot + L.s_up; }
    const uint32_t qrow = mx ? (uint32_t)(K / 2) : (uint32_t)(K / 4);
    const uint32_t srow = mx ? (uint32_t)(K / 32) : (uint32_t)(K / 64);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      // rows past the end (ragged shapes only) re-read the last row; the epilogue drops them
      const uint32_t n = (uint32_t)min(rb * ROWS + nb * 16 + i16, NROWS - 1);
      d.qo[nb] = n * qrow;
      d.so[nb] = n * srow;
    }
    const uint32_t lq = mx ? (uint32_t)(pq * 16) : (uint32_t)(kq * 16);   // per lane
    const uint32_t uq0 = mx ? (uint32_t)(gpair * 64) : (uint32_t)(gpair * 32);
    const uint32_t us0 = mx ? (uint32_t)(gpair * 4) : (uint32_t)(gpair * 2);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      d.qo[nb] += lq + uq0;
      d.so[nb] += us0;
    }
    d.dq0 = uq0;  // (MXFP4: the row start plus the lane's k-part offset is qo - dq0)
    d.ds0 = us0;
    // The lone delta is relative to the VQ2 lane part (kq*16), which an MXFP4 d does not
    // hold (pq*16): there it could reach below the row start and wrap.  An MXFP4 tile
    // never reads its lone slot, so that load goes to the lane's row start instead.
    d.dq1 = mx ? 0u - uq0 : lone_dq;
    d.ds1 = mx ? 0u - us0 : lone_ds;
    return d;
  };
  auto load_pair = [&](const MfAddr& d, int pi, int m, int nb) __attribute__((always_inline)) -> Pair {
    Pair c;
    c.q = *reinterpret_cast<const uint4*>(d.qb[m] + d.qo[nb] + pi * 64);
    if constexpr (!SST) c.s = *reinterpret_cast<const uint32_t*>(d.sb[m] + d.so[nb] + pi * 4);
    return c;
  };
  auto load_one = [&](const MfAddr& d, int m, int nb) __attribute__((always_inline)) -> One {
    One c;
    // (the sums wrap in 32 bits: the lone group can lie before slot 0; the true sum is
    // never negative)
    c.q = *reinterpret_cast<const uint2*>(d.qb[m] + (uint32_t)(d.qo[nb] + d.dq1));
    if constexpr (!SST) c.s = *reinterpret_cast<const uint16_t*>(d.sb[m] + (uint32_t)(d.so[nb] + d.ds1));
    return c;
  };

  // SST: thread tid's 16-byte chunk of a tile's scales is loaded at the start of the
  // previous tile (before its ring refills, so that waiting for it never waits for
  // them) and written to LDS before that tile's closing barrier.  Buffer sbuf holds the
  // current tile's scales, sbuf ^ 1 the next tile's.
  int sbuf = 0;
  const bool sc_thr = tid < SCHUNKS;
  const int sc_m = tid / (ROWS * SCH), sc_r = (tid / SCH) % ROWS, sc_j = tid % SCH;
  const uint32_t sc_wr = (uint32_t)((sc_m * ROWS + sc_r) * SRS + 16 * sc_j);
  const uint32_t sc_rd = (uint32_t)(i16 * SRS + 2 * gpair);  // the lane's row, first pair
  uint4 scv = make_uint4(0u, 0u, 0u, 0u);
  auto sc_load = [&](const RecS& r, int rb) __attribute__((always_inline)) {
    if (sc_thr) {
      const uint8_t* slot = a.pool + r.slot_off;
      const uint8_t* sbm = slot + (sc_m == 0 ? (FC1 ? a.vq2.s_gate : a.vq2.s_down) : a.vq2.s_up);
      const uint32_t n = (uint32_t)min(rb * ROWS + sc_r, NROWS - 1);
      scv = *reinterpret_cast<const uint4*>(sbm + n * (uint32_t)SROWB + 16 * sc_j);
    }
  };
  auto sc_store = [&](int b) __attribute__((always_inline)) {
    if (sc_thr) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(sc_lds + b * SCB + sc_wr);
      dst[0] = scv.x;
      dst[1] = scv.y;
      dst[2] = scv.z;
      dst[3] = scv.w;
    }
  };
  // the two scales of pair slot pi (row block nb of matrix m), and the lone group's
  auto sc_pair = [&](int m, int nb, int pi) __attribute__((always_inline)) -> uint32_t {
    return *reinterpret_cast<const uint32_t*>(sc_lds + sbuf * SCB + (m * ROWS + nb * 16) * SRS + sc_rd + 4 * pi);
  };
  auto sc_lone = [&](int m, int nb) __attribute__((always_inline)) -> uint32_t {
    return *reinterpret_cast<const uint16_t*>(sc_lds + sbuf * SCB + (m * ROWS + nb * 16) * SRS + sc_rd + 2 * (gone - gpair));
  };

  f32x4_t acc[NM][NB];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[m][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };

  // 8 code bytes of one group (this lane's k-part) -> its 4 B fragments
  auto b_frags = [&](uint32_t w0, uint32_t w1, half8_t (&bfr)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t wd = s < 2 ? w0 : w1;
      const uint2 e0 = tab_lookup(tab, tab_addr_sel(wd, laneoff, (2 * s) & 3));
      const uint2 e1 = tab_lookup(tab, tab_addr_sel(wd, laneoff, (2 * s + 1) & 3));
      bfr[s] = __builtin_bit_cast(half8_t, make_uint4(e0.x, e0.y, e1.x, e1.y));
    }
  };
  // (the activation factors are one per D row for the wave's whole part of K: they
  // multiply the tile's sums once, after its last group)
  auto group_mma = [&](int gi, const half8_t (&bfr)[4], float sc, f32x4_t& ac) __attribute__((always_inline)) {
    f32x4_t tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) tmp = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[gi][s], bfr[s], tmp, 0, 0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) ac[q] = fmaf(sc, tmp[q], ac[q]);
  };

  // VQ2 tile: consume the ring, refilling each slot with the next tile's codes.  Slot j
  // is (pair, matrix, row block) for j < NPS, then (matrix, row block) of the lone
  // group; unit u is one scale group of a slot (two per pair slot).  Software pipeline:
  // the lookups of unit u + 1 are issued before the matrix ops of unit u, so the LDS
  // latency hides behind them.  The refill is issued for every slot; without a next
  // VQ2 tile it re-reads this tile's codes (cache hits), which keeps the loop free of
  // branches.
  Pair ringP[NPAIR > 0 ? NPAIR : 1][NM][NB];
  One ringS[ODD ? NM : 1][ODD ? NB : 1];
  constexpr int NPS = NPAIR * NM * NB;                // pair slots
  constexpr int NU = 2 * NPS + (ODD ? NM * NB : 0);   // units
  struct UDec {
    half8_t b[4];
    float sc;
  };
  uint32_t pw2, pw3, ps;  // second group of the pair slot being consumed (words, scale bits)
  auto decode = [&](int u, const MfAddr& dn) __attribute__((always_inline)) -> UDec {
    UDec d;
    if (u < 2 * NPS) {
      const int j = u >> 1;
      const int pi = j / (NM * NB), m = (j / NB) % NM, nb = j % NB;
      if ((u & 1) == 0) {
        // the slot is consumed (swap, scales) before its refill is issued, so the refill
        // can land in the same registers
        const Pair c = ringP[pi][m][nb];
        const auto lo = __builtin_amdgcn_permlane32_swap(reg_copy(c.q.x), reg_copy(c.q.z), false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap(reg_copy(c.q.y), reg_copy(c.q.w), false, false);
        pw2 = lo[1];
        pw3 = hi[1];
        uint32_t cs;
        if constexpr (SST) cs = sc_pair(m, nb, pi);
        else cs = reg_copy(c.s);
        ps = cs >> 16;
        d.sc = f16_bits_to_f32(cs & 0xFFFFu);
        ringP[pi][m][nb] = load_pair(dn, pi, m, nb);
        b_frags(lo[0], hi[0], d.b);
      } else {
        d.sc = f16_bits_to_f32(ps);
        b_frags(pw2, pw3, d.b);
      }
    } else {
      const int m = ((u - 2 * NPS) / NB) % NM, nb = (u - 2 * NPS) % NB;
      const One c = ringS[ODD ? m : 0][ODD ? nb : 0];
      const uint32_t c0 = reg_copy(c.q.x), c1 = reg_copy(c.q.y);
      if constexpr (SST) d.sc = f16_bits_to_f32(sc_lone(m, nb));
      else d.sc = f16_bits_to_f32(reg_copy(c.s));
      ringS[ODD ? m : 0][ODD ? nb : 0] = load_one(dn, m, nb);
      b_frags(c0, c1, d.b);
    }
    return d;
  };
  auto unit_mma = [&](int u, const UDec& d) __attribute__((always_inline)) {
    if (u < 2 * NPS) {
      const int j = u >> 1;
      const int pi = j / (NM * NB), m = (j / NB) % NM, nb = j % NB;
      group_mma(2 * pi + (u & 1), d.b, d.sc, acc[m][nb]);
    } else {
      const int m = ((u - 2 * NPS) / NB) % NM, nb = (u - 2 * NPS) % NB;
      group_mma(NGQ - 1, d.b, d.sc, acc[m][nb]);
    }
  };
  auto compute_vq = [&](bool refill, const RecS& rn, int rbn, const RecS& rcur, int rbc)
                        __attribute__((always_inline)) {
    const MfAddr dn = refill ? vq_addr(rn, rbn) : vq_addr(rcur, rbc);
    // (FC1 at K = 7168 has the 17 registers this takes: B32 FC1 201.7 -> 199.1 us)
    UDec cur = decode(0, dn);
    static_for<0, NU>([&](auto U_) __attribute__((always_inline)) {
      constexpr int u = decltype(U_)::value;
      UDec nxt;
      if (u + 1 < NU) nxt = decode(u + 1, dn);
      unit_mma(u, cur);
      if (u + 1 < NU) cur = nxt;
    });
  };

  // MXFP4 tile (not in the ring): the groups of the wave's part of K load in passes of up
  // to MXG groups.  Each lane reads the 32 weights of its k-part p(q) of a group.
  // e: the four E8M0 bytes of this row's group (one dword); the lane's block is byte pq
  auto mx_unit = [&](int gi, const uint4& q, uint32_t e, int m, int nb) __attribute__((always_inline)) {
    // e_max over the four blocks of this row's group, which the lanes i16, i16 + 16, + 32
    // and + 48 hold: all four bytes are in every lane's dword
    const int em = (int)max(max(e & 0xFFu, (e >> 8) & 0xFFu), max((e >> 16) & 0xFFu, e >> 24));
    const float es = ldexp2(1.0f, (int)((e >> (8 * pq)) & 0xFFu) - em);  // 2^(e - e_max), in (0, 1]
    half8_t bfr[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t wd = s == 0 ? q.x : s == 1 ? q.y : s == 2 ? q.z : q.w;
      const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, es, 0);
      const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, es, 1);
      const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, es, 2);
      const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, es, 3);
      bfr[s] = half8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    }
    group_mma(gi, bfr, e8m0_to_f32((uint32_t)em), acc[m][nb]);
  };
  auto compute_mx = [&](const RecS& r, int rb) __attribute__((always_inline)) {
    const MfAddr d = vq_addr(r, rb);
    // Groups load in passes of NH.  Where the register budget holds two or more groups,
    // and in FC2, the passes are one group each in two buffers, and the loads of pass
    // h + 1 are issued before pass h is decoded, so that they arrive while it decodes
    // (buffers of two groups each spill at K = 7168).
    constexpr bool DB = (G::MXG >= 2 || !FC1) && NGQ >= 2;
    constexpr int NH = DB ? 1 : G::MXG;
    constexpr int NPASS = (NGQ + NH - 1) / NH;
    MfMx mx[DB ? 2 : 1][NH][NM][NB];
    auto mx_load = [&](int h) __attribute__((always_inline)) {
      const int b = DB ? (h & 1) : 0;
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        const int gi = h * NH + j;
        if (gi < NGQ)
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              const uint32_t g = (uint32_t)gid(gi);
              mx[b][j][m][nb].q = *reinterpret_cast<const uint4*>(d.qb[m] + (uint32_t)(d.qo[nb] - d.dq0 + g * 64));
              mx[b][j][m][nb].e = *reinterpret_cast<const uint32_t*>(d.sb[m] + (uint32_t)(d.so[nb] - d.ds0 + g * 4));
            }
      }
    };
    if (DB) mx_load(0);
    static_for<0, NPASS>([&](auto H_) __attribute__((always_inline)) {
      constexpr int h = decltype(H_)::value;
      if (!DB) mx_load(h);
      else if (h + 1 < NPASS) mx_load(h + 1);
      const int b = DB ? (h & 1) : 0;
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        const int gi = h * NH + j;
        if (gi >= NGQ) break;
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) mx_unit(gi, mx[b][j][m][nb].q, mx[b][j][m][nb].e, m, nb);
      }
    });
  };

  // End of a tile: the waves' partial sums meet in LDS, then the outputs.  LDS
  // layout [wave][matrix][token][row] with a padded token stride.
  // gb: the current group's half of s_pair; the next group's pairs (arow_next, lanes 0-15
  // of wave 0) go to the other half after the barrier, when every wave is past the
  // previous tile's reads of it.
  auto finish = [&](const RecS& r, int rb, int buf, int gb, bool wr_next, int arow_next) __attribute__((always_inline)) {
    float* R = red + (NBUF > 1 ? buf * RED : 0);
    if (NBUF == 1) __syncthreads();  // the previous tile's sums have been read
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (4 * kq + q < r.mcount) R[((wave * NM + m) * MF_MT + 4 * kq + q) * QS + nb * 16 + i16] = acc[m][nb][q];
    __syncthreads();
    if (wr_next && wave == 0 && kq == 0) {
      s_pair[gb ^ 1][i16] = arow_next;
      if (!FC1) s_w[gb ^ 1][i16] = hw;  // (act_load has loaded the next group's weights)
    }
    const int nout = ROWS * r.mcount;
    for (int o = tid; o < nout; o += MF_THREADS) {
      const int q = o / ROWS, ri = o % ROWS;
      const int n = rb * ROWS + ri;
      if (n < NROWS) {
        float v[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          float sum = R[(m * MF_MT + q) * QS + ri];
#pragma unroll
          for (int w = 1; w < MF_WAVES; ++w) sum += R[((w * NM + m) * MF_MT + q) * QS + ri];
          v[m] = sum;
        }
        const int p = s_pair[gb][q];
        if (FC1) a.out[(size_t)p * a.I + n] = swiglu(v[0], v[NM - 1], a.lim);
        else a.out[(size_t)p * a.H + n] = v[0] * s_w[gb][q];
      }
    }
  };

  // Loads of a whole ring for tile (r, rb), in the order the refills use; the
  // scheduling barriers keep that order, so that the count of loads in flight after
  // each slot is the same whichever way the loop is entered.
  auto ring_load = [&](const RecS& r, int rb) __attribute__((always_inline)) {
    const MfAddr d = vq_addr(r, rb);
#pragma unroll
    for (int pi = 0; pi < NPAIR; ++pi)
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          ringP[pi][m][nb] = load_pair(d, pi, m, nb);
          __builtin_amdgcn_sched_barrier(0);
        }
    if (ODD) {
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          ringS[ODD ? m : 0][ODD ? nb : 0] = load_one(d, m, nb);
          __builtin_amdgcn_sched_barrier(0);
        }
    }
  };

  auto ring_clear = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int pi = 0; pi < (NPAIR > 0 ? NPAIR : 1); ++pi)
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) ringP[pi][m][nb] = Pair{};
#pragma unroll
    for (int m = 0; m < (ODD ? NM : 1); ++m)
#pragma unroll
      for (int nb = 0; nb < (ODD ? NB : 1); ++nb) ringS[m][nb] = One{};
  };

  // A workgroup's tiles run group by group (row blocks of one token group, then the
  // next group's), so a record is needed once per group change: the current group's and
  // the next one's are held, and the record after them is read when the group changes.
  // Records are read-only for the whole launch and read through the constant address
  // space (scalar loads): a vector load's value waits for every older vector load (they
  // complete in order), here the whole ring in flight.  A scalar load in flight holds up
  // every LDS wait of the wave (they share a counter), so it is issued only where the
  // group change drains the loads anyway, never once per tile.
  typedef const int __attribute__((address_space(4))) cint_t;
  auto load_rec_c = [&](int g) __attribute__((always_inline)) -> RecS {
    cint_t* w = reinterpret_cast<cint_t*>(reinterpret_cast<uintptr_t>(a.rec + g));
    RecS r{};
    r.slot_off = ((uint64_t)(uint32_t)w[1] << 32) | (uint32_t)w[0];
    r.p0 = w[2];
    r.mcount = w[3];
    r.fmt = (uint32_t)w[4];
    return r;
  };

  auto sel_rec = [&](bool c, const RecS& x, const RecS& y) __attribute__((always_inline)) -> RecS {
    RecS r{};
    r.slot_off = c ? x.slot_off : y.slot_off;
    r.p0 = c ? x.p0 : y.p0;
    r.mcount = c ? x.mcount : y.mcount;
    r.fmt = c ? x.fmt : y.fmt;
    return r;
  };

  // ---- prologue
  int t = t_begin;
  int g = t / RB, rb = t - g * RB;      // the tile's token group and row block
  const int g_last = (t_end - 1) / RB;  // the last group of the workgroup's tiles
  const RecRaw raw_c = load_rec_raw(a.rec, g);
  const RecRaw raw_n = load_rec_raw(a.rec, min(g + 1, g_last));
  RecS rc = rec_from_raw(raw_c);
  RecS rg1 = rec_from_raw(raw_n);  // the next group (the last one again at the end)
  const Tok t0 = tok_load(rc);
  act_load(t0, rc);
  if (rc.fmt == MOE_VQ_FMT_VQ2) {
    if (SST) sc_load(rc, rb);
    ring_load(rc, rb);
  }
  // (after the ring's loads: the weight's load is then waited for with the ring in flight)
  if (wave == 0 && kq == 0) {
    s_pair[0][i16] = t0.arow;
    if (!FC1) s_w[0][i16] = hw;
  }
  bool ring_ok = rc.fmt == MOE_VQ_FMT_VQ2;  // the ring holds this tile's codes
  if (tid < 256) write_table_entry(tab, cbv, tid);  // (every block has >= 256 threads)
  if (SST && rc.fmt == MOE_VQ_FMT_VQ2) sc_store(0);
  __syncthreads();

  if (FC1) convert_x(rc);
  else convert_h(rc);
  int buf = 0, gb = 0;
  for (;;) {
    const bool more = t + 1 < t_end;
    const bool next_group = more && rb + 1 == RB;
    const int rbn = next_group ? 0 : rb + 1;  // the next tile's row block
    const RecS rn = sel_rec(next_group, rg1, rc);
    const bool next_vq = more && rn.fmt == MOE_VQ_FMT_VQ2;  // the ring takes the next tile's codes
    if (SST && next_vq) sc_load(rn, rbn);  // (before this tile's refills)
    Tok tk;  // (no initial value: writing one would wait for the last group's row loads)
    if (next_group) tk = tok_load(rn);
    zero_acc();
    // The ring is defined in this branch only (a second definition elsewhere in the loop
    // makes the compiler keep it in other registers and copy it back at the loop's back
    // edge, waiting for every load in flight).  After a tile of another format it is
    // stale, and the VQ2 tile loads its own codes first.
    if (rc.fmt == MOE_VQ_FMT_VQ2) {
      if (!ring_ok) ring_load(rc, rb);
      compute_vq(next_vq, rn, rbn, rc, rb);  // refills the ring with the next tile's codes
    } else if (rc.fmt == MOE_VQ_FMT_MXFP4) {
      compute_mx(rc, rb);
    }
    // (an absent expert keeps zeros; the worklist has recorded MOE_VQ_ENOTRESIDENT)
    // The activation factors of this token group, before a group change replaces them.
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[m][nb][q] *= fw[q];
    ring_ok = rc.fmt == MOE_VQ_FMT_VQ2 && next_vq;
    RecS rg2 = rg1;
    if (next_group) {
      rg2 = load_rec_c(min(g + 2, g_last));  // the group after the next one
      tk = tok_fence(tk);
      act_load(tk, rn);  // this tile was the last use of the activations
      // (waits for the loads here: fp32 h and bf16 x are not kept across tiles)
      if (FC1) convert_x(rn);
      else convert_h(rn);
      // The activations and the record are complete before the next tile, on this
      // path: otherwise the tile body would carry a wait for them that, on every other
      // tile, waits for the ring in flight too.  (s_waitcnt vmcnt(0) lgkmcnt(0).)
      __builtin_amdgcn_s_waitcnt(0x0070);
    }
    if (SST && next_vq) sc_store(sbuf ^ 1);  // (read after finish's barrier)
    finish(rc, rb, buf, gb, next_group, tk.arow);
    if (!more) break;
    sbuf ^= 1;
    if (next_group) {
      gb ^= 1;
      g += 1;
      rc = rg1;
      rg1 = rg2;
    }
    rb = rbn;
    t += 1;
    buf ^= NBUF - 1;
  }
}

// ---------------------------------------------------------------------------------------
// Host launcher
// ---------------------------------------------------------------------------------------

template <bool FC1>
hipError_t launch_mfma(const FcArgs& a, int K, int MT, int max_groups, int n_cu, hipStream_t st, bool* done) {
  *done = false;
  if (MT != MF_MT || !mf_supported(K, FC1)) return hipSuccess;
  const int cpl = K / 1024;
  const int nrows = FC1 ? a.I : a.H;
  // (one workgroup per CU: a workgroup fills the CU's registers)
#define MVQ_MFMA_CASE(C)                                                                     \
  if (cpl == C) {                                                                            \
    const int grid = mf_grid(n_cu, max_groups, nrows, MfGeom<C, FC1>::ROWS);                 \
    *done = true;                                                                            \
    if (grid <= 0) return hipSuccess;                                                        \
    FcArgs b = a;                                                                            \
    if (grid > MAX_PART) b.part = nullptr; /* (the split table's size) */                    \
    launch_fc_kernel(fc_mfma_kernel<C, FC1>, (unsigned)grid, MfGeom<C, FC1>::THREADS, 0, st, b); \
    return hipGetLastError();                                                                \
  }
  MVQ_MFMA_CASE(1) MVQ_MFMA_CASE(2)
  if constexpr (FC1) { MVQ_MFMA_CASE(7) }
#undef MVQ_MFMA_CASE
  return hipErrorInvalidValue;
}

template hipError_t launch_mfma<true>(const FcArgs&, int, int, int, int, hipStream_t, bool*);
template hipError_t launch_mfma<false>(const FcArgs&, int, int, int, int, hipStream_t, bool*);

}  // namespace mvq
