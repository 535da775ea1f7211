// FC2 (down) with the weighted combine, for a step of one token: y = sum_i w_i W_d,i h_i.
//
// Sources: FC2 per routed expert decoded from the 2-bit codes, then the experts' outputs
// added with the routing weights (Tandem-vLLM 0.2.0 announcement, "How it works";
// vLLM-Moet README, "2-bit experts on vLLM v0.24.0"); no padding rows written back
// (vLLM-Moet README, "What we changed against official vLLM", row "MoE at decode").
//
// With one token the k routed experts all write the same output rows.  A workgroup here
// owns a block of 28 output rows and has one wave per routed expert.  Lane (c, r) of a
// wave takes the 64-column chunk c of every r-th row of the block: it holds that chunk
// of its pair's h in registers (fp16, with the power-of-two factor of its 1024-column
// slice, as the other FC2 kernels scale h), issues the code loads of all its rows up
// front, and decodes them against the same registers, so h is read once per lane and
// never from LDS.  Each row's partial products are summed over the chunk lanes with
// DPP and then over the experts, in the worklist's expert order, through a small LDS
// array; y is written directly: no per-pair outputs and no separate combine launch.
// H = 7168 is 256 workgroups, one per CU.
#include "fc_common.h"

namespace mvq {

constexpr int F2S_KMAX = 8;                 // routed experts per token this kernel takes
constexpr int F2S_THREADS = 64 * F2S_KMAX;  // one wave per routed expert
constexpr int F2S_ROWS = 28;                // output rows per workgroup
constexpr int F2S_AHEAD = 3;                // rows of codes in flight ahead of the decode

template <int CPL>
__global__ __launch_bounds__(F2S_THREADS, 1) void fc2_single_kernel(FcArgs a) {
  constexpr int K = 1024 * CPL;
  constexpr int NCH = K / 64;           // 64-column chunks per row: lanes per row
  constexpr int RGW = 64 / NCH;         // row groups per wave
  constexpr int RPL = F2S_ROWS / RGW;   // rows per lane
  constexpr int MXP = RPL > 7 ? 7 : RPL;  // MXFP4 rows loaded per pass
  static_assert(F2S_ROWS % RGW == 0, "rows per workgroup");
  __shared__ uint2 tab[256 * TAB_COPIES];
  __shared__ float red[F2S_KMAX][F2S_ROWS];

  const int tid = threadIdx.x, g = tid >> 6, lane = tid & 63;
  const int c = lane % NCH, rgi = lane / NCH;
  const uint32_t laneoff = (uint32_t)(lane & 31) << 3;
  const int row0 = blockIdx.x * F2S_ROWS;

  const uint2 cbv = reinterpret_cast<const uint2*>(a.codebook)[tid & 127];
  // this wave's record, read together with the header rather than after it (record
  // min(g, max_groups - 1) lies in the record array whatever the header says); nothing
  // read from it is used before the header check has passed
  const int4* rp = reinterpret_cast<const int4*>(a.rec + (g < a.max_groups ? g : a.max_groups - 1));
  const int4 w0 = rp[0], w1 = rp[1];
  // The kernel arguments span five scalar-cache lines: the ones holding h, the routing
  // weights and the down matrices' offsets are read here, with the header, rather than
  // first where they are used, behind a miss.
  asm volatile("" ::"s"(a.h_in), "s"(a.vq2.s_down));
  if (!ws_ok(a, false, 1)) return;
  const int G = (int)a.hdr[HDR_GROUPS2];  // one group per routed pair
  if (G > F2S_KMAX) {                     // (the launcher takes this kernel only for k <= 8)
    if (blockIdx.x == 0 && tid == 0) a.hdr[HDR_STATUS] = MOE_VQ_EINVAL;
    return;
  }
  const bool live = g < G;
  const uint64_t slot_off = ((uint64_t)(uint32_t)uni(w0.y) << 32) | (uint32_t)uni(w0.x);
  const uint32_t fmt = live ? (uint32_t)uni(w1.x) : (uint32_t)MOE_VQ_FMT_ABSENT;
  const int p = live ? uni(w1.z) : 0;  // the pair (only pair[0] of a one-token group)
  const uint8_t* slot = a.pool + slot_off;

  // ---- this lane's chunk of h, then the first rows' code loads.  At K = 2048 lanes c and
  // c + 32 take the same chunk: each loads one half of it, and the halves are exchanged
  // after the fp16 conversion (h is read once per workgroup, not twice).
  constexpr int HV = NCH == 32 ? 8 : 16;  // float4 of h this lane loads
  float4 hv[HV];
  if (live) {
    const int half = NCH == 32 ? lane >> 5 : 0;
    const float4* src = reinterpret_cast<const float4*>(a.h_in + (size_t)p * K + c * 64 + half * 32);
#pragma unroll
    for (int i = 0; i < HV; ++i) hv[i] = src[i];
  }
  // Only the first F2S_AHEAD rows' codes are issued before the barrier: issuing them all
  // would hold the wave until the memory pipeline had taken every load, so that the
  // decode could start only once nearly all the data had arrived.  The other rows are
  // issued in the decode loop, each F2S_AHEAD rows ahead of the row being decoded.
  uint4 q[RPL];
  uint32_t s[RPL];
  const uint8_t* qb = slot + a.vq2.q_down + c * 16;
  const uint8_t* sb = slot + a.vq2.s_down + (c >> 1) * 2;
  auto load_row = [&](int i) __attribute__((always_inline)) {
    // rows past the end re-read the last row; their sums are never written
    const int n = min(row0 + rgi + RGW * i, a.H - 1);
    q[i] = *reinterpret_cast<const uint4*>(qb + (size_t)n * (K / 4));
    s[i] = *reinterpret_cast<const uint16_t*>(sb + (size_t)n * (K / 64));
  };
  if (fmt == MOE_VQ_FMT_VQ2) {
#pragma unroll
    for (int i = 0; i < F2S_AHEAD && i < RPL; ++i) load_row(i);
  }

  // ---- h to fp16 with one power-of-two factor per 1024-column slice (16 chunk lanes)
  uint32_t xw[32];
  float xsc = 1.f;
  if (live) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < HV; ++i)
      m = fmaxf(m, fmaxf(fmaxf(fabsf(hv[i].x), fabsf(hv[i].y)), fmaxf(fabsf(hv[i].z), fabsf(hv[i].w))));
    m = fmaxf(m, dpp_f32<dpp::QUAD_XOR1>(m));
    m = fmaxf(m, dpp_f32<dpp::QUAD_XOR2>(m));
    m = fmaxf(m, dpp_f32<dpp::ROW_HALF_MIRROR>(m));
    m = fmaxf(m, dpp_f32<dpp::ROW_MIRROR>(m));
    if constexpr (NCH == 32) {
      // v_permlane32_swap of a value with itself gives {lanes 0..31's value, lanes
      // 32..63's value} in every lane pair (l, l + 32): here the two halves' maxima
      const auto mm = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, m),
                                                       __builtin_bit_cast(uint32_t, m), false, false);
      m = fmaxf(__builtin_bit_cast(float, (uint32_t)mm[0]), __builtin_bit_cast(float, (uint32_t)mm[1]));
    }
    int ex = 0;
    if (m > 0.f && m < INFINITY) ex = frexp_exponent(m) - 15;
    uint32_t own[2 * HV];
#pragma unroll
    for (int i = 0; i < HV; ++i) {
      own[2 * i] = pack_half2(ldexp2(hv[i].x, -ex), ldexp2(hv[i].y, -ex));
      own[2 * i + 1] = pack_half2(ldexp2(hv[i].z, -ex), ldexp2(hv[i].w, -ex));
    }
    if constexpr (NCH == 32) {
#pragma unroll
      for (int d = 0; d < 16; ++d) {
        const auto r = __builtin_amdgcn_permlane32_swap(own[d], own[d], false, false);
        xw[d] = r[0];       // first half of the chunk (lane c's)
        xw[16 + d] = r[1];  // second half (lane c + 32's)
      }
    } else {
#pragma unroll
      for (int d = 0; d < 32; ++d) xw[d] = own[d];
    }
    xsc = ldexp2(1.0f, ex);
  }
  if (tid < 256) write_table_entry(tab, cbv, tid);
  __syncthreads();

  // ---- this lane's rows against its chunk
  const float w = live ? a.pair_w[p] : 0.f;
  float acc[RPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i) acc[i] = 0.f;
  if (fmt == MOE_VQ_FMT_VQ2) {
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      if (i + F2S_AHEAD < RPL) load_row(i + F2S_AHEAD);
      float pr = 0.f;
#pragma unroll
      for (int d = 0; d < 4; ++d) pr = vq2_dword_dot(tab, dword_of(q[i], d), laneoff, xw + 8 * d, pr);
      acc[i] = (w * f16_bits_to_f32(s[i]) * xsc) * pr;
    }
  } else if (fmt == MOE_VQ_FMT_MXFP4) {
    // two 32-weight blocks per row and lane, MXP rows per pass
    const uint8_t* qb = slot + a.mx4.q_down + c * 32;
    const uint8_t* eb = slot + a.mx4.s_down + c * 2;
#pragma unroll
    for (int i0 = 0; i0 < RPL; i0 += MXP) {
      uint4 qm[MXP][2];
      uint32_t em[MXP];
#pragma unroll
      for (int ii = 0; ii < MXP; ++ii) {
        const int n = min(row0 + rgi + RGW * (i0 + ii), a.H - 1);
        if (i0 + ii < RPL) {
          qm[ii][0] = *reinterpret_cast<const uint4*>(qb + (size_t)n * (K / 2));
          qm[ii][1] = *reinterpret_cast<const uint4*>(qb + (size_t)n * (K / 2) + 16);
          em[ii] = *reinterpret_cast<const uint16_t*>(eb + (size_t)n * (K / 32));
        }
      }
#pragma unroll
      for (int ii = 0; ii < MXP; ++ii) {
        if (i0 + ii < RPL) {
          const float p0 = mx4_chunk_dot(qm[ii][0], xw);
          const float p1 = mx4_chunk_dot(qm[ii][1], xw + 16);
          float v = (w * e8m0_to_f32(em[ii] & 0xFF) * xsc) * p0;
          acc[i0 + ii] = fmaf(w * e8m0_to_f32(em[ii] >> 8) * xsc, p1, v);
        }
      }
    }
  }
  // (an absent expert adds nothing; the worklist has recorded MOE_VQ_ENOTRESIDENT)

  // ---- each row: sum over its chunk lanes, then over the experts in order
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    float v = group_sum<16>(acc[i]);
    if (NCH == 32) v += __shfl_xor(v, 16);
    if (c == 0) red[g][rgi + RGW * i] = v;
  }
  __syncthreads();
  if (tid < F2S_ROWS && row0 + tid < a.H) {
    float y = a.accumulate ? a.y[row0 + tid] : 0.f;  // (the shared expert adds to y)
#pragma unroll
    for (int gg = 0; gg < F2S_KMAX; ++gg)
      if (gg < G) y += red[gg][tid];
    a.y[row0 + tid] = y;
  }
}

// y for a one-token step straight from the experts (K = 1024 or 2048, k <= 8); *done
// says whether it took the call.
hipError_t launch_fc2_single(const FcArgs& a, int MT, hipStream_t st, bool* done) {
  *done = false;
  if (a.T != 1 || MT != 1 || a.k > F2S_KMAX || (a.I != 1024 && a.I != 2048)) return hipSuccess;
  const int grid = (a.H + F2S_ROWS - 1) / F2S_ROWS;
  *done = true;
  if (a.I == 1024) launch_fc_kernel(fc2_single_kernel<1>, (unsigned)grid, F2S_THREADS, 0, st, a);
  else launch_fc_kernel(fc2_single_kernel<2>, (unsigned)grid, F2S_THREADS, 0, st, a);
  return hipGetLastError();
}

}  // namespace mvq
