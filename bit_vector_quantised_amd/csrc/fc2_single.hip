// FC2 (down) with the weighted combine, for a step of one token: y = sum_i w_i W_d,i h_i.
//
// Sources: FC2 per routed expert decoded from the 2-bit codes, then the experts' outputs
// added with the routing weights (Tandem-vLLM 0.2.0 announcement, "How it works";
// vLLM-Moet README, "2-bit experts on vLLM v0.24.0"); no padding rows written back
// (vLLM-Moet README, "What we changed against official vLLM", row "MoE at decode").
//
// With one token the k routed experts all write the same output rows.  A workgroup here
// owns a block of output rows and walks every expert for them: it stages all k pairs' h
// once (fp16, one power-of-two factor per pair and 1024 columns, as the other FC2
// kernels do), issues every VQ2 code load of its rows up front, and adds w_i times each
// expert's partial dot product in registers, in the worklist's expert order.  The 16
// lanes of a row are reduced once, at the end, and y is written directly: no per-pair
// outputs and no separate combine launch.  Seven waves of four rows give 28 rows per
// workgroup, so H = 7168 is 256 workgroups, one per CU.
#include "fc_common.h"

namespace mvq {

constexpr int F2S_WAVES = 7;
constexpr int F2S_THREADS = 64 * F2S_WAVES;
constexpr int F2S_ROWS = 4 * F2S_WAVES;  // 16 lanes per row, 4 rows per wave
constexpr int F2S_KMAX = 8;              // routed experts per token this kernel takes

template <int CPL>
__global__ __launch_bounds__(F2S_THREADS, 1) void fc2_single_kernel(FcArgs a) {
  constexpr int K = 1024 * CPL;
  constexpr int KS = CPL;                      // activation slices of 1024 columns
  constexpr int XT = (K / 64) * XCHUNK_UNITS;  // padded 16-byte units per pair
  constexpr int NGS = F2S_KMAX * KS;           // (pair, slice) units to stage, at most
  constexpr int GSW = (NGS + F2S_WAVES - 1) / F2S_WAVES;  // of them per wave, at most
  __shared__ uint2 tab[256 * TAB_COPIES];
  __shared__ uint4 xs[F2S_KMAX * XT];
  __shared__ float xsc[NGS];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rg = lane >> 4, sub = lane & 15;
  const uint32_t laneoff = (uint32_t)(lane & 31) << 3;
  const int n_raw = blockIdx.x * F2S_ROWS + wave * 4 + rg;
  const int n = min(n_raw, a.H - 1);  // rows past the end re-read the last row, written never

  const uint2 cbv = reinterpret_cast<const uint2*>(a.codebook)[tid & 127];
  if (!ws_ok(a, false, 1)) return;
  const int G = (int)a.hdr[HDR_GROUPS2];  // one group per routed pair
  if (G > F2S_KMAX) return;               // (the launcher takes this kernel only for k <= 8)

  // the routed pairs, in the worklist's expert order
  RecS rec[F2S_KMAX];
#pragma unroll
  for (int g = 0; g < F2S_KMAX; ++g) rec[g] = load_rec(a.rec, g < G ? g : 0);

  // ---- h of this wave's (pair, slice) units: issued before the code loads, which are
  // the bulk of the traffic
  float4 hv[GSW][4];
#pragma unroll
  for (int i = 0; i < GSW; ++i) {
    const int gs = wave + i * F2S_WAVES;
    if (gs < G * KS) {
      const int g = gs / KS, sl = gs % KS;
      int p = rec[0].pair[0];
#pragma unroll
      for (int gg = 1; gg < F2S_KMAX; ++gg) p = g == gg ? rec[gg].pair[0] : p;
      const float4* row = reinterpret_cast<const float4*>(a.h_in + (size_t)p * K + sl * SLICE);
#pragma unroll
      for (int r = 0; r < 4; ++r) hv[i][r] = row[r * 64 + lane];
    }
  }

  // ---- every VQ2 code load of this lane's row, for all experts
  uint4 q[F2S_KMAX][CPL];
  uint32_t s[F2S_KMAX][CPL];
#pragma unroll
  for (int g = 0; g < F2S_KMAX; ++g) {
    if (g < G && rec[g].fmt == MOE_VQ_FMT_VQ2) {
      const uint8_t* slot = a.pool + rec[g].slot_off;
      const uint8_t* qb = slot + a.vq2.q_down + (size_t)n * (K / 4) + sub * 16;
      const uint8_t* sb = slot + a.vq2.s_down + (size_t)n * (K / 64) + (sub >> 1) * 2;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        q[g][j] = *reinterpret_cast<const uint4*>(qb + j * 256);
        s[g][j] = *reinterpret_cast<const uint16_t*>(sb + j * 16);
      }
    }
  }

  // ---- stage h: fp16 with one power-of-two factor per (pair, slice); one wave per unit
#pragma unroll
  for (int i = 0; i < GSW; ++i) {
    const int gs = wave + i * F2S_WAVES;
    if (gs < G * KS) {
      const int g = gs / KS, sl = gs % KS;
      float m = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        m = fmaxf(m, fmaxf(fmaxf(fabsf(hv[i][r].x), fabsf(hv[i][r].y)), fmaxf(fabsf(hv[i][r].z), fabsf(hv[i][r].w))));
      m = wave_max(m);
      int ex = 0;
      if (m > 0.f && m < INFINITY) ex = frexp_exponent(m) - 15;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float4 v = hv[i][r];
        const int f = r * 64 + lane;          // float4 index within the slice
        const int u = sl * (SLICE / 8) + (f >> 1);  // 16-byte unit within the pair
        reinterpret_cast<uint2*>(xs)[(g * XT + x_unit(u)) * 2 + (f & 1)] =
            make_uint2(pack_half2(ldexp2(v.x, -ex), ldexp2(v.y, -ex)), pack_half2(ldexp2(v.z, -ex), ldexp2(v.w, -ex)));
      }
      if (lane == 0) xsc[gs] = ldexp2(1.0f, ex);
    }
  }
  if (tid < 256) write_table_entry(tab, cbv, tid);
  __syncthreads();

  // ---- every expert's product for this row, weighted, summed in expert order
  float acc = 0.f;
#pragma unroll
  for (int g = 0; g < F2S_KMAX; ++g) {
    if (g < G) {
      const RecS& r = rec[g];
      const float w = a.pair_w[r.pair[0]];
      if (r.fmt == MOE_VQ_FMT_VQ2) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          const uint4* xp = xs + g * XT + (sub + 16 * j) * XCHUNK_UNITS;
          float pr = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint4 xr[2] = {xp[2 * i], xp[2 * i + 1]};
            pr = vq2_dword_dot(tab, dword_of(q[g][j], i), laneoff, reinterpret_cast<const uint32_t*>(xr), pr);
          }
          acc = fmaf(w * f16_bits_to_f32(s[g][j]) * xsc[g * KS + j], pr, acc);
        }
      } else if (r.fmt == MOE_VQ_FMT_MXFP4) {
        // MXFP4 experts (not in flight ahead): 2 * CPL chunks of 32 weights per lane
        const uint8_t* slot = a.pool + r.slot_off;
        const uint8_t* qb = slot + a.mx4.q_down + (size_t)n * (K / 2);
        const uint8_t* eb = slot + a.mx4.s_down + (size_t)n * (K / 32);
        uint4 qm[2 * CPL];
        uint32_t em[2 * CPL];
#pragma unroll
        for (int j = 0; j < 2 * CPL; ++j) {
          const int c = sub + 16 * j;
          qm[j] = *reinterpret_cast<const uint4*>(qb + c * 16);
          em[j] = eb[c];
        }
#pragma unroll
        for (int j = 0; j < 2 * CPL; ++j) {
          const int c = sub + 16 * j;
          const uint4* xp = xs + g * XT + (c >> 1) * XCHUNK_UNITS + (c & 1) * 4;
          uint4 xr[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) xr[i] = xp[i];
          const float pr = mx4_chunk_dot(qm[j], reinterpret_cast<const uint32_t*>(xr));
          acc = fmaf(w * e8m0_to_f32(em[j]) * xsc[g * KS + (c >> 5)], pr, acc);
        }
      }
      // (an absent expert adds nothing; the worklist has recorded MOE_VQ_ENOTRESIDENT)
    }
  }
  acc = group_sum<16>(acc);
  if (sub == 0 && n_raw < a.H) a.y[n_raw] = acc;
}

// y for a one-token step straight from the experts (K = 1024 or 2048, k <= 8); *done
// says whether it took the call.
hipError_t launch_fc2_single(const FcArgs& a, int MT, hipStream_t st, bool* done) {
  *done = false;
  if (a.T != 1 || MT != 1 || a.k > F2S_KMAX || (a.I != 1024 && a.I != 2048)) return hipSuccess;
  const int grid = (a.H + F2S_ROWS - 1) / F2S_ROWS;
  *done = true;
  if (a.I == 1024) fc2_single_kernel<1><<<grid, F2S_THREADS, 0, st>>>(a);
  else fc2_single_kernel<2><<<grid, F2S_THREADS, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace mvq
