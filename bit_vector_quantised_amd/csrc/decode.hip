// Decode one expert matrix to fp32 or bf16 -- the test hook that pins the on-device
// decode bit-exactly.  It uses the same LDS table and FP4 convert as the FC kernels.
//
// VQ2: W[n, 4j+d] = S[n, (4j+d)/128] * sgn(b) * CB[b & 0x7F][d] for word b = codes[n][j]
// (Tandem-vLLM 0.2.0 announcement, "How it works": 2-bit vector codes; vLLM-Moet
// README, "2-bit experts on vLLM v0.24.0": sign-symmetric codebook).  The product of
// the fp16 scale and the fp16 codebook component is exact in fp32.
// MXFP4: W[n, k] = E2M1(q) * 2^(e-127), low nibble = even k (Tandem-vLLM announcement,
// "Quality vs the official FP4 checkpoint": the most-routed experts kept in FP4).
#include "moe_vq_device.h"
#include "moe_vq_launch.h"

namespace mvq {

constexpr int DEC_THREADS = 256;
constexpr int DEC_ROWS = 16;  // rows per workgroup

__global__ __launch_bounds__(DEC_THREADS) void decode_expert_kernel(
    const uint8_t* __restrict__ pool, const moe_vq_slot* __restrict__ slots, uint64_t pool_bytes,
    const uint16_t* __restrict__ codebook, int H, int I, int expert, int matrix, int out_dtype,
    void* __restrict__ out, int32_t* __restrict__ status_dev) {
  __shared__ uint2 tab[256 * TAB_COPIES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const moe_vq_slot sl = slots[expert];
  const uint32_t fmt = sl.format;
  uint64_t need = 0;
  if (fmt == MOE_VQ_FMT_VQ2 || fmt == MOE_VQ_FMT_MXFP4) need = slot_layout((int)fmt, H, I).total;
  const bool ok = need != 0 && (sl.byte_offset & 255) == 0 && sl.byte_offset <= pool_bytes &&
                  need <= pool_bytes - sl.byte_offset;
  if (blockIdx.x == 0 && tid == 0 && status_dev) *status_dev = ok ? MOE_VQ_OK : MOE_VQ_ENOTRESIDENT;
  if (!ok) return;
  const SlotLayout L = slot_layout((int)fmt, H, I);
  const uint8_t* slot = pool + sl.byte_offset;
  const int rows = matrix == MOE_VQ_MAT_DOWN ? H : I;
  const int K = matrix == MOE_VQ_MAT_DOWN ? I : H;
  const uint64_t qoff = matrix == MOE_VQ_MAT_GATE ? L.q_gate : matrix == MOE_VQ_MAT_UP ? L.q_up : L.q_down;
  const uint64_t soff = matrix == MOE_VQ_MAT_GATE ? L.s_gate : matrix == MOE_VQ_MAT_UP ? L.s_up : L.s_down;
  const uint32_t laneoff = (uint32_t)(lane & 31) << 3;
  float* of = static_cast<float*>(out);
  uint16_t* ob = static_cast<uint16_t*>(out);

  if (fmt == MOE_VQ_FMT_VQ2) {
    build_vq2_table(tab, codebook, tid, DEC_THREADS);
    __syncthreads();
    const uint8_t* q = slot + qoff;
    const uint16_t* s = reinterpret_cast<const uint16_t*>(slot + soff);
    const int wpr = K / 4;
    for (int r = wave; r < DEC_ROWS; r += DEC_THREADS / 64) {
      const int n = blockIdx.x * DEC_ROWS + r;
      if (n >= rows) break;
      for (int j = lane; j < wpr; j += 64) {
        const uint32_t word = q[(size_t)n * wpr + j];
        const uint2 v = tab_lookup(tab, tab_addr<0>(word, laneoff));
        const float sc = f16_bits_to_f32(s[(size_t)n * (K / 128) + (4 * j) / 128]);
        const float w4[4] = {f16_bits_to_f32(v.x & 0xFFFFu) * sc, f16_bits_to_f32(v.x >> 16) * sc,
                             f16_bits_to_f32(v.y & 0xFFFFu) * sc, f16_bits_to_f32(v.y >> 16) * sc};
        const size_t o = (size_t)n * K + 4 * j;
        if (out_dtype == MOE_VQ_F32) {
          *reinterpret_cast<float4*>(of + o) = make_float4(w4[0], w4[1], w4[2], w4[3]);
        } else {
          ob[o] = f32_to_bf16_rne(w4[0]); ob[o + 1] = f32_to_bf16_rne(w4[1]);
          ob[o + 2] = f32_to_bf16_rne(w4[2]); ob[o + 3] = f32_to_bf16_rne(w4[3]);
        }
      }
    }
  } else {
    const uint8_t* q = slot + qoff;
    const uint8_t* s = slot + soff;
    const int bpr = K / 2;
    for (int r = wave; r < DEC_ROWS; r += DEC_THREADS / 64) {
      const int n = blockIdx.x * DEC_ROWS + r;
      if (n >= rows) break;
      for (int j = lane; j < bpr; j += 64) {
        const uint32_t byte = q[(size_t)n * bpr + j];
        const half2_t hv = fp4x2_to_half2<0>(byte);
        const float sc = e8m0_to_f32(s[(size_t)n * (K / 32) + (2 * j) / 32]);
        const float w0 = (float)hv.x * sc, w1 = (float)hv.y * sc;
        const size_t o = (size_t)n * K + 2 * j;
        if (out_dtype == MOE_VQ_F32) {
          of[o] = w0; of[o + 1] = w1;
        } else {
          ob[o] = f32_to_bf16_rne(w0); ob[o + 1] = f32_to_bf16_rne(w1);
        }
      }
    }
  }
}

hipError_t launch_decode_expert(const uint8_t* pool, const moe_vq_slot* slots, uint64_t pool_bytes,
                                const uint16_t* codebook, int H, int I, int expert, int matrix,
                                int out_dtype, void* out, int32_t* status_dev, hipStream_t st) {
  (void)hipGetLastError();  // start from a clean error state: report only our own launches
  const int rows = matrix == MOE_VQ_MAT_DOWN ? H : I;
  decode_expert_kernel<<<(rows + DEC_ROWS - 1) / DEC_ROWS, DEC_THREADS, 0, st>>>(
      pool, slots, pool_bytes, codebook, H, I, expert, matrix, out_dtype, out, status_dev);
  return hipGetLastError();
}

}  // namespace mvq
