// Routed experts computed on the host cores: the experts of a step that are not resident
// in the device slot pool, read from the host pool of the expert tier and decoded in
// fp32, while the GPU computes the resident ones (Tandem-vLLM 0.2.0 announcement, "How it
// works": experts that miss the GPU's cache are computed by the CPU in parallel with the
// GPU; "What you need": an AVX2 or AVX-512 CPU).
//
// For each selected expert e the call computes, for its tokens t (pairs (t, i) with
// topk_ids[t][i] == e): g = W_g x_t, u = W_u x_t, h = silu(g) * u (with the layer's SwiGLU
// clamp, if any), o = W_d h, and adds
// topk_w[t][i] * o to y[t].  Weights are decoded exactly (VQ2: scale times the signed
// codebook vector, a product of two fp16 values; MXFP4: E2M1 value times 2^(e - 127)),
// products and sums are fp32, so the result differs from the GPU's only in summation
// order and in the GPU's fp16 staging of the activations.
//
// Work: the FC1 rows of every computed expert (then, after a barrier, their FC2 rows) are
// split over a team of host threads in items of 16 rows; each row is decoded once into a
// per-thread fp32 buffer and applied to all of the expert's tokens.  y is accumulated
// after the team, experts in ascending id and pairs in order, so results are reproducible.  The hot loops are compiled for AVX-512, AVX2 + FMA and a
// generic x86-64 target, chosen at load time (function multiversioning).
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <condition_variable>
#include <functional>
#include <memory>
#include <mutex>
#include <thread>

#include "moe_vq.h"

namespace {

constexpr int CPU_MAX_THREADS = 256;

// fp16 bits -> fp32, exact (normal, subnormal, zero, inf, NaN).
float f16_to_f32(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  const uint32_t exp = (h >> 10) & 0x1Fu, man = h & 0x3FFu;
  uint32_t bits;
  if (exp == 0) {
    if (man == 0) {
      bits = sign;
    } else {  // subnormal: man * 2^-24
      float v = (float)man * 5.9604644775390625e-8f;
      memcpy(&bits, &v, 4);
      bits |= sign;
    }
  } else if (exp == 31) {
    bits = sign | 0x7F800000u | (man << 13);
  } else {
    bits = sign | ((exp + 112) << 23) | (man << 13);
  }
  float f;
  memcpy(&f, &bits, 4);
  return f;
}

float bf16_to_f32(uint16_t b) {
  const uint32_t bits = (uint32_t)b << 16;
  float f;
  memcpy(&f, &bits, 4);
  return f;
}

// OCP MX v1.0 FP4 (E2M1) element values of codes 0..15.
const float E2M1[16] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f, -0.f, -0.5f, -1.f, -1.5f, -2.f, -3.f, -4.f, -6.f};

// 2^(e - 127) for an E8M0 byte (255 encodes NaN).
float e8m0_to_f32(uint32_t e) { return e == 255 ? NAN : ldexpf(1.0f, (int)e - 127); }

// silu(g) * u, or with the SwiGLU clamp of limit lim > 0, silu(min(g, lim)) *
// clamp(u, -lim, lim) (a NaN stays NaN)
float swiglu(float g, float u, float lim) {
  if (lim > 0.f) {
    g = g > lim ? lim : g;
    u = u > lim ? lim : (u < -lim ? -lim : u);
  }
  return g / (1.0f + expf(-g)) * u;
}

struct Slot {
  int fmt;
  const uint8_t* q[3];  // gate, up, down payload
  const uint8_t* s[3];  // gate, up, down scales
};

// Row n of matrix m ([rows][K]) decoded to fp32.
void decode_row(const Slot& sl, const float (*tab)[4], int m, int n, int K, float* out) {
  if (sl.fmt == MOE_VQ_FMT_VQ2) {
    const uint8_t* q = sl.q[m] + (size_t)n * (K / 4);
    const uint16_t* sc = reinterpret_cast<const uint16_t*>(sl.s[m]) + (size_t)n * (K / 128);
    for (int g = 0; g < K / 128; ++g) {
      const float s = f16_to_f32(sc[g]);
      for (int j = 0; j < 32; ++j) {
        const float* v = tab[q[g * 32 + j]];
        float* o = out + g * 128 + 4 * j;
        o[0] = s * v[0];
        o[1] = s * v[1];
        o[2] = s * v[2];
        o[3] = s * v[3];
      }
    }
  } else {
    const uint8_t* q = sl.q[m] + (size_t)n * (K / 2);
    const uint8_t* e = sl.s[m] + (size_t)n * (K / 32);
    for (int b = 0; b < K / 32; ++b) {
      const float s = e8m0_to_f32(e[b]);
      for (int j = 0; j < 16; ++j) {
        const uint8_t byte = q[b * 16 + j];
        out[b * 32 + 2 * j] = E2M1[byte & 0xF] * s;     // low nibble: even index
        out[b * 32 + 2 * j + 1] = E2M1[byte >> 4] * s;
      }
    }
  }
}

// dot of one decoded row with each of m vectors [m][K]: out[i] = sum_k w[k] v[i][k]
__attribute__((target_clones("avx512f", "avx2,fma", "default")))
void dot_rows(const float* w, const float* v, int m, int K, float* out) {
  for (int i = 0; i < m; ++i) {
    const float* x = v + (size_t)i * K;
    // sixteen partial sums, so the compiler vectorises without reordering one chain
    float acc[16] = {};
    int k = 0;
    for (; k + 16 <= K; k += 16)
      for (int j = 0; j < 16; ++j) acc[j] += w[k + j] * x[k + j];
    float s = 0.f;
    for (; k < K; ++k) s += w[k] * x[k];
    for (int j = 0; j < 16; ++j) s += acc[j];
    out[i] = s;
  }
}

// One call's threads: phase 1 work items, a barrier, phase 2 work items (the caller's
// thread takes part).  Items are taken in order from a shared counter.
void run_two_phases(int n_threads, int items1, const std::function<void(int)>& f1, int items2,
                    const std::function<void(int)>& f2) {
  std::atomic<int> next1{0}, next2{0};
  std::mutex mu;
  std::condition_variable cv;
  int arrived = 0;
  auto body = [&]() {
    for (int i; (i = next1.fetch_add(1)) < items1;) f1(i);
    {
      std::unique_lock<std::mutex> lock(mu);
      if (++arrived == n_threads) cv.notify_all();
      else cv.wait(lock, [&] { return arrived == n_threads; });
    }
    for (int i; (i = next2.fetch_add(1)) < items2;) f2(i);
  };
  std::unique_ptr<std::thread[]> ts(new std::thread[n_threads - 1]);
  for (int i = 0; i < n_threads - 1; ++i) ts[i] = std::thread(body);
  body();
  for (int i = 0; i < n_threads - 1; ++i) ts[i].join();
}

}  // namespace

extern "C" {

int moe_vq_cpu_experts(const moe_vq_layer* layer, const uint8_t* host_pool, uint64_t host_pool_bytes,
                       const moe_vq_slot* host_slots, const void* codebook, const void* x, int x_dtype,
                       int n_tokens, const int32_t* topk_ids, const float* topk_w, const uint8_t* compute, float* y,
                       int n_threads) {
  if (!layer) return MOE_VQ_EINVAL;
  const int H = layer->hidden, I = layer->inter, E = layer->n_experts, k = layer->top_k;
  if (H < 128 || H > 16384 || H % 128 || I < 128 || I > 16384 || I % 128 || E < 1 || E > 1024 || k < 1 || k > 32 ||
      k > E)
    return MOE_VQ_EINVAL;
  if (n_tokens < 0 || n_tokens > 65536 || (x_dtype != MOE_VQ_F32 && x_dtype != MOE_VQ_BF16)) return MOE_VQ_EINVAL;
  const float lim = layer->swiglu_limit;
  if (!(lim >= 0.f && lim <= 3.4e38f)) return MOE_VQ_EINVAL;  // finite, >= 0 (NaN fails)
  if (layer->delta_slots) return MOE_VQ_EUNSUPPORTED;  // the FP4 delta cache is device-side only
  if (n_tokens == 0) return MOE_VQ_OK;
  if (!host_pool || !host_slots || !codebook || !x || !topk_ids || !topk_w || !compute || !y) return MOE_VQ_EINVAL;
  if (n_threads < 1 || n_threads > CPU_MAX_THREADS) return MOE_VQ_EINVAL;
  const int T = n_tokens;

  // which experts this call computes (pairs grouped per expert, in pair order), and their
  // slots checked before any work.  (Fixed-size arrays: the library exports no standard
  // library template code.)
  const int P_all = T * k;
  std::unique_ptr<int[]> cnt(new int[E + 1]());
  for (int p = 0; p < P_all; ++p) {
    const int e = topk_ids[p];
    if (e < 0 || e >= E) return MOE_VQ_EINVAL;
    if (compute[e]) ++cnt[e + 1];
  }
  for (int e = 0; e < E; ++e) cnt[e + 1] += cnt[e];  // first pair of expert e in plist
  std::unique_ptr<int[]> plist(new int[P_all > 0 ? P_all : 1]);
  {
    std::unique_ptr<int[]> fill(new int[E]);
    for (int e = 0; e < E; ++e) fill[e] = cnt[e];
    for (int p = 0; p < P_all; ++p)
      if (compute[topk_ids[p]]) plist[fill[topk_ids[p]]++] = p;
  }
  std::unique_ptr<int[]> experts(new int[E]);
  int nE = 0;
  std::unique_ptr<Slot[]> slots(new Slot[E]);
  for (int e = 0; e < E; ++e) {
    if (cnt[e + 1] == cnt[e]) continue;
    const moe_vq_slot hs = host_slots[e];
    const size_t need = moe_vq_expert_bytes((int)hs.format, H, I);
    if (need == 0) return MOE_VQ_ENOTRESIDENT;  // not in the host pool either: nothing to compute it from
    if (hs.byte_offset > host_pool_bytes || need > host_pool_bytes - hs.byte_offset) return MOE_VQ_ENOTRESIDENT;
    uint64_t off[7];
    moe_vq_slot_layout((int)hs.format, H, I, off);
    Slot& sl = slots[e];
    sl.fmt = (int)hs.format;
    const uint8_t* base = host_pool + hs.byte_offset;
    for (int m = 0; m < 3; ++m) {
      sl.q[m] = base + off[m];
      sl.s[m] = base + off[3 + m];
    }
    experts[nE++] = e;
  }
  if (nE == 0) return MOE_VQ_OK;

  // signed codebook in fp32: word b -> sgn(b) * CB[b & 0x7F] (exact)
  float tab[256][4];
  const uint16_t* cb = static_cast<const uint16_t*>(codebook);
  for (int b = 0; b < 256; ++b)
    for (int d = 0; d < 4; ++d) {
      const float v = f16_to_f32(cb[(b & 0x7F) * 4 + d]);
      tab[b][d] = (b & 0x80) ? -v : v;
    }

  // every computed expert's tokens' activations in fp32 (exact: bf16 or fp32 values),
  // then FC1 rows and FC2 rows of all experts as the two phases' work items
  // base[j]: first pair of the j-th computed expert in plist (its pairs are contiguous)
  std::unique_ptr<size_t[]> base(new size_t[nE + 1]);
  for (int j = 0; j < nE; ++j) base[j] = (size_t)cnt[experts[j]];
  std::unique_ptr<size_t[]> rank(new size_t[nE + 1]);  // row of the j-th expert's first pair in xs/hs/os
  rank[0] = 0;
  for (int j = 0; j < nE; ++j) rank[j + 1] = rank[j] + (size_t)(cnt[experts[j] + 1] - cnt[experts[j]]);
  const size_t P = rank[nE];
  std::unique_ptr<float[]> xs(new float[P * H]), hs(new float[P * I]), os(new float[P * H]);
  for (int j = 0; j < nE; ++j)
    for (size_t i = 0; i < rank[j + 1] - rank[j]; ++i) {
      const int t = plist[base[j] + i] / k;
      float* dst = xs.get() + (rank[j] + i) * H;
      for (int c = 0; c < H; ++c)
        dst[c] = x_dtype == MOE_VQ_BF16 ? bf16_to_f32(static_cast<const uint16_t*>(x)[(size_t)t * H + c])
                                        : static_cast<const float*>(x)[(size_t)t * H + c];
    }
  constexpr int ROWS = 16;  // rows per work item
  const int c1 = (I + ROWS - 1) / ROWS, c2 = (H + ROWS - 1) / ROWS;
  // per-thread row buffers: two decoded rows of length max(H, I) and the m dot products
  const size_t mmax = (size_t)k * T;
  auto fc1 = [&](int item) {
    const int j = item / c1, r0 = (item % c1) * ROWS;
    const Slot& sl = slots[experts[j]];
    const int m = (int)(rank[j + 1] - rank[j]);
    std::unique_ptr<float[]> buf(new float[2 * (size_t)H + 2 * mmax]);
    float *wg = buf.get(), *wu = wg + H, *g = wu + H, *u = g + mmax;
    for (int n = r0; n < std::min(I, r0 + ROWS); ++n) {
      decode_row(sl, tab, 0, n, H, wg);
      decode_row(sl, tab, 1, n, H, wu);
      dot_rows(wg, xs.get() + rank[j] * H, m, H, g);
      dot_rows(wu, xs.get() + rank[j] * H, m, H, u);
      for (int i = 0; i < m; ++i) hs[(rank[j] + i) * I + n] = swiglu(g[i], u[i], lim);
    }
  };
  auto fc2 = [&](int item) {
    const int j = item / c2, r0 = (item % c2) * ROWS;
    const Slot& sl = slots[experts[j]];
    const int m = (int)(rank[j + 1] - rank[j]);
    std::unique_ptr<float[]> buf(new float[(size_t)I + mmax]);
    float *wd = buf.get(), *o = wd + I;
    for (int n = r0; n < std::min(H, r0 + ROWS); ++n) {
      decode_row(sl, tab, 2, n, I, wd);
      dot_rows(wd, hs.get() + rank[j] * I, m, I, o);
      for (int i = 0; i < m; ++i) os[(rank[j] + i) * H + n] = o[i];
    }
  };
  run_two_phases(n_threads, nE * c1, fc1, nE * c2, fc2);
  // y[t] += w * o, experts in ascending id, each expert's pairs in pair order
  for (int j = 0; j < nE; ++j)
    for (size_t i = 0; i < rank[j + 1] - rank[j]; ++i) {
      const int p = plist[base[j] + i], t = p / k;
      const float w = topk_w[p];
      const float* o = os.get() + (rank[j] + i) * H;
      for (int c = 0; c < H; ++c) y[(size_t)t * H + c] += w * o[c];
    }
  return MOE_VQ_OK;
}

}  // extern "C"
