// Streaming read probe: the HBM read rate this device reaches with plain 16-byte loads,
// against which the decode kernels' code-stream rate is compared (a roofline measured on
// the same device beside the published peak).
#include "moe_vq_launch.h"

namespace mvq {

constexpr int PROBE_THREADS = 256;
constexpr int PROBE_UNROLL = 4;  // independent 16-byte loads per thread and pass: 16 KB per workgroup

// Each workgroup reads contiguous 16 KB blocks, grid-strided; the loads are XOR-folded
// and the fold is stored only if it equals a constant no data produces in practice, so
// that no load can be dropped while nothing is written on a normal run.
__global__ __launch_bounds__(PROBE_THREADS) void read_probe_kernel(const uint4* __restrict__ buf, size_t n16,
                                                                   uint32_t* sink) {
  const size_t block = (size_t)PROBE_THREADS * PROBE_UNROLL;
  uint32_t acc = 0;
  for (size_t base = (size_t)blockIdx.x * block; base < n16; base += (size_t)gridDim.x * block) {
    uint4 v[PROBE_UNROLL];
#pragma unroll
    for (int j = 0; j < PROBE_UNROLL; ++j) {
      const size_t i = base + (size_t)j * PROBE_THREADS + threadIdx.x;
      v[j] = i < n16 ? buf[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int j = 0; j < PROBE_UNROLL; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, int n_cu, hipStream_t st) {
  const size_t n16 = bytes / 16;
  const size_t blocks = (n16 + PROBE_THREADS * PROBE_UNROLL - 1) / (PROBE_THREADS * PROBE_UNROLL);
  size_t grid = (size_t)n_cu * 4;
  if (blocks < grid) grid = blocks;
  launch_fc_kernel(read_probe_kernel, (unsigned)grid, PROBE_THREADS, 0, st, static_cast<const uint4*>(buf), n16, sink);
  return hipGetLastError();
}

}  // namespace mvq
