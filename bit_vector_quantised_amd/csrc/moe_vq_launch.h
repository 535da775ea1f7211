// Host-side launch entry points of the kernel translation units.
#pragma once

#include <hip/hip_ext.h>

#include "moe_vq_internal.h"

namespace mvq {

// Measurement hook (moe_vq_time_next_kernel): events that the next FC kernel launched on
// this thread records at its start and at its end.
struct KernelTiming {
  hipEvent_t start = nullptr, stop = nullptr;
};
KernelTiming& kernel_timing();  // this thread's hook

// Launch one FC kernel; with the thread's hook set, through hipExtLaunchKernelGGL with
// the hook's events (which then time the kernel alone), clearing the hook.
template <typename... KArgs, typename... Args>
inline void launch_fc_kernel(void (*kern)(KArgs...), unsigned grid, unsigned block, uint32_t shmem,
                             hipStream_t st, Args... args) {
  KernelTiming& t = kernel_timing();
  if (t.start || t.stop) {
    const KernelTiming use = t;
    t = KernelTiming{};
    hipExtLaunchKernelGGL(kern, dim3(grid), dim3(block), shmem, st, use.start, use.stop, 0, args...);
  } else {
    kern<<<grid, block, shmem, st>>>(args...);
  }
}

hipError_t launch_route(const RouteArgs& ra, int x_dtype, const WorklistArgs& wa, hipStream_t st);

// FC1 / FC2 (+ combine) of the decode path; MT = token-group size, max_groups = the
// worst-case number of token groups for this n_tokens, n_cu = compute units.
// Matrix-core decode kernel for token groups of 16 (K = 1024, 2048; FC1 also 7168);
// *done says whether it took the call.
template <bool FC1>
hipError_t launch_mfma(const FcArgs& a, int K, int MT, int max_groups, int n_cu, hipStream_t st, bool* done);

// FC2 and the combine at once for a one-token step (K = 1024 or 2048, k <= 8).
hipError_t launch_fc2_single(const FcArgs& a, int MT, hipStream_t st, bool* done);

hipError_t launch_fc1(const FcArgs& a, int MT, int max_groups, int n_cu, hipStream_t st);
hipError_t launch_fc2(const FcArgs& a, int MT, int max_groups, int n_cu, hipStream_t st);

// y[t] = sum_i o_buf[t*k + i] (the per-pair outputs, already weighted).
void launch_combine(const float* o_buf, float* y, int T, int H, int k, int accumulate, int blocks, hipStream_t st);

// Prefill: stage x, token tiles, FC1 and FC2 as grouped MFMA GEMMs, combine.
hipError_t launch_prefill(const PrefillArgs& a, int x_dtype, hipStream_t st);

// Streaming read of bytes (a multiple of 16) at buf; sink[0] is written only in a case
// that does not occur in practice.
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, int n_cu, hipStream_t st);

hipError_t launch_decode_expert(const uint8_t* pool, const moe_vq_slot* slots, uint64_t pool_bytes,
                                const uint16_t* codebook, int H, int I, int expert, int matrix,
                                int out_dtype, void* out, int32_t* status_dev, hipStream_t st);

}  // namespace mvq
