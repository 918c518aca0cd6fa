// sd_internal.hpp -- host-side launchers shared between the kernel files and the C ABI.
// Each launcher assumes the arguments were validated by api.hip and returns the
// hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sd {

// Largest head count / head dim / top-k the kernels are instantiated for.
constexpr int kMaxHeads = 64;
constexpr int kMaxDim = 512;
constexpr int kMaxWindow = 128;
constexpr int kMaxTopK = 1024;
constexpr int kMaxKlK = 4096;

hipError_t launch_window_lse(const void *q, const void *kwin, const float *sink, const int32_t *seg, int B,
                             int S, int H, int D, int W, float scale, int dtype, float *nc_lse,
                             hipStream_t stream);

hipError_t launch_distill_target(const void *q, const void *pool, const int32_t *idx, const float *nc_lse,
                                 int B, int S, int H, int D, int N, int K, float scale, float l1_floor,
                                 int dtype, float *target, hipStream_t stream);

hipError_t launch_distill_target_fused(const void *q, const void *kwin, const float *sink, const int32_t *seg,
                                       const void *pool, const int32_t *idx, int B, int S, int H, int D, int N,
                                       int K, int W, float scale, float l1_floor, int dtype, float *target,
                                       float *nc_out, hipStream_t stream);

size_t kl_workspace_bytes(int B, int S, int K);
hipError_t launch_distill_kl(const float *target, const float *logits, const int32_t *idx, int B, int S,
                             int K, int N, float grad_scale, float *kl_rows, float *dlogits, float *stats,
                             void *workspace, hipStream_t stream);

}  // namespace sd
