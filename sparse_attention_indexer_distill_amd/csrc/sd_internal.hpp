// sd_internal.hpp -- host-side launchers shared between the kernel files and the C ABI.
// Each launcher assumes the arguments were validated by api.hip and returns the
// hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace sd {

// LDS per CU on gfx950.
constexpr int kLdsBytes = 160 * 1024;

// Opts kernel KFN in to the whole 160 KiB of LDS as dynamic shared memory (the default cap
// is 64 KiB).  The attribute is set once per (kernel, device) -- not on every launch -- and
// remembered in a per-kernel bit mask of devices (devices past 63 set it on every call).
template <auto KFN>
hipError_t allow_full_lds() {
    static std::atomic<uint64_t> done{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
    if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(KFN), hipFuncAttributeMaxDynamicSharedMemorySize,
                            kLdsBytes);
    if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_release);
    return e;
}

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
// Rows the allocation-free KL entry point takes (its partials live in a fixed 2 MiB array).
constexpr int64_t kNoAllocMaxRows = (int64_t)1 << 21;
hipError_t launch_distill_kl_noalloc(const float *target, const float *logits, const int32_t *idx, int B, int S,
                                     int K, int N, float grad_scale, float *kl_rows, float *dlogits, float *stats,
                                     hipStream_t stream);
hipError_t launch_distill_kl(const float *target, const float *logits, const int32_t *idx, int B, int S,
                             int K, int N, float grad_scale, float *kl_rows, float *dlogits, float *stats,
                             void *workspace, hipStream_t stream);

constexpr int kMaxTopkN = 4096;
constexpr int kMaxTopkK = 4096;
hipError_t launch_indexer_topk(const float *scores, const int32_t *seg, int B, int S, int N, int K, int ratio,
                               int32_t *idx, float *values, hipStream_t stream);
hipError_t launch_indexer_topk_bwd(const float *dvalues, const int32_t *idx, int B, int S, int N, int K,
                                   float *dscores, hipStream_t stream);

bool compressor_supported(int ratio, int overlap);
size_t compressor_bwd_workspace_bytes(int B, int S, int D, int ratio, int overlap);
hipError_t launch_compressor_pool(const void *kv, const void *score, const float *ape, const int32_t *seg, int B,
                                  int S, int D, int ratio, int overlap, int dtype, float *pool, hipStream_t stream);
hipError_t launch_compressor_pool_bwd(const void *kv, const void *score, const float *ape, const int32_t *seg,
                                      const float *dpool, int B, int S, int D, int ratio, int overlap, int dtype,
                                      float *dkv, float *dscore, float *dape, void *workspace, hipStream_t stream);

}  // namespace sd
