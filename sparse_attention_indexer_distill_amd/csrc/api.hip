// api.hip -- the C ABI (include/sparse_distill.h): argument validation, then one or two
// kernel launches on the caller's stream.  Validation happens entirely on the host and
// before any HIP call, so every rejection path is exercised without a GPU.
#include <math.h>
#include <stdint.h>
#include <stdarg.h>
#include <stdio.h>

#include "../../include/sparse_distill.h"
#include "sd_internal.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_err[0] = '\0';
    return SD_OK;
}

int hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(SD_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int check_common(int dtype, int B, int S, int H, int D) {
    if (dtype != SD_BF16 && dtype != SD_F32) return fail(SD_ERR_DTYPE, "unknown dtype code %d", dtype);
    if (B <= 0 || S <= 0 || H <= 0 || D <= 0)
        return fail(SD_ERR_BAD_SHAPE, "sizes must be positive (B=%d S=%d H=%d D=%d)", B, S, H, D);
    if ((int64_t)B * S * H * D > ((int64_t)1 << 40)) return fail(SD_ERR_BAD_SHAPE, "q is too large");
    if (D % 32 != 0 || D > sd::kMaxDim)
        return fail(SD_ERR_UNSUPPORTED, "head dim D=%d must be a multiple of 32 and at most %d", D, sd::kMaxDim);
    if (H > sd::kMaxHeads) return fail(SD_ERR_UNSUPPORTED, "H=%d heads exceeds the supported %d", H, sd::kMaxHeads);
    return SD_OK;
}

// The kernels address one batch row of pool or window keys through a 32-bit buffer range
// with 32-bit signed row offsets (row * D * element size), so each such row must stay
// below 2^31 bytes; row indices are multiplied in 24 bits, so at most 2^24 rows.
int check_rows(const char *fn, const char *what, int64_t rows, int D, int dtype) {
    const int64_t eb = dtype == SD_F32 ? 4 : 2;
    if (rows * D * eb > (((int64_t)1 << 31) - 1))
        return fail(SD_ERR_UNSUPPORTED, "%s: %s of %lld rows x D=%d exceeds 2^31 bytes per batch", fn, what,
                    (long long)rows, D);
    if (rows > ((int64_t)1 << 24))
        return fail(SD_ERR_UNSUPPORTED, "%s: %s of %lld rows exceeds 2^24 rows per batch", fn, what,
                    (long long)rows);
    return SD_OK;
}

// A dispatch counts its grid in work-items with 32-bit sizes, so blocks * threads per
// block must stay at or below 2^32 - 1.  The limits are checked here, before any HIP call,
// with the widest workgroup each entry point can launch.
int check_grid(const char *fn, int64_t blocks, int threads, const char *limit) {
    if (blocks * threads > (int64_t)UINT32_MAX)
        return fail(SD_ERR_UNSUPPORTED, "%s: %s (the grid would hold %lld work-items, above 2^32 - 1)", fn, limit,
                    (long long)(blocks * threads));
    return SD_OK;
}

}  // namespace

extern "C" {

const char *sd_status_string(int status) {
    switch (status) {
        case SD_OK: return "SD_OK";
        case SD_ERR_NULL_ARG: return "SD_ERR_NULL_ARG";
        case SD_ERR_BAD_SHAPE: return "SD_ERR_BAD_SHAPE";
        case SD_ERR_UNSUPPORTED: return "SD_ERR_UNSUPPORTED";
        case SD_ERR_DTYPE: return "SD_ERR_DTYPE";
        case SD_ERR_HIP: return "SD_ERR_HIP";
        default: return "SD_ERR_UNKNOWN";
    }
}

const char *sd_last_error(void) { return g_err; }

int window_lse(const void *q, const void *kwin, const float *sink, const int32_t *seg, int B, int S, int H, int D,
               int W, float scale, int dtype, float *nc_lse, hipStream_t stream) {
    if (!q || !kwin || !nc_lse) return fail(SD_ERR_NULL_ARG, "window_lse: q, kwin and nc_lse are required");
    int st = check_common(dtype, B, S, H, D);
    if (st != SD_OK) return st;
    if (W <= 0) return fail(SD_ERR_BAD_SHAPE, "window_lse: W=%d must be positive", W);
    if (W > sd::kMaxWindow) return fail(SD_ERR_UNSUPPORTED, "window_lse: W=%d exceeds %d", W, sd::kMaxWindow);
    if (!isfinite(scale)) return fail(SD_ERR_BAD_SHAPE, "window_lse: scale must be finite");
    if ((st = check_rows("window_lse", "kwin", S, D, dtype)) != SD_OK) return st;
    if ((st = check_grid("window_lse", ((int64_t)S + 1) / 2, 512, "S must be at most 2^24 - 2")) != SD_OK) return st;
    return hip_status(sd::launch_window_lse(q, kwin, sink, seg, B, S, H, D, W, scale, dtype, nc_lse, stream),
                      "window_lse launch");
}

int distill_target(const void *q, const void *pool, const int32_t *idx, const float *nc_lse, int B, int S, int H,
                   int D, int N, int K, float scale, float l1_floor, int dtype, float *target, hipStream_t stream) {
    if (!q || !pool || !idx || !target)
        return fail(SD_ERR_NULL_ARG, "distill_target: q, pool, idx and target are required");
    int st = check_common(dtype, B, S, H, D);
    if (st != SD_OK) return st;
    if (N <= 0 || K <= 0) return fail(SD_ERR_BAD_SHAPE, "distill_target: N=%d and K=%d must be positive", N, K);
    if (K > sd::kMaxTopK) return fail(SD_ERR_UNSUPPORTED, "distill_target: K=%d exceeds %d", K, sd::kMaxTopK);
    if (!isfinite(scale) || !(scale > 0.f) || isnan(l1_floor))
        return fail(SD_ERR_BAD_SHAPE, "distill_target: scale must be positive and finite, l1_floor not NaN");
    if ((st = check_rows("distill_target", "pool", N, D, dtype)) != SD_OK) return st;
    if ((st = check_grid("distill_target", (int64_t)B * S, 1024, "B*S must be below 2^22")) != SD_OK) return st;
    return hip_status(sd::launch_distill_target(q, pool, idx, nc_lse, B, S, H, D, N, K, scale, l1_floor, dtype,
                                                target, stream),
                      "distill_target launch");
}

int distill_target_fused(const void *q, const void *kwin, const float *sink, const int32_t *seg, const void *pool,
                         const int32_t *idx, int B, int S, int H, int D, int N, int K, int W, float scale,
                         float l1_floor, int dtype, float *target, float *nc_lse_out, hipStream_t stream) {
    if (!q || !kwin || !pool || !idx || !target)
        return fail(SD_ERR_NULL_ARG, "distill_target_fused: q, kwin, pool, idx and target are required");
    int st = check_common(dtype, B, S, H, D);
    if (st != SD_OK) return st;
    if (N <= 0 || K <= 0) return fail(SD_ERR_BAD_SHAPE, "distill_target_fused: N=%d and K=%d must be positive", N, K);
    if (W <= 0) return fail(SD_ERR_BAD_SHAPE, "distill_target_fused: W=%d must be positive", W);
    if (K > sd::kMaxTopK) return fail(SD_ERR_UNSUPPORTED, "distill_target_fused: K=%d exceeds %d", K, sd::kMaxTopK);
    if (W > sd::kMaxWindow) return fail(SD_ERR_UNSUPPORTED, "distill_target_fused: W=%d exceeds %d", W, sd::kMaxWindow);
    if (!isfinite(scale) || !(scale > 0.f) || isnan(l1_floor))
        return fail(SD_ERR_BAD_SHAPE, "distill_target_fused: scale must be positive and finite, l1_floor not NaN");
    if ((st = check_rows("distill_target_fused", "pool", N, D, dtype)) != SD_OK) return st;
    if ((st = check_rows("distill_target_fused", "kwin", S, D, dtype)) != SD_OK) return st;
    if ((st = check_grid("distill_target_fused", (int64_t)B * S, 1024, "B*S must be below 2^22")) != SD_OK)
        return st;
    return hip_status(sd::launch_distill_target_fused(q, kwin, sink, seg, pool, idx, B, S, H, D, N, K, W, scale,
                                                      l1_floor, dtype, target, nc_lse_out, stream),
                      "distill_target_fused launch");
}

size_t distill_kl_workspace_bytes(int B, int S, int K) {
    if (B <= 0 || S <= 0 || K <= 0) return 0;
    return sd::kl_workspace_bytes(B, S, K);
}

int distill_kl_fwd_bwd(const float *target, const float *logits, const int32_t *idx, int B, int S, int K, int N,
                       float grad_scale, float *kl_rows, float *dlogits, float *stats, void *workspace,
                       size_t workspace_bytes, hipStream_t stream) {
    if (!target || !logits || !idx || !kl_rows || !stats || !workspace)
        return fail(SD_ERR_NULL_ARG, "distill_kl_fwd_bwd: target, logits, idx, kl_rows, stats and workspace are required");
    if (B <= 0 || S <= 0 || K <= 0 || N <= 0)
        return fail(SD_ERR_BAD_SHAPE, "distill_kl_fwd_bwd: sizes must be positive (B=%d S=%d K=%d N=%d)", B, S, K, N);
    if (K > sd::kMaxKlK) return fail(SD_ERR_UNSUPPORTED, "distill_kl_fwd_bwd: K=%d exceeds %d", K, sd::kMaxKlK);
    // stats[1] counts rows in float32, which is exact up to 2^24
    if ((int64_t)B * S > ((int64_t)1 << 24))
        return fail(SD_ERR_UNSUPPORTED, "distill_kl_fwd_bwd: B*S=%lld exceeds 2^24 rows (the float32 row count "
                    "in stats[1] is exact only up to 2^24)", (long long)B * S);
    if (!isfinite(grad_scale)) return fail(SD_ERR_BAD_SHAPE, "distill_kl_fwd_bwd: grad_scale must be finite");
    const size_t need = sd::kl_workspace_bytes(B, S, K);
    if (workspace_bytes < need)
        return fail(SD_ERR_BAD_SHAPE, "distill_kl_fwd_bwd: workspace of %zu bytes, %zu needed", workspace_bytes, need);
    if ((uintptr_t)workspace % 16 != 0)
        return fail(SD_ERR_BAD_SHAPE, "distill_kl_fwd_bwd: workspace must be 16-byte aligned");
    return hip_status(sd::launch_distill_kl(target, logits, idx, B, S, K, N, grad_scale, kl_rows, dlogits, stats,
                                            workspace, stream),
                      "distill_kl_fwd_bwd launch");
}

int indexer_topk(const float *scores, const int32_t *seg, int B, int S, int N, int K, int ratio, int32_t *idx,
                 float *values, hipStream_t stream) {
    if (!scores || !idx) return fail(SD_ERR_NULL_ARG, "indexer_topk: scores and idx are required");
    if (B <= 0 || S <= 0 || N <= 0 || K <= 0 || ratio <= 0)
        return fail(SD_ERR_BAD_SHAPE, "indexer_topk: sizes must be positive (B=%d S=%d N=%d K=%d ratio=%d)", B, S, N, K,
                    ratio);
    if (N > sd::kMaxTopkN || K > sd::kMaxTopkK)
        return fail(SD_ERR_UNSUPPORTED, "indexer_topk: N=%d and K=%d must be at most %d and %d", N, K, sd::kMaxTopkN,
                    sd::kMaxTopkK);
    int st = check_grid("indexer_topk", ((int64_t)B * S + 3) / 4, 256, "B*S must be below 2^26");
    if (st != SD_OK) return st;
    return hip_status(sd::launch_indexer_topk(scores, seg, B, S, N, K, ratio, idx, values, stream),
                      "indexer_topk launch");
}

int indexer_topk_bwd(const float *dvalues, const int32_t *idx, int B, int S, int N, int K, float *dscores,
                     hipStream_t stream) {
    if (!dvalues || !idx || !dscores)
        return fail(SD_ERR_NULL_ARG, "indexer_topk_bwd: dvalues, idx and dscores are required");
    if (B <= 0 || S <= 0 || N <= 0 || K <= 0)
        return fail(SD_ERR_BAD_SHAPE, "indexer_topk_bwd: sizes must be positive (B=%d S=%d N=%d K=%d)", B, S, N, K);
    if (N > sd::kMaxTopkN || K > sd::kMaxTopkK)
        return fail(SD_ERR_UNSUPPORTED, "indexer_topk_bwd: N=%d and K=%d must be at most %d and %d", N, K,
                    sd::kMaxTopkN, sd::kMaxTopkK);
    int st = check_grid("indexer_topk_bwd", ((int64_t)B * S + 3) / 4, 256, "B*S must be below 2^26");
    if (st != SD_OK) return st;
    return hip_status(sd::launch_indexer_topk_bwd(dvalues, idx, B, S, N, K, dscores, stream),
                      "indexer_topk_bwd launch");
}

namespace {

// Shared checks of the compressor entry points (sizes, dtype, supported windows, alignment of
// the 16-byte vector accesses, grid size).
int check_compressor(const char *fn, int B, int S, int D, int ratio, int overlap, int dtype,
                     const void *const *ptrs, int nptrs) {
    if (dtype != SD_BF16 && dtype != SD_F32) return fail(SD_ERR_DTYPE, "%s: unknown dtype code %d", fn, dtype);
    if (B <= 0 || S <= 0 || D <= 0 || ratio <= 0 || (overlap != 0 && overlap != 1))
        return fail(SD_ERR_BAD_SHAPE, "%s: sizes must be positive and overlap 0 or 1 (B=%d S=%d D=%d ratio=%d "
                    "overlap=%d)", fn, B, S, D, ratio, overlap);
    if (S < ratio) return fail(SD_ERR_BAD_SHAPE, "%s: S=%d holds no complete block of %d tokens", fn, S, ratio);
    if (D % 4 != 0) return fail(SD_ERR_UNSUPPORTED, "%s: D=%d must be a multiple of 4", fn, D);
    if (!sd::compressor_supported(ratio, overlap))
        return fail(SD_ERR_UNSUPPORTED, "%s: ratio=%d with overlap=%d is not covered (powers of two up to 128 "
                    "without overlap, up to 16 with overlap)", fn, ratio, overlap);
    for (int i = 0; i < nptrs; ++i)
        if (ptrs[i] && (uintptr_t)ptrs[i] % 16 != 0)
            return fail(SD_ERR_BAD_SHAPE, "%s: array argument %d is not 16-byte aligned", fn, i);
    return check_grid(fn, ((int64_t)B * (S / ratio) * D + 255) / 256, 256, "B*(S/ratio)*D must be below 2^32");
}

}  // namespace

int compressor_pool(const void *kv, const void *score, const float *ape, const int32_t *seg, int B, int S, int D,
                    int ratio, int overlap, int dtype, float *pool, hipStream_t stream) {
    if (!kv || !score || !ape || !pool)
        return fail(SD_ERR_NULL_ARG, "compressor_pool: kv, score, ape and pool are required");
    const void *ptrs[] = {kv, score, ape, pool};
    int st = check_compressor("compressor_pool", B, S, D, ratio, overlap, dtype, ptrs, 4);
    if (st != SD_OK) return st;
    return hip_status(sd::launch_compressor_pool(kv, score, ape, seg, B, S, D, ratio, overlap, dtype, pool, stream),
                      "compressor_pool launch");
}

size_t compressor_pool_bwd_workspace_bytes(int B, int S, int D, int ratio, int overlap) {
    if (B <= 0 || S <= 0 || D <= 0 || ratio <= 0 || S < ratio || (overlap != 0 && overlap != 1)) return 0;
    return sd::compressor_bwd_workspace_bytes(B, S, D, ratio, overlap);
}

int compressor_pool_bwd(const void *kv, const void *score, const float *ape, const int32_t *seg, const float *dpool,
                        int B, int S, int D, int ratio, int overlap, int dtype, float *dkv, float *dscore, float *dape,
                        void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!kv || !score || !ape || !dpool || !dkv || !dscore || !dape || !workspace)
        return fail(SD_ERR_NULL_ARG, "compressor_pool_bwd: kv, score, ape, dpool, dkv, dscore, dape and workspace "
                    "are required");
    const void *ptrs[] = {kv, score, ape, dpool, dkv, dscore, dape, workspace};
    int st = check_compressor("compressor_pool_bwd", B, S, D, ratio, overlap, dtype, ptrs, 8);
    if (st != SD_OK) return st;
    const size_t need = sd::compressor_bwd_workspace_bytes(B, S, D, ratio, overlap);
    if (workspace_bytes < need)
        return fail(SD_ERR_BAD_SHAPE, "compressor_pool_bwd: workspace of %zu bytes, %zu needed", workspace_bytes, need);
    return hip_status(sd::launch_compressor_pool_bwd(kv, score, ape, seg, dpool, B, S, D, ratio, overlap, dtype, dkv,
                                                     dscore, dape, workspace, stream),
                      "compressor_pool_bwd launch");
}

int distill_kl_fwd_bwd_noalloc(const float *target, const float *logits, const int32_t *idx, int B, int S, int K,
                               int N, float grad_scale, float *kl_rows, float *dlogits, float *stats,
                               hipStream_t stream) {
    if (!target || !logits || !idx || !kl_rows || !stats)
        return fail(SD_ERR_NULL_ARG, "distill_kl_fwd_bwd_noalloc: target, logits, idx, kl_rows and stats are required");
    if (B <= 0 || S <= 0 || K <= 0 || N <= 0)
        return fail(SD_ERR_BAD_SHAPE, "distill_kl_fwd_bwd_noalloc: sizes must be positive (B=%d S=%d K=%d N=%d)", B, S,
                    K, N);
    if (K > sd::kMaxKlK)
        return fail(SD_ERR_UNSUPPORTED, "distill_kl_fwd_bwd_noalloc: K=%d exceeds %d", K, sd::kMaxKlK);
    if ((int64_t)B * S > sd::kNoAllocMaxRows)
        return fail(SD_ERR_UNSUPPORTED, "distill_kl_fwd_bwd_noalloc: B*S=%lld exceeds the %lld rows its fixed scratch "
                    "array holds; use distill_kl_fwd_bwd with a workspace", (long long)B * S,
                    (long long)sd::kNoAllocMaxRows);
    if (!isfinite(grad_scale)) return fail(SD_ERR_BAD_SHAPE, "distill_kl_fwd_bwd_noalloc: grad_scale must be finite");
    return hip_status(sd::launch_distill_kl_noalloc(target, logits, idx, B, S, K, N, grad_scale, kl_rows, dlogits,
                                                    stats, stream),
                      "distill_kl_fwd_bwd_noalloc launch");
}

}  // extern "C"
