/*
 * sparse_distill.h -- C ABI of the MI355X (gfx950) CSA indexer-distillation library
 * (libsparse_distill.so).
 *
 * The operations follow the DeepSeek-V4 compressed-sparse-attention (CSA) layer as the
 * Primus PR "perf(deepseek-v4): fuse and enable the indexer distillation loss"
 * describes it: one softmax per head over [sliding-window keys | top-k selected
 * compressed pool rows | per-head sink]; the indexer (student) is trained by
 * KL(target || softmax(indexer logits)) where the target is that softmax's
 * conditional on the selected rows, summed over heads and L1-renormalised.
 *
 * Conventions shared by every entry point
 *   - Every array argument is a DEVICE pointer owned by the caller, contiguous and
 *     row-major in the shape given; the library allocates no device memory and keeps
 *     no state beyond a thread-local error string.
 *   - Work is enqueued on `stream` (0 = the null stream) and returns without waiting:
 *     no host synchronisation, no device-to-host copy.  Launch errors are reported
 *     through the return status; a fault inside a kernel surfaces at the caller's next
 *     synchronisation.
 *   - Host-side validation runs before any HIP call.  A rejected call returns a
 *     non-zero status, enqueues nothing and sets sd_last_error().
 *   - Results are deterministic: every reduction has a fixed order.
 *   - A top-k slot k of row (b,t) is VALID iff 0 <= idx[b,t,k] < N.  -1 is the usual
 *     padding value (MaxText PR "Add Indexer Loss [Deepseek v4]", review comments:
 *     unused top-k slots hold -1); any other out-of-range value is treated the same.
 *     Causality and segment membership of idx are the caller's contract.
 *   - Element types of q / kwin / pool: SD_BF16 (bfloat16) or SD_F32 (float32); all
 *     other arrays are float32 or int32 as stated.  Arithmetic is fp32 with fp32
 *     accumulation of bf16 (or fp32) products.
 */
#ifndef SPARSE_DISTILL_H
#define SPARSE_DISTILL_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    SD_OK = 0,
    SD_ERR_NULL_ARG = 1,    /* a required pointer is NULL                         */
    SD_ERR_BAD_SHAPE = 2,   /* a size is non-positive or sizes are inconsistent     */
    SD_ERR_UNSUPPORTED = 3, /* valid request outside the shapes the kernels cover   */
    SD_ERR_DTYPE = 4,       /* unknown element-type code                           */
    SD_ERR_HIP = 5          /* the HIP runtime reported an error at launch          */
};

enum { SD_BF16 = 0, SD_F32 = 1 };

/*
 * window_lse -- log-mass of the non-compressed part of each head's joint softmax.
 *
 *   nc_lse[b,t,h] = log( sum_{j in win(t)} exp(scale * <q[b,t,h,:], kwin[b,j,:]>)
 *                        + exp(sink[h]) )
 *   win(t) = { j : max(0, t-W+1) <= j <= t  and  seg[b,j] == seg[b,t] }
 *
 * Defined by the Primus PR above, commit "fix: build the target from the layer's
 * joint softmax, add the sliding-window LSE kernel": the sliding-window plus sink
 * log-mass is carried into the target's denominator.  The window holds the W keys
 * ending at and including t; the sink is a raw per-head logit (not scaled).
 *
 *   q      [B,S,H,D]  dtype           queries (one row per token and head)
 *   kwin   [B,S,D]    dtype           sliding-window keys, shared by all heads
 *   sink   [H]        float32 or NULL per-head sink logit; NULL drops the term
 *   seg    [B,S]      int32 or NULL   packed-segment ids; NULL = one segment
 *   nc_lse [B,S,H]    float32 out     natural-log mass (never -inf: j = t is in win(t))
 * Limits: D % 32 == 0, D <= 512; H <= 64; 1 <= W <= 128; S * D * element size < 2^31
 * bytes (one batch row of kwin) and S <= 2^24 rows; S <= 2^24 - 2 (the grid has one
 * 512-lane workgroup per two tokens, and a dispatch counts at most 2^32 - 1 work-items).
 */
int window_lse(const void *q, const void *kwin, const float *sink, const int32_t *seg,
               int B, int S, int H, int D, int W, float scale, int dtype, float *nc_lse,
               hipStream_t stream);

/*
 * distill_target -- the KL target over each token's top-k compressed-pool rows.
 *
 *   c[h,k]   = scale * <q[b,t,h,:], pool[b, idx[b,t,k], :]>        for valid k
 *   full_h   = log( sum_{valid k} exp(c[h,k]) + exp(nc_lse[b,t,h]) )
 *   m_k      = sum_h exp(c[h,k] - full_h)
 *   target[b,t,k] = m_k / max(sum_{valid k} m_k, l1_floor)   (valid k);  exactly 0 otherwise
 *
 * Defined by the Primus PR above, PR body "Why the target was wrong" and the
 * joint-softmax commit: the target is the conditional, on the selected compressed
 * entries, of the layer's single softmax over window keys, compressed entries and
 * sink; the per-head share exp(compressed_lse - full_lse) is kept, heads are summed,
 * and the row is L1-renormalised with a float32-tiny floor.  The pool rows are read
 * through idx inside the kernel (commit "fuse the KL target and the KL tail into
 * Triton kernels": no gathered [B,S,K,D] tensor exists).
 *
 *   q      [B,S,H,D] dtype            queries
 *   pool   [B,N,D]   dtype            compressed rows, shared by all heads
 *   idx    [B,S,K]   int32            top-k pool rows; invalid slots as above
 *   nc_lse [B,S,H]   float32 or NULL  from window_lse; NULL = legacy per-branch target
 *                                     (each head renormalised over its compressed part)
 *   scale            softmax scale, positive and finite (1/sqrt(D) for the method)
 *   l1_floor         <= 0 selects FLT_MIN (2^-126); 1e-10 reproduces the legacy floor
 *   target [B,S,K]   float32 out      a row with no valid slot is all zeros
 * Limits: D % 32 == 0, D <= 512; H <= 64; K <= 1024; N * D * element size < 2^31 bytes
 * (one batch row of pool) and N <= 2^24 rows; B * S < 2^22 (one workgroup of up to 1024 lanes per token, and a
 * dispatch counts at most 2^32 - 1 work-items).  A non-positive or non-finite scale is rejected with
 * SD_ERR_BAD_SHAPE.
 */
int distill_target(const void *q, const void *pool, const int32_t *idx, const float *nc_lse,
                   int B, int S, int H, int D, int N, int K, float scale, float l1_floor,
                   int dtype, float *target, hipStream_t stream);

/*
 * distill_target_fused -- distill_target with its window part computed in the same pass.
 *
 *   nc_h   = log( sum_{j in win(t)} exp(scale * <q[b,t,h,:], kwin[b,j,:]>) + exp(sink[h]) )
 *   then exactly as distill_target with nc_lse = nc.
 *
 * The joint softmax runs over the window keys, the selected compressed rows and the sink
 * at once (the target defined by the Primus PR "perf(deepseek-v4): fuse and enable the
 * indexer distillation loss", body "Why the target was wrong", computed from the
 * attention's own entries), so the queries are read from HBM once for the whole target
 * instead of once by window_lse and once by distill_target.  win(t), sink and seg as in
 * window_lse; pool, idx, l1_floor and target as in distill_target.
 *
 *   nc_lse_out [B,S,H] float32 out or NULL: the window+sink LSE (what window_lse returns)
 * Limits: those of window_lse and distill_target together; scale positive and finite.
 */
int distill_target_fused(const void *q, const void *kwin, const float *sink, const int32_t *seg,
                         const void *pool, const int32_t *idx, int B, int S, int H, int D, int N,
                         int K, int W, float scale, float l1_floor, int dtype, float *target,
                         float *nc_lse_out, hipStream_t stream);

/*
 * distill_kl_fwd_bwd -- KL(target || softmax(logits)) per row, fused with its gradient.
 *
 *   V       = valid slots of the row;  lse = log sum_{k in V} exp(logits_k)
 *   kl_rows[b,t] = sum_{k in V, target_k > 0} target_k * (log target_k - logits_k + lse)
 *   dlogits[b,t,k] = grad_scale * ((sum_{j in V} target_j) * exp(logits_k - lse) - target_k)
 *                    for k in V;  exactly 0 for k not in V
 *   stats[0] = sum of kl_rows over rows with V non-empty;  stats[1] = number of such rows
 * A row with no valid slot gives kl 0 and gradient 0; logits at invalid slots are never
 * read into the arithmetic (they may hold NaN).  A row whose valid logits are all -inf
 * is outside the contract.
 *
 * Defined by the Primus PR above, commit "fuse the KL target and the KL tail into
 * Triton kernels" (KL(attention || indexer) with an analytic backward that saves
 * nothing beyond its inputs), and the MaxText PR "Add Indexer Loss [Deepseek v4]",
 * review comments (log-softmax KL without epsilon, exact gradient Q - P) and
 * Description (queries that see no completed block are shielded from the loss).
 * grad_scale carries the loss coefficient and the mean's 1/count.
 *
 *   target, logits [B,S,K] float32;  idx [B,S,K] int32 (validity only, 0 <= idx < N)
 *   kl_rows [B,S] float32 out;  dlogits [B,S,K] float32 out or NULL (forward only)
 *   stats [2] float32 out
 *   workspace: device scratch of distill_kl_workspace_bytes(B,S,K) bytes, 16-byte
 *   aligned, owned by the caller; its contents need no initialisation and are
 *   overwritten.  Calls that share a workspace must be ordered (same stream).
 * Limits: K <= 4096; B * S <= 2^24 (stats[1] is a float32 count, exact up to 2^24; larger
 * requests return SD_ERR_UNSUPPORTED).  Target values may be subnormal: log T is taken exactly
 * for every positive float32.
 */
size_t distill_kl_workspace_bytes(int B, int S, int K);
int distill_kl_fwd_bwd(const float *target, const float *logits, const int32_t *idx,
                       int B, int S, int K, int N, float grad_scale, float *kl_rows,
                       float *dlogits, float *stats, void *workspace, size_t workspace_bytes,
                       hipStream_t stream);

/*
 * indexer_topk -- the indexer's top-k block selection under the causal block mask and the
 * segment (packing) mask: the step that produces idx and the student logits of the KL.
 *
 *   block n covers tokens ratio*n .. ratio*n + ratio - 1 of its batch row; it is VISIBLE to
 *   token t iff n < N, ratio*n + ratio - 1 <= t (complete at t) and every one of its tokens
 *   carries seg[b,t]'s id (seg NULL: one segment).
 *   idx[b,t,:]    = the min(K, #visible) visible blocks with the largest scores[b,t,n], in
 *                   ascending block order, then -1.  Equal scores prefer the smaller block
 *                   index; a NaN score ranks below every number (-inf included).
 *   values[b,t,k] = scores[b,t,idx[b,t,k]];  -inf at a -1 slot
 *
 * Defined by the MaxText PR "Add Indexer Loss [Deepseek v4]": the indexer keeps the top-k
 * compressed blocks of each query, the teacher and the student share the causal block mask
 * combined with the segment/packing mask (commit list: no probability mass on future
 * blocks; for t = 4 block 0 is visible and block 1 is not, compress ratio 4), and the slots
 * it cannot fill become -1 (review comment on jnp.where(invalid, -1, top_k_indices)).  The
 * kept set is what distill_target and distill_kl_fwd_bwd use; its order within a row does
 * not change their results, and ascending block order is the one written here.
 *
 *   scores [B,S,N] float32       the student's per-(token, block) scores
 *   seg    [B,S]   int32 or NULL packed-segment ids
 *   idx    [B,S,K] int32 out;  values [B,S,K] float32 out or NULL
 * Limits: 1 <= N <= 4096; 1 <= K <= 4096; ratio >= 1; B * S < 2^26 (one 256-lane workgroup
 * per four rows).
 */
int indexer_topk(const float *scores, const int32_t *seg, int B, int S, int N, int K, int ratio,
                 int32_t *idx, float *values, hipStream_t stream);

/*
 * indexer_topk_bwd -- gradient of indexer_topk's values with respect to the scores: the
 * adjoint of the gather values[b,t,k] = scores[b,t,idx[b,t,k]].
 *
 *   dscores[b,t,n] = sum of dvalues[b,t,k] over the slots k with idx[b,t,k] == n, added in
 *                    slot order;  0 for every block no slot holds
 * A slot is valid iff 0 <= idx < N (-1 and out-of-range slots carry no gradient).  Slots
 * of one selection are distinct, so each kept block receives exactly its slot's gradient.
 *
 *   dvalues [B,S,K] float32;  idx [B,S,K] int32;  dscores [B,S,N] float32 out (all written)
 * Limits: 1 <= N <= 4096; 1 <= K <= 4096; B * S < 2^26.
 */
int indexer_topk_bwd(const float *dvalues, const int32_t *idx, int B, int S, int N, int K,
                     float *dscores, hipStream_t stream);

/*
 * compressor_pool -- the compressor that builds the compressed rows the target gathers.
 *
 *   Entry n (n < N = floor(S / ratio)) pools the Wc = ratio * (1 + overlap) tokens
 *   j = ratio*n - overlap*ratio + i, i < Wc, of its batch row: its own block, and with
 *   overlap the block before it too (position i is absent when j < 0, or when token j's
 *   segment differs from that of the entry's last token, ratio*n + ratio - 1):
 *     w_i        = softmax over the present i of (score[b,j,d] + ape[i,d]), per channel d
 *     pool[b,n,d] = sum_i w_i kv[b,j,d]
 *
 * Defined by the Primus PR "Docker Build for DeepSeek-v4 (Don't Merge)", commit fusing the
 * compressed-attention small kernels: score + ape, softmax over the window and the weighted
 * sum in one launch; HCA windows (overlap 0, e.g. ratio 128) do not overlap, CSA windows
 * (overlap 1, ratio 4) do.  ape carries one bias per window position and channel.
 *
 *   kv, score [B,S,D] dtype;  ape [Wc,D] float32;  seg [B,S] int32 or NULL
 *   pool [B,N,D] float32 out
 * Limits: D % 4 == 0; ratio a power of two, <= 128 without overlap, <= 16 with it; S >=
 * ratio; every array 16-byte aligned (SD_ERR_BAD_SHAPE otherwise); B * N * D < 2^32.
 */
int compressor_pool(const void *kv, const void *score, const float *ape, const int32_t *seg,
                    int B, int S, int D, int ratio, int overlap, int dtype, float *pool,
                    hipStream_t stream);

/*
 * compressor_pool_bwd -- the analytic backward of compressor_pool for an upstream dpool.
 *
 *   dkv[b,j,d]    = sum over the entries n holding j:  w dpool[b,n,d]
 *   dscore[b,j,d] = sum over the entries n holding j:  w (kv[b,j,d] - pool[b,n,d]) dpool[b,n,d]
 *   dape[i,d]     = sum over b and n of the same product at position i
 * (the softmax Jacobian applied to the kv-weighted gradient; same commit: "analytic
 * backward").  Tokens held by no entry (past N * ratio, or absent) get 0.  pool is
 * recomputed, not read.
 *
 *   dpool [B,N,D] float32;  dkv, dscore [B,S,D] float32 out;  dape [Wc,D] float32 out
 *   workspace: compressor_pool_bwd_workspace_bytes(B,S,D,ratio,overlap) bytes of caller
 *   device memory, 16-byte aligned; no initialisation needed; calls sharing it must be ordered.
 * Limits: those of compressor_pool.
 */
size_t compressor_pool_bwd_workspace_bytes(int B, int S, int D, int ratio, int overlap);
int compressor_pool_bwd(const void *kv, const void *score, const float *ape, const int32_t *seg,
                        const float *dpool, int B, int S, int D, int ratio, int overlap,
                        int dtype, float *dkv, float *dscore, float *dape, void *workspace,
                        size_t workspace_bytes, hipStream_t stream);

/*
 * distill_kl_fwd_bwd_noalloc -- distill_kl_fwd_bwd without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc.  Same arguments, results and limits as distill_kl_fwd_bwd
 * minus the workspace; the call allocates nothing.
 *
 * The per-block partial sums live in a fixed 2 MiB array of the library's device memory,
 * one per GPU, held until the process ends (its address is resolved on the first call on
 * each device).  Hence B * S <= 2^21 (larger requests return SD_ERR_UNSUPPORTED: use
 * distill_kl_fwd_bwd with a workspace).  Every call on a GPU uses that GPU's array and
 * overwrites what it reads, so calls ordered on one stream are fine, but calls that overlap
 * in time on one GPU (unordered streams, or other host threads) race on it.
 */
int distill_kl_fwd_bwd_noalloc(const float *target, const float *logits, const int32_t *idx,
                               int B, int S, int K, int N, float grad_scale, float *kl_rows,
                               float *dlogits, float *stats, hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char *sd_status_string(int status);
/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char *sd_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_DISTILL_H */
