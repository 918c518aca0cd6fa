/*
 * oracle.c -- plain fp64 CPU reference for the DeepSeek-V4 CSA indexer-distillation
 * path.  TEST INFRASTRUCTURE ONLY: the product path never links, loads or calls this
 * file.  Only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
 *
 * Sources (web pages, cited by title and section):
 *   [P1] Primus PR "perf(deepseek-v4): fuse and enable the indexer distillation loss"
 *        - commit "fix: build the target from the layer's joint softmax, add the
 *          sliding-window LSE kernel" and the PR body section "Why the target was
 *          wrong": the target is the conditional, on the selected compressed entries,
 *          of ONE softmax taken over [window keys | selected compressed entries | sink];
 *          heads are summed and the sum is L1-renormalised with a float32-tiny floor
 *          (the legacy floor was 1e-10, the legacy denominator the compressed part alone).
 *        - commit "fuse the KL target and the KL tail into Triton kernels": the KL tail
 *          KL(attention || indexer) has an analytic backward.
 *   [P3] MaxText PR "Add Indexer Loss [Deepseek v4]"
 *        - review comments: the loss is a log-softmax KL whose exact gradient is Q - P,
 *          masks are applied by boolean selection, -1 marks a padded top-k slot.
 *        - Description / commit list: queries that see no completed block produce no
 *          loss and no NaN.
 *
 * Everything is evaluated in double precision, written as the definition reads, with
 * no blocking, fusion or reordering: for each query row the explicit list of logits is
 * built, its log-sum-exp taken, and the probabilities formed.  Inputs arrive as fp32
 * arrays; bf16 and fp32 values convert to double exactly.
 *
 * Row selection: every function takes `rows` (flat b*S+t indices) and `nrows`; with
 * rows == NULL all B*S rows are computed in order.  Outputs are compact per selected
 * row (output row r corresponds to rows[r]).
 */
#include <float.h>
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Number of OpenMP threads the oracle will use (for reporting the CPU baseline). */
int oracle_num_threads(void) { return omp_get_max_threads(); }
void oracle_set_num_threads(int n) { if (n > 0) omp_set_num_threads(n); }

/* log(sum(exp(v[0..n)))) the textbook way, with the maximum factored out.
 * An empty list, or one holding only -inf, has log-mass -inf. */
static double logsumexp(const double *v, int n) {
    double m = -INFINITY;
    for (int i = 0; i < n; ++i)
        if (v[i] > m) m = v[i];
    if (m == -INFINITY) return -INFINITY;
    double s = 0.0;
    for (int i = 0; i < n; ++i) s += exp(v[i] - m);
    return m + log(s);
}

static double dot(const float *a, const float *b, int D) {
    double s = 0.0;
    for (int d = 0; d < D; ++d) s += (double)a[d] * (double)b[d];
    return s;
}

static int64_t row_of(const int64_t *rows, int64_t r) { return rows ? rows[r] : r; }

/* Does window key j belong to query t's sliding window?  The window is the W keys
 * ending at and including t, restricted to t's own packed segment (seg == NULL means
 * one segment).  [P1] sliding-window keys of the CSA layer; [P3] segment (packing)
 * mask combined with the causal mask. */
static int in_window(int64_t t, int64_t j, int W, const int32_t *seg_b) {
    if (j < 0 || j > t || j < t - W + 1) return 0;
    if (seg_b && seg_b[j] != seg_b[t]) return 0;
    return 1;
}

/* ----------------------------------------------------------------------------------
 * Non-compressed log-mass: nc_lse[b,t,h] = log( sum_{j in win(t)} exp(scale*<q,k_j>)
 *                                              + exp(sink[h]) )
 * [P1] commit adding the sliding-window LSE kernel: the mass of the window keys and the
 * per-head sink is what the joint denominator adds to the compressed part.  The sink is
 * a raw (unscaled) logit; sink == NULL drops that term.
 * out: [nrows, H] */
void oracle_window_lse(const float *q, const float *kwin, const float *sink,
                       const int32_t *seg, int B, int S, int H, int D, int W,
                       double scale, const int64_t *rows, int64_t nrows, double *out) {
    if (!rows) nrows = (int64_t)B * S;
    #pragma omp parallel
    {
        double *L = (double *)malloc(sizeof(double) * (size_t)(W + 2));
        #pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t row = row_of(rows, r);
            int64_t b = row / S, t = row % S;
            const int32_t *seg_b = seg ? seg + b * S : NULL;
            for (int h = 0; h < H; ++h) {
                const float *qh = q + ((row * H) + h) * (int64_t)D;
                int n = 0;
                for (int64_t j = t - W + 1; j <= t; ++j)
                    if (in_window(t, j, W, seg_b))
                        L[n++] = scale * dot(qh, kwin + (b * S + j) * (int64_t)D, D);
                if (sink) L[n++] = (double)sink[h];
                out[r * H + h] = logsumexp(L, n);
            }
        }
        free(L);
    }
}

/* ----------------------------------------------------------------------------------
 * KL target, the long way.  For query row (b,t):
 *   V   = { k : 0 <= idx[b,t,k] < N }            ([P3] -1 pads an unused top-k slot)
 *   c_hk = scale * <q[b,t,h], pool[b, idx[b,t,k]]>   for k in V
 *   for each head h, one joint list of logits:
 *       nc_lse != NULL : [ nc_lse[b,t,h] ] ++ [ c_hk : k in V ]
 *       otherwise      : [ window logits if kwin != NULL ] ++ [ sink[h] if sink ]
 *                        ++ [ c_hk : k in V ]
 *     full_h = log-sum-exp of that list,  p_hk = exp(c_hk - full_h)
 *   m_k = sum_h p_hk ;  T_k = m_k / max(sum_{k in V} m_k, floor) on V, 0 elsewhere.
 * floor <= 0 selects float32 tiny, 2^-126 ([P1]: the floor moved from 1e-10 to
 * float32 tiny).  With kwin == sink == nc_lse == NULL the list is the compressed part
 * alone, i.e. the legacy per-branch target ([P1] the previous behaviour; [P3] the
 * formula quoted in review, softmax per head over the compressed entries, summed and
 * L1-normalised).
 * outT: [nrows, K] */
void oracle_target(const float *q, const float *pool, const int32_t *idx,
                   const float *kwin, const float *sink, const int32_t *seg,
                   const double *nc_lse, int B, int S, int H, int D, int N, int K, int W,
                   double scale, double floor_, const int64_t *rows, int64_t nrows,
                   double *outT) {
    if (!rows) nrows = (int64_t)B * S;
    const double fl = floor_ > 0.0 ? floor_ : (double)FLT_MIN; /* FLT_MIN = 2^-126 */
    #pragma omp parallel
    {
        double *L = (double *)malloc(sizeof(double) * (size_t)(W + K + 2));
        double *c = (double *)malloc(sizeof(double) * (size_t)K);
        double *m = (double *)malloc(sizeof(double) * (size_t)K);
        #pragma omp for schedule(dynamic, 2)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t row = row_of(rows, r);
            int64_t b = row / S, t = row % S;
            const int32_t *id = idx + row * (int64_t)K;
            const int32_t *seg_b = seg ? seg + b * S : NULL;
            double *T = outT + r * (int64_t)K;
            for (int k = 0; k < K; ++k) m[k] = 0.0;
            int any = 0;
            for (int k = 0; k < K; ++k) any |= (id[k] >= 0 && id[k] < N);
            if (!any) {
                for (int k = 0; k < K; ++k) T[k] = 0.0;
                continue;
            }
            for (int h = 0; h < H; ++h) {
                const float *qh = q + ((row * H) + h) * (int64_t)D;
                int n = 0;
                if (nc_lse) {
                    L[n++] = nc_lse[r * H + h];
                } else {
                    if (kwin)
                        for (int64_t j = t - W + 1; j <= t; ++j)
                            if (in_window(t, j, W, seg_b))
                                L[n++] = scale * dot(qh, kwin + (b * S + j) * (int64_t)D, D);
                    if (sink) L[n++] = (double)sink[h];
                }
                for (int k = 0; k < K; ++k) {
                    if (id[k] >= 0 && id[k] < N) {
                        c[k] = scale * dot(qh, pool + (b * N + id[k]) * (int64_t)D, D);
                        L[n++] = c[k];
                    }
                }
                double full = logsumexp(L, n);
                for (int k = 0; k < K; ++k)
                    if (id[k] >= 0 && id[k] < N) m[k] += exp(c[k] - full);
            }
            double tot = 0.0;
            for (int k = 0; k < K; ++k)
                if (id[k] >= 0 && id[k] < N) tot += m[k];
            double den = tot > fl ? tot : fl;
            for (int k = 0; k < K; ++k)
                T[k] = (id[k] >= 0 && id[k] < N) ? m[k] / den : 0.0;
        }
        free(L);
        free(c);
        free(m);
    }
}

/* ----------------------------------------------------------------------------------
 * KL(target || softmax(student)) per row, with its exact gradient.
 *   V      = { k : 0 <= idx[b,t,k] < N }; the student softmax runs over V only.
 *   lse_z  = log-sum-exp_{k in V} z_k,   log Q_k = z_k - lse_z
 *   KL     = sum_{k in V, T_k > 0} T_k (log T_k - log Q_k)       (0 log 0 := 0)
 *   dKL/dz_k = (sum_{j in V} T_j) Q_k - T_k on V, 0 off V        ([P3] exact Q - P)
 * An empty row (V empty) has KL 0 and gradient 0.  dz is scaled by grad_scale.
 * kl_out: [nrows]; dz_out: [nrows, K] or NULL; stats[0] = sum of KL over selected
 * non-empty rows, stats[1] = their count.  ([P1] fused KL tail with analytic backward;
 * [P3] log-softmax KL with no epsilon, rows before the first completed block shielded.) */
void oracle_kl(const float *T, const float *z, const int32_t *idx, int B, int S, int K,
               int N, double grad_scale, const int64_t *rows, int64_t nrows,
               double *kl_out, double *dz_out, double *stats) {
    if (!rows) nrows = (int64_t)B * S;
    #pragma omp parallel
    {
        double *L = (double *)malloc(sizeof(double) * (size_t)K);
        #pragma omp for schedule(static)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t row = row_of(rows, r);
            const int32_t *id = idx + row * (int64_t)K;
            const float *Tr = T + row * (int64_t)K;
            const float *zr = z + row * (int64_t)K;
            int n = 0;
            double sumT = 0.0;
            for (int k = 0; k < K; ++k)
                if (id[k] >= 0 && id[k] < N) {
                    L[n++] = (double)zr[k];
                    sumT += (double)Tr[k];
                }
            if (n == 0) {
                kl_out[r] = 0.0;
                if (dz_out)
                    for (int k = 0; k < K; ++k) dz_out[r * (int64_t)K + k] = 0.0;
                continue;
            }
            double lse = logsumexp(L, n);
            double kl = 0.0;
            for (int k = 0; k < K; ++k) {
                int v = id[k] >= 0 && id[k] < N;
                double t = (double)Tr[k];
                double logq = (double)zr[k] - lse;
                if (v && t > 0.0) kl += t * (log(t) - logq);
                if (dz_out)
                    dz_out[r * (int64_t)K + k] = v ? grad_scale * (sumT * exp(logq) - t) : 0.0;
            }
            kl_out[r] = kl;
        }
        free(L);
    }
    double s = 0.0, cnt = 0.0;
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t row = row_of(rows, r);
        const int32_t *id = idx + row * (int64_t)K;
        int any = 0;
        for (int k = 0; k < K; ++k) any |= (id[k] >= 0 && id[k] < N);
        if (any) {
            s += kl_out[r];
            cnt += 1.0;
        }
    }
    stats[0] = s;
    stats[1] = cnt;
}

/* ----------------------------------------------------------------------------------
 * Indexer top-k selection, the step before the target ([P3] MaxText PR "Add Indexer Loss
 * [Deepseek v4]": the indexer keeps the top-k compressed blocks of each query under the
 * causal block mask combined with the segment (packing) mask -- commit list: "0.0
 * probability mass on all future blocks", "segment/packing mask"; the t=4 example: block 0
 * visible, block 1 masked -- and turns the slots it cannot fill into -1, review comment on
 * jnp.where(invalid, -1, top_k_indices)).
 *
 *   block n (tokens ratio*n .. ratio*n + ratio - 1) is visible to token t iff n < N, the
 *   block is complete at t (ratio*n + ratio - 1 <= t) and every one of its tokens carries
 *   t's segment id (seg == NULL: one segment).
 *   Among the visible blocks, the K with the largest score are kept; equal scores prefer
 *   the smaller block index; a NaN score ranks below every number.  The kept blocks are
 *   written in ascending block order, then -1 for the slots left over; values[k] is the
 *   kept block's score, -inf at a -1 slot.
 * out_idx, out_val: [nrows, K] */
typedef struct {
    float s;
    int32_t n;
} oracle_cand;

/* a before b in the selection order: larger score first, NaN last, then smaller index */
static int cand_rank_cmp(const void *pa, const void *pb) {
    const oracle_cand *a = (const oracle_cand *)pa, *b = (const oracle_cand *)pb;
    const int na = isnan(a->s), nb = isnan(b->s);
    if (na != nb) return na ? 1 : -1;
    if (!na && a->s != b->s) return a->s > b->s ? -1 : 1;
    return a->n < b->n ? -1 : (a->n > b->n ? 1 : 0);
}

static int cand_index_cmp(const void *pa, const void *pb) {
    const oracle_cand *a = (const oracle_cand *)pa, *b = (const oracle_cand *)pb;
    return a->n < b->n ? -1 : (a->n > b->n ? 1 : 0);
}

void oracle_indexer_topk(const float *scores, const int32_t *seg, int B, int S, int N, int K,
                         int ratio, const int64_t *rows, int64_t nrows, int32_t *out_idx,
                         float *out_val) {
    if (!rows) nrows = (int64_t)B * S;
    #pragma omp parallel
    {
        oracle_cand *c = (oracle_cand *)malloc(sizeof(oracle_cand) * (size_t)(N > 0 ? N : 1));
        #pragma omp for schedule(dynamic, 8)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t row = row_of(rows, r);
            int64_t b = row / S, t = row % S;
            const float *sc = scores + row * (int64_t)N;
            int m = 0;
            for (int n = 0; n < N; ++n) {
                int64_t last = (int64_t)ratio * n + ratio - 1;
                if (last > t) continue;                       /* not complete at t (causal) */
                int same = 1;
                if (seg)
                    for (int64_t j = (int64_t)ratio * n; j <= last; ++j)
                        if (seg[b * S + j] != seg[b * S + t]) same = 0;
                if (!same) continue;                          /* another document's block */
                c[m].s = sc[n];
                c[m].n = n;
                ++m;
            }
            qsort(c, (size_t)m, sizeof(oracle_cand), cand_rank_cmp);
            int kept = m < K ? m : K;
            qsort(c, (size_t)kept, sizeof(oracle_cand), cand_index_cmp);
            for (int k = 0; k < K; ++k) {
                out_idx[r * (int64_t)K + k] = k < kept ? c[k].n : -1;
                out_val[r * (int64_t)K + k] = k < kept ? c[k].s : -INFINITY;
            }
        }
        free(c);
    }
}

/* Gradient of the selection's values with respect to the block scores: the adjoint of the
 * gather values[k] = scores[idx[k]] (valid slots, 0 <= idx < N).  Each block receives the
 * gradients of the slots that hold it, added in slot order; every other entry is 0.
 * out: [nrows, N] */
void oracle_indexer_topk_bwd(const float *dval, const int32_t *idx, int B, int S, int N, int K,
                             const int64_t *rows, int64_t nrows, double *out) {
    if (!rows) nrows = (int64_t)B * S;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t row = row_of(rows, r);
        double *o = out + r * (int64_t)N;
        for (int n = 0; n < N; ++n) o[n] = 0.0;
        for (int k = 0; k < K; ++k) {
            int32_t n = idx[row * (int64_t)K + k];
            if (n >= 0 && n < N) o[n] += (double)dval[row * (int64_t)K + k];
        }
    }
}

/* ----------------------------------------------------------------------------------
 * Compressor pool, the step that builds the compressed rows ([P2] Primus PR "Docker Build
 * for DeepSeek-v4 (Don't Merge)", commit fusing the compressed-attention small kernels:
 * compressor_pool fuses score+ape, a softmax over the window and the weighted sum, with an
 * analytic backward for kv, score and ape; HCA windows do not overlap, CSA windows do).
 *
 * Readings (the page gives the steps, not the shapes):
 *   kv, score: [B,S,D] per-token values and compression logits; ape: [Wc,D], a learned
 *   bias per window position and channel; ratio r; entry n (n < N = floor(S/r)) pools
 *     HCA (overlap 0): tokens r*n .. r*n + r - 1                     (Wc = r)
 *     CSA (overlap 1): tokens r*(n-1) .. r*n + r - 1, its own block and the one before
 *                      (Wc = 2r; positions before token 0 are absent)
 *   position i of entry n is token j = r*n - overlap*r + i; it is present iff j >= 0 and
 *   seg[j] equals the segment of the entry's last token (seg == NULL: one segment).
 *   For each channel d, over the present positions:
 *     w_i = softmax_i(score[j_i,d] + ape[i,d]);   pool[n,d] = sum_i w_i kv[j_i,d]
 * out pool: [B,N,D] */
static int cp_token(int n, int i, int r, int overlap) { return r * n - overlap * r + i; }

static int cp_present(const int32_t *seg_b, int S, int n, int i, int r, int overlap) {
    int j = cp_token(n, i, r, overlap);
    if (j < 0 || j >= S) return 0;
    if (seg_b && seg_b[j] != seg_b[r * n + r - 1]) return 0;
    return 1;
}

void oracle_compressor_pool(const float *kv, const float *score, const float *ape, const int32_t *seg,
                            int B, int S, int D, int r, int overlap, double *pool) {
    const int N = S / r, Wc = r * (1 + overlap);
    #pragma omp parallel
    {
        double *l = (double *)malloc(sizeof(double) * (size_t)Wc);
        #pragma omp for schedule(static)
        for (int64_t bn = 0; bn < (int64_t)B * N; ++bn) {
            int64_t b = bn / N;
            int n = (int)(bn % N);
            const int32_t *seg_b = seg ? seg + b * S : NULL;
            for (int d = 0; d < D; ++d) {
                double m = -INFINITY;
                for (int i = 0; i < Wc; ++i) {
                    if (!cp_present(seg_b, S, n, i, r, overlap)) continue;
                    int64_t j = cp_token(n, i, r, overlap);
                    l[i] = (double)score[(b * S + j) * D + d] + (double)ape[(int64_t)i * D + d];
                    if (l[i] > m) m = l[i];
                }
                double den = 0.0, num = 0.0;
                for (int i = 0; i < Wc; ++i) {
                    if (!cp_present(seg_b, S, n, i, r, overlap)) continue;
                    int64_t j = cp_token(n, i, r, overlap);
                    double e = exp(l[i] - m);
                    den += e;
                    num += e * (double)kv[(b * S + j) * D + d];
                }
                pool[bn * D + d] = num / den;
            }
        }
        free(l);
    }
}

/* Analytic backward of oracle_compressor_pool for an upstream gradient dpool [B,N,D]:
 *   dkv[j,d]    = sum over entries n containing j:  w_{n,i(j),d} dpool[n,d]
 *   dscore[j,d] = sum over entries n containing j:  w_{n,i(j),d} (kv[j,d] - pool[n,d]) dpool[n,d]
 *   dape[i,d]   = sum over b and n with position i present: the same product
 * (the softmax Jacobian diag(w) - w w^T applied to the kv-weighted gradient).  Tokens in no
 * entry (the tail past N*r, or absent positions) get 0.
 * out dkv, dscore: [B,S,D]; dape: [Wc,D] */
void oracle_compressor_pool_bwd(const float *kv, const float *score, const float *ape, const int32_t *seg,
                                const float *dpool, int B, int S, int D, int r, int overlap,
                                double *dkv, double *dscore, double *dape) {
    const int N = S / r, Wc = r * (1 + overlap);
    for (int64_t x = 0; x < (int64_t)B * S * D; ++x) dkv[x] = dscore[x] = 0.0;
    for (int64_t x = 0; x < (int64_t)Wc * D; ++x) dape[x] = 0.0;
    double *w = (double *)malloc(sizeof(double) * (size_t)Wc);
    /* sequential over entries: several entries add into the same token and position */
    for (int64_t b = 0; b < B; ++b) {
        const int32_t *seg_b = seg ? seg + b * S : NULL;
        for (int n = 0; n < N; ++n) {
            for (int d = 0; d < D; ++d) {
                double m = -INFINITY;
                for (int i = 0; i < Wc; ++i) {
                    if (!cp_present(seg_b, S, n, i, r, overlap)) continue;
                    int64_t j = cp_token(n, i, r, overlap);
                    w[i] = (double)score[(b * S + j) * D + d] + (double)ape[(int64_t)i * D + d];
                    if (w[i] > m) m = w[i];
                }
                double den = 0.0;
                for (int i = 0; i < Wc; ++i)
                    if (cp_present(seg_b, S, n, i, r, overlap)) den += exp(w[i] - m);
                double p = 0.0;
                for (int i = 0; i < Wc; ++i) {
                    if (!cp_present(seg_b, S, n, i, r, overlap)) continue;
                    int64_t j = cp_token(n, i, r, overlap);
                    w[i] = exp(w[i] - m) / den;
                    p += w[i] * (double)kv[(b * S + j) * D + d];
                }
                double g = (double)dpool[(b * N + n) * (int64_t)D + d];
                for (int i = 0; i < Wc; ++i) {
                    if (!cp_present(seg_b, S, n, i, r, overlap)) continue;
                    int64_t j = cp_token(n, i, r, overlap);
                    double kvj = (double)kv[(b * S + j) * D + d];
                    dkv[(b * S + j) * D + d] += w[i] * g;
                    dscore[(b * S + j) * D + d] += w[i] * (kvj - p) * g;
                    dape[(int64_t)i * D + d] += w[i] * (kvj - p) * g;
                }
            }
        }
    }
    free(w);
}
