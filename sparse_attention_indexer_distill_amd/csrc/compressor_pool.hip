// compressor_pool.hip -- the compressor that builds the compressed pool rows, on gfx950.
//
// Primus PR "Docker Build for DeepSeek-v4 (Don't Merge)", commit fusing the compressed-
// attention small kernels: score + ape, a softmax over the window and the weighted sum in
// one launch, with an analytic backward for kv, score and ape; HCA windows do not overlap,
// CSA windows do.  Entry n pools the tokens j = r*n - OVL*r + i, i < Wc = r*(1+OVL), of its
// batch row (positions before token 0, or whose token lies in another segment than the
// entry's last token, are absent):
//     w_i = softmax_i(score[j,d] + ape[i,d]) per channel d,   pool[n,d] = sum_i w_i kv[j,d]
// Backward for dpool:
//     dkv[j,d]    = sum over entries holding j of w dpool
//     dscore[j,d] = sum over entries holding j of w (kv[j,d] - pool[n,d]) dpool
//     dape[i,d]   = sum over b, n of the same product at position i
//
// The work is a stream over kv and score (HBM-bound; every token row is read by one or two
// entries, the second time from L2).  Forward: one thread per (entry, CPT consecutive
// channels), a softmax in exp2 form over the window (all positions in registers for windows
// of up to 16, an online pass for larger ones).  Backward: one thread per
// (chunk of kChunk entries, CPT channels), 64 channel groups to a wave and kBwdWaves
// consecutive chunks to a workgroup; for every window it recomputes the weights and the
// pooled value, then writes each block's dkv and dscore once (with overlap a block takes
// contributions from two windows, so a chunk also recomputes the first window of the next
// chunk) and accumulates dape for its own windows in registers.  Small windows (KEEP) request
// all of the chunk's tokens, dpool rows and ape rows up front and keep them in registers, so
// each weight costs one exp2 and no token is loaded twice by a thread; large windows make an
// online pass and a second pass that reloads.  The workgroup's waves add their dape in LDS in
// a fixed order, and a second kernel adds the per-workgroup partials in a fixed order, so
// every result is bitwise repeatable.
#include "sd_device.hpp"
#include "sd_internal.hpp"

namespace sd {
namespace {

constexpr int kChunk = 1;        // entries per backward thread
constexpr int kPoolThreads = 256;
constexpr int kBwdWaves = 8;     // chunks per backward workgroup, one wave each

// CPT consecutive channels of one row (bf16 or fp32) as fp32.
template <int DT, int CPT>
__device__ __forceinline__ void load_ch(const void *base, int64_t elem, float (&o)[CPT]) {
    if constexpr (DT == 0) {
        const uint16_t *p = reinterpret_cast<const uint16_t *>(base) + elem;
        if constexpr (CPT == 4) {
            const uint2 v = *reinterpret_cast<const uint2 *>(p);
            o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
            o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
        } else if constexpr (CPT == 2) {
            const uint32_t v = *reinterpret_cast<const uint32_t *>(p);
            o[0] = __uint_as_float(v << 16); o[1] = __uint_as_float(v & 0xffff0000u);
        } else {
            o[0] = __uint_as_float((uint32_t)p[0] << 16);
        }
    } else {
        const float *p = reinterpret_cast<const float *>(base) + elem;
        if constexpr (CPT == 4) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(p);
            o[0] = v[0]; o[1] = v[1]; o[2] = v[2]; o[3] = v[3];
        } else {
#pragma unroll
            for (int c = 0; c < CPT; ++c) o[c] = p[c];
        }
    }
}

template <int CPT>
__device__ __forceinline__ void load_f32(const float *p, float (&o)[CPT]) {
    if constexpr (CPT == 4) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(p);
        o[0] = v[0]; o[1] = v[1]; o[2] = v[2]; o[3] = v[3];
    } else {
#pragma unroll
        for (int c = 0; c < CPT; ++c) o[c] = p[c];
    }
}

// Output rows are written once and not read again by the kernel: streaming (non-temporal)
// stores, which measured faster than ordinary ones for the gradient rows.
typedef float f32x2 __attribute__((ext_vector_type(2)));
template <int CPT>
__device__ __forceinline__ void store_f32(float *p, const float (&v)[CPT]) {
    if constexpr (CPT == 4) {
        __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4 *>(p));
    } else if constexpr (CPT == 2) {
        __builtin_nontemporal_store(f32x2{v[0], v[1]}, reinterpret_cast<f32x2 *>(p));
    } else {
#pragma unroll
        for (int c = 0; c < CPT; ++c) p[c] = v[c];
    }
}

struct PoolArgs {
    const void *kv, *score;
    const float *ape;
    const int32_t *seg;
    const float *dpool;
    float *pool, *dkv, *dscore, *dape_part, *dape;
    int B, S, D, N, nchunk, ncb;  // ncb: workgroups of kBwdWaves chunks per batch row
};

// Is position i of entry n present (token inside the row, same segment as the entry's last)?
template <int R, int OVL>
__device__ __forceinline__ bool present(const int32_t *sg, int n, int i, int32_t seg_last) {
    const int j = R * n - OVL * R + i;
    return j >= 0 && (sg == nullptr || sg[j] == seg_last);
}

template <int DT, int R, int OVL, int CPT>
__global__ __launch_bounds__(kPoolThreads) void compressor_pool_kernel(const PoolArgs a) {
    constexpr int Wc = R * (1 + OVL);
    const int G = a.D / CPT;
    const int64_t tid = (int64_t)blockIdx.x * kPoolThreads + threadIdx.x;
    if (tid >= (int64_t)a.B * a.N * G) return;
    const int g = (int)(tid % G);
    const int64_t bn = tid / G;
    const int n = (int)(bn % a.N);
    const int64_t b = bn / a.N;
    const int d0 = g * CPT;
    const int32_t *sg = a.seg ? a.seg + b * a.S : nullptr;
    const int32_t seg_last = sg ? sg[R * n + R - 1] : 0;
    if constexpr (Wc <= 16) {
        // Small windows: every position's loads are issued at once (absent positions read a
        // clamped row whose values are replaced), then the maximum, the exponentials and the sums.
        float l[Wc][CPT], k[Wc][CPT];
#pragma unroll
        for (int i = 0; i < Wc; ++i) {
            const int j = R * n - OVL * R + i;
            const bool pr = present<R, OVL>(sg, n, i, seg_last);
            const int64_t row = b * a.S + (j > 0 ? j : 0);
            float s[CPT], ap[CPT];
            load_ch<DT, CPT>(a.score, row * a.D + d0, s);
            load_ch<DT, CPT>(a.kv, row * a.D + d0, k[i]);
            load_f32<CPT>(a.ape + (int64_t)i * a.D + d0, ap);
#pragma unroll
            for (int c = 0; c < CPT; ++c) {  // an absent row's values never reach the sums, NaN included
                l[i][c] = pr ? (s[c] + ap[c]) * kLog2e : -INFINITY;
                k[i][c] = pr ? k[i][c] : 0.f;
            }
        }
        float out[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            float m = l[Wc - 1][c];  // the entry's last token is always present
#pragma unroll
            for (int i = 0; i < Wc - 1; ++i) m = fmaxf(m, l[i][c]);
            float den = 0.f, num = 0.f;
#pragma unroll
            for (int i = 0; i < Wc; ++i) {
                const float e = fast_exp2(l[i][c] - m);  // 0 at absent positions
                den += e;
                num = fmaf(e, k[i][c], num);
            }
            out[c] = num / den;
        }
        store_f32<CPT>(a.pool + bn * a.D + d0, out);
        return;
    }
    float m[CPT], den[CPT], num[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        m[c] = -INFINITY;
        den[c] = 0.f;
        num[c] = 0.f;
    }
#pragma unroll 8
    for (int i = 0; i < Wc; ++i) {
        if (!present<R, OVL>(sg, n, i, seg_last)) continue;
        const int64_t row = b * a.S + (R * n - OVL * R + i);
        float s[CPT], k[CPT], ap[CPT];
        load_ch<DT, CPT>(a.score, row * a.D + d0, s);
        load_ch<DT, CPT>(a.kv, row * a.D + d0, k);
        load_f32<CPT>(a.ape + (int64_t)i * a.D + d0, ap);
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const float l = (s[c] + ap[c]) * kLog2e;
            if (l > m[c]) {                       // new running maximum: rescale the sums
                const float f = fast_exp2(m[c] - l);
                den[c] *= f;
                num[c] *= f;
                m[c] = l;
            }
            const float e = fast_exp2(l - m[c]);
            den[c] += e;
            num[c] = fmaf(e, k[c], num[c]);
        }
    }
    float out[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) out[c] = num[c] / den[c];   // the entry's last token is always present
    store_f32<CPT>(a.pool + bn * a.D + d0, out);
}

// Statistics of window n for CPT channels in one online pass: the log2-domain maximum m, the
// sum of exponentials den and the pooled value.
template <int DT, int R, int OVL, int CPT>
__device__ __forceinline__ void window_stats(const PoolArgs &a, const int32_t *sg, int64_t b, int n, int d0,
                                             int32_t seg_last, float (&m)[CPT], float (&den)[CPT],
                                             float (&pool)[CPT]) {
    constexpr int Wc = R * (1 + OVL);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        m[c] = -INFINITY;
        den[c] = 0.f;
        pool[c] = 0.f;
    }
#pragma unroll(Wc <= 16 ? Wc : 8)
    for (int i = 0; i < Wc; ++i) {
        if (!present<R, OVL>(sg, n, i, seg_last)) continue;
        const int64_t row = b * a.S + (R * n - OVL * R + i);
        float s[CPT], k[CPT], ap[CPT];
        load_ch<DT, CPT>(a.score, row * a.D + d0, s);
        load_ch<DT, CPT>(a.kv, row * a.D + d0, k);
        load_f32<CPT>(a.ape + (int64_t)i * a.D + d0, ap);
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const float l = (s[c] + ap[c]) * kLog2e;
            if (l > m[c]) {
                const float f = fast_exp2(m[c] - l);
                den[c] *= f;
                pool[c] *= f;
                m[c] = l;
            }
            const float e = fast_exp2(l - m[c]);
            den[c] += e;
            pool[c] = fmaf(e, k[c], pool[c]);
        }
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) pool[c] /= den[c];
}

// grid: (ceil(G / 64), B * ncb); lane -> channel group, wave -> chunk
template <int DT, int R, int OVL, int CPT>
__global__ __launch_bounds__(kBwdWaves * 64) void compressor_pool_bwd_kernel(const PoolArgs a) {
    constexpr int Wc = R * (1 + OVL);
    constexpr bool KEEP = Wc * CPT <= 16;                   // the chunk's tokens held in registers
    constexpr int NB = kChunk + 1 + OVL;                    // KEEP: token blocks a chunk reads
    constexpr int SL = Wc * CPT <= 32 ? Wc : (32 / CPT);   // positions per LDS reduction slice
    __shared__ float red[kBwdWaves][SL][64 * CPT];
    const int G = a.D / CPT;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int g = blockIdx.x * 64 + lane;
    const int64_t b = blockIdx.y / a.ncb;
    const int cb = (int)(blockIdx.y - b * a.ncb);
    const int chunk = cb * kBwdWaves + w;
    const bool active = g < G && chunk < a.nchunk;   // inactive lanes still meet the barriers below
    const int d0 = (g < G ? g : 0) * CPT;
    const int32_t *sg = a.seg ? a.seg + b * a.S : nullptr;
    const int n0 = chunk * kChunk;
    const int n_own_end = !active ? n0 : (n0 + kChunk < a.N ? n0 + kChunk : a.N);   // windows [n0, n_own_end)
    // with overlap, block n_own_end - 1 also takes a contribution from window n_own_end
    const int n_last = !active ? n0 - 1 : (OVL && n_own_end < a.N ? n_own_end : n_own_end - 1);

    float dape_acc[KEEP ? Wc : 1][CPT];  // KEEP: this thread's dape (large windows reduce in LDS as they go)
#pragma unroll
    for (int i = 0; i < (KEEP ? Wc : 1); ++i)
#pragma unroll
        for (int c = 0; c < CPT; ++c) dape_acc[i][c] = 0.f;
    float carry_g[OVL ? R : 1][CPT], carry_h[OVL ? R : 1][CPT];  // block n's share from window n (overlap)

    // dkv/dscore of window n at position i (token j), written once complete (with overlap a
    // block's first share is carried).
    auto emit = [&](int n, int i, int j, bool own, const float (&gv)[CPT], const float (&hv)[CPT]) {
        if constexpr (OVL == 0) {
            const int64_t o = (b * a.S + j) * a.D + d0;
            store_f32<CPT>(a.dkv + o, gv);
            store_f32<CPT>(a.dscore + o, hv);
        } else if (i < R) {
            // the previous block: complete it when this thread owns it (window n-1 was its first share)
            if (n - 1 >= n0 && j >= 0) {
                float g2[CPT], h2[CPT];
#pragma unroll
                for (int c = 0; c < CPT; ++c) {
                    g2[c] = carry_g[i][c] + gv[c];
                    h2[c] = carry_h[i][c] + hv[c];
                }
                const int64_t o = (b * a.S + j) * a.D + d0;
                store_f32<CPT>(a.dkv + o, g2);
                store_f32<CPT>(a.dscore + o, h2);
            }
        } else if (own) {
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                carry_g[i - R][c] = gv[c];
                carry_h[i - R][c] = hv[c];
            }
        }
    };

    if constexpr (KEEP) {
        // Every token, dpool row and ape row the chunk needs is requested before any is used:
        // blocks n0 - OVL .. n0 + kChunk (token t of block n0 - OVL + u at index R*u + t).
        float ts[KEEP ? NB * R : 1][CPT], tk[KEEP ? NB * R : 1][CPT], tap[KEEP ? Wc : 1][CPT], dps[kChunk + 1][CPT];
#pragma unroll
        for (int u = 0; u < NB * R; ++u) {
            const int j = R * (n0 - OVL) + u;
            if (active && j >= 0 && j < R * (n_last + 1)) {
                const int64_t row = b * a.S + j;
                load_ch<DT, CPT>(a.score, row * a.D + d0, ts[u]);
                load_ch<DT, CPT>(a.kv, row * a.D + d0, tk[u]);
            } else {
#pragma unroll
                for (int c = 0; c < CPT; ++c) ts[u][c] = tk[u][c] = 0.f;
            }
        }
#pragma unroll
        for (int q = 0; q <= kChunk; ++q) {
            if (n0 + q <= n_last) {
                load_f32<CPT>(a.dpool + (b * a.N + n0 + q) * a.D + d0, dps[q]);
            } else {
#pragma unroll
                for (int c = 0; c < CPT; ++c) dps[q][c] = 0.f;
            }
        }
#pragma unroll
        for (int i = 0; i < Wc; ++i) load_f32<CPT>(a.ape + (int64_t)i * a.D + d0, tap[i]);

#pragma unroll
        for (int q = 0; q <= kChunk; ++q) {
            const int n = n0 + q;
            if (n > n_last) break;
            const int32_t seg_last = sg ? sg[R * n + R - 1] : 0;
            bool pr[Wc];    // uniform over the wave
            float e[Wc][CPT], m[CPT], den[CPT], pool[CPT];
#pragma unroll
            for (int c = 0; c < CPT; ++c) m[c] = -INFINITY;
#pragma unroll
            for (int i = 0; i < Wc; ++i) {
                pr[i] = present<R, OVL>(sg, n, i, seg_last);
#pragma unroll
                for (int c = 0; c < CPT; ++c) {
                    e[i][c] = (ts[R * q + i][c] + tap[i][c]) * kLog2e;
                    if (pr[i]) m[c] = fmaxf(m[c], e[i][c]);
                }
            }
#pragma unroll
            for (int c = 0; c < CPT; ++c) den[c] = pool[c] = 0.f;
#pragma unroll
            for (int i = 0; i < Wc; ++i) {
                if (!pr[i]) continue;  // absent positions take no part, whatever their values
#pragma unroll
                for (int c = 0; c < CPT; ++c) {  // the entry's last token is present, so m is finite
                    e[i][c] = fast_exp2(e[i][c] - m[c]);
                    den[c] += e[i][c];
                    pool[c] = fmaf(e[i][c], tk[R * q + i][c], pool[c]);
                }
            }
            float gsc[CPT];  // dpool / den: the weight of position i is e_i / den
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                const float rden = 1.f / den[c];
                pool[c] *= rden;
                gsc[c] = dps[q][c] * rden;
            }
            const bool own = n < n_own_end;
#pragma unroll
            for (int i = 0; i < Wc; ++i) {
                float gv[CPT], hv[CPT];
#pragma unroll
                for (int c = 0; c < CPT; ++c) {
                    gv[c] = pr[i] ? e[i][c] * gsc[c] : 0.f;
                    hv[c] = pr[i] ? gv[c] * (tk[R * q + i][c] - pool[c]) : 0.f;
                }
                if (own) {
#pragma unroll
                    for (int c = 0; c < CPT; ++c) dape_acc[KEEP ? i : 0][c] += hv[c];
                }
                emit(n, i, R * n - OVL * R + i, own, gv, hv);
            }
        }
    } else {
        // Large windows, one own window per thread (kChunk == 1): an online pass for the
        // statistics, then the gradient pass reloads each position; the own window's dape goes
        // to LDS slice by slice and is reduced over the workgroup at once (no per-position
        // accumulators).  With overlap, window n0 + 1 then completes block n0.
        static_assert(kChunk == 1, "large windows reduce one own window per thread");
        auto grad = [&](bool live, int n, int i, int32_t seg_last, const float (&m)[CPT], const float (&den)[CPT],
                        const float (&pool)[CPT], const float (&dp)[CPT], float (&gv)[CPT], float (&hv)[CPT]) {
            const bool pres = live && present<R, OVL>(sg, n, i, seg_last);
            float sc[CPT] = {}, k[CPT] = {}, ap[CPT] = {};
            if (pres) {
                const int64_t row = b * a.S + (R * n - OVL * R + i);
                load_ch<DT, CPT>(a.score, row * a.D + d0, sc);
                load_ch<DT, CPT>(a.kv, row * a.D + d0, k);
                load_f32<CPT>(a.ape + (int64_t)i * a.D + d0, ap);
            }
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                const float g = fast_exp2((sc[c] + ap[c]) * kLog2e - m[c]) / den[c] * dp[c];
                gv[c] = pres ? g : 0.f;
                hv[c] = pres ? g * (k[c] - pool[c]) : 0.f;
            }
        };
        float m[CPT] = {}, den[CPT] = {}, pool[CPT] = {}, dp[CPT] = {};
        int32_t seg_last = 0;
        if (active) {
            seg_last = sg ? sg[R * n0 + R - 1] : 0;
            window_stats<DT, R, OVL, CPT>(a, sg, b, n0, d0, seg_last, m, den, pool);
            load_f32<CPT>(a.dpool + (b * a.N + n0) * a.D + d0, dp);
        }
        float *part = a.dape_part + (int64_t)blockIdx.y * Wc * a.D;
        for (int i0 = 0; i0 < Wc; i0 += SL) {
#pragma unroll
            for (int ii = 0; ii < SL; ++ii) {
                float gv[CPT], hv[CPT];
                grad(active, n0, i0 + ii, seg_last, m, den, pool, dp, gv, hv);
                if (active) emit(n0, i0 + ii, R * n0 - OVL * R + i0 + ii, true, gv, hv);
#pragma unroll
                for (int c = 0; c < CPT; ++c) red[w][ii][lane * CPT + c] = hv[c];
            }
            __syncthreads();
            for (int e = threadIdx.x; e < SL * 64 * CPT; e += kBwdWaves * 64) {
                const int ii = e / (64 * CPT), x = e - ii * (64 * CPT);
                const int d = blockIdx.x * 64 * CPT + x;
                if (d < a.D) {
                    float v = red[0][ii][x];
#pragma unroll
                    for (int u = 1; u < kBwdWaves; ++u) v += red[u][ii][x];
                    part[(int64_t)(i0 + ii) * a.D + d] = v;
                }
            }
            __syncthreads();
        }
        if (OVL && active && n_last > n0) {  // window n0 + 1: its first R positions complete block n0
            const int n = n0 + 1;
            const int32_t sl = sg ? sg[R * n + R - 1] : 0;
            float m1[CPT], den1[CPT], pool1[CPT], dp1[CPT];
            window_stats<DT, R, OVL, CPT>(a, sg, b, n, d0, sl, m1, den1, pool1);
            load_f32<CPT>(a.dpool + (b * a.N + n) * a.D + d0, dp1);
#pragma unroll
            for (int i = 0; i < R; ++i) {
                float gv[CPT], hv[CPT];
                grad(true, n, i, sl, m1, den1, pool1, dp1, gv, hv);
                emit(n, i, R * n - OVL * R + i, false, gv, hv);
            }
        }
    }
    if constexpr (OVL == 1) {
        if (active && n_own_end == a.N) {  // the last block has no later window
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const int64_t o = (b * a.S + (int64_t)R * (a.N - 1) + i) * a.D + d0;
                store_f32<CPT>(a.dkv + o, carry_g[i]);
                store_f32<CPT>(a.dscore + o, carry_h[i]);
            }
        }
    }
    if (active && n_own_end == a.N) {      // tokens past the last entry are in no window
        float z[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) z[c] = 0.f;
        for (int j = R * a.N; j < a.S; ++j) {
            const int64_t o = (b * a.S + j) * a.D + d0;
            store_f32<CPT>(a.dkv + o, z);
            store_f32<CPT>(a.dscore + o, z);
        }
    }
    // KEEP: the workgroup's dape, its waves (chunks) added in order, one slice of positions at
    // a time (large windows have done this above)
    if constexpr (!KEEP) return;
    float *part = a.dape_part + (int64_t)blockIdx.y * Wc * a.D;
#pragma unroll
    for (int i0 = 0; i0 < Wc; i0 += SL) {
#pragma unroll
        for (int ii = 0; ii < SL; ++ii)
#pragma unroll
            for (int c = 0; c < CPT; ++c) red[w][ii][lane * CPT + c] = dape_acc[KEEP ? i0 + ii : 0][c];
        __syncthreads();
        for (int e = threadIdx.x; e < SL * 64 * CPT; e += kBwdWaves * 64) {
            const int ii = e / (64 * CPT), x = e - ii * (64 * CPT);
            const int d = blockIdx.x * 64 * CPT + x;
            if (d < a.D) {
                float v = red[0][ii][x];
#pragma unroll
                for (int u = 1; u < kBwdWaves; ++u) v += red[u][ii][x];
                part[(int64_t)(i0 + ii) * a.D + d] = v;
            }
        }
        __syncthreads();
    }
}

// dape[x] = sum over the per-workgroup partials: wave u adds partials u, u+16, ... in order
// (eight loads in flight), then the sixteen wave sums are added in order (64 entries x per
// workgroup).
constexpr int kDapeWaves = 16;
__global__ __launch_bounds__(kDapeWaves * 64) void compressor_dape_kernel(const float *__restrict__ part, int nparts,
                                                                          int64_t WcD, float *__restrict__ dape) {
    __shared__ float red[kDapeWaves][64];
    const int lane = threadIdx.x & 63, u = threadIdx.x >> 6;
    const int64_t x = (int64_t)blockIdx.x * 64 + lane;
    float s = 0.f;
    if (x < WcD) {
        int p = u;
        for (; p + 7 * kDapeWaves < nparts; p += 8 * kDapeWaves) {
            float v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = part[(int64_t)(p + q * kDapeWaves) * WcD + x];
#pragma unroll
            for (int q = 0; q < 8; ++q) s += v[q];
        }
        for (; p < nparts; p += kDapeWaves) s += part[(int64_t)p * WcD + x];
    }
    red[u][lane] = s;
    __syncthreads();
    if (u == 0 && x < WcD) {
        float t = red[0][lane];
#pragma unroll
        for (int i = 1; i < kDapeWaves; ++i) t += red[i][lane];
        dape[x] = t;
    }
}

template <int R, int OVL>
constexpr int cpt_for() {
    return R * (1 + OVL) <= 2 ? 4 : (R * (1 + OVL) <= 16 ? 2 : 1);
}

template <int DT, int R, int OVL>
hipError_t launch_fwd(const PoolArgs &a, hipStream_t stream) {
    constexpr int CPT = cpt_for<R, OVL>();
    const int64_t threads = (int64_t)a.B * a.N * (a.D / CPT);
    hipLaunchKernelGGL((compressor_pool_kernel<DT, R, OVL, CPT>), dim3((unsigned)((threads + kPoolThreads - 1) / kPoolThreads)),
                       dim3(kPoolThreads), 0, stream, a);
    return hipGetLastError();
}

template <int DT, int R, int OVL>
hipError_t launch_bwd(const PoolArgs &a, hipStream_t stream) {
    constexpr int CPT = cpt_for<R, OVL>();
    constexpr int Wc = R * (1 + OVL);
    const int G = a.D / CPT;
    const dim3 grid((unsigned)((G + 63) / 64), (unsigned)((int64_t)a.B * a.ncb));
    hipLaunchKernelGGL((compressor_pool_bwd_kernel<DT, R, OVL, CPT>), grid, dim3(kBwdWaves * 64), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t WcD = (int64_t)Wc * a.D;
    hipLaunchKernelGGL(compressor_dape_kernel, dim3((unsigned)((WcD + 63) / 64)), dim3(kDapeWaves * 64), 0, stream,
                       a.dape_part, a.B * a.ncb, WcD, a.dape);
    return hipGetLastError();
}

template <int DT, bool BWD>
hipError_t dispatch(const PoolArgs &a, int ratio, int overlap, hipStream_t stream) {
#define SD_CP(R, O) return BWD ? launch_bwd<DT, R, O>(a, stream) : launch_fwd<DT, R, O>(a, stream)
    if (overlap) {
        switch (ratio) {
            case 1: SD_CP(1, 1);
            case 2: SD_CP(2, 1);
            case 4: SD_CP(4, 1);
            case 8: SD_CP(8, 1);
            case 16: SD_CP(16, 1);
            default: return hipErrorInvalidValue;
        }
    }
    switch (ratio) {
        case 1: SD_CP(1, 0);
        case 2: SD_CP(2, 0);
        case 4: SD_CP(4, 0);
        case 8: SD_CP(8, 0);
        case 16: SD_CP(16, 0);
        case 32: SD_CP(32, 0);
        case 64: SD_CP(64, 0);
        case 128: SD_CP(128, 0);
        default: return hipErrorInvalidValue;
    }
#undef SD_CP
}

}  // namespace

bool compressor_supported(int ratio, int overlap) {
    const bool pow2 = ratio > 0 && (ratio & (ratio - 1)) == 0;
    return pow2 && (overlap ? ratio <= 16 : ratio <= 128);
}

size_t compressor_bwd_workspace_bytes(int B, int S, int D, int ratio, int overlap) {
    const int64_t N = S / ratio;
    const int64_t nchunk = (N + kChunk - 1) / kChunk;
    const int64_t ncb = (nchunk + kBwdWaves - 1) / kBwdWaves;
    return (size_t)((int64_t)B * ncb * ratio * (1 + overlap) * D * (int64_t)sizeof(float));
}

hipError_t launch_compressor_pool(const void *kv, const void *score, const float *ape, const int32_t *seg, int B,
                                  int S, int D, int ratio, int overlap, int dtype, float *pool, hipStream_t stream) {
    PoolArgs a{};
    a.kv = kv; a.score = score; a.ape = ape; a.seg = seg; a.pool = pool;
    a.B = B; a.S = S; a.D = D; a.N = S / ratio;
    return dtype == 0 ? dispatch<0, false>(a, ratio, overlap, stream) : dispatch<1, false>(a, ratio, overlap, stream);
}

hipError_t launch_compressor_pool_bwd(const void *kv, const void *score, const float *ape, const int32_t *seg,
                                      const float *dpool, int B, int S, int D, int ratio, int overlap, int dtype,
                                      float *dkv, float *dscore, float *dape, void *workspace, hipStream_t stream) {
    PoolArgs a{};
    a.kv = kv; a.score = score; a.ape = ape; a.seg = seg; a.dpool = dpool;
    a.dkv = dkv; a.dscore = dscore; a.dape = dape; a.dape_part = reinterpret_cast<float *>(workspace);
    a.B = B; a.S = S; a.D = D; a.N = S / ratio;
    a.nchunk = (a.N + kChunk - 1) / kChunk;
    a.ncb = (a.nchunk + kBwdWaves - 1) / kBwdWaves;
    return dtype == 0 ? dispatch<0, true>(a, ratio, overlap, stream) : dispatch<1, true>(a, ratio, overlap, stream);
}

}  // namespace sd
