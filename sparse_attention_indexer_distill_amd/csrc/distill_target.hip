// distill_target.hip -- KL target of the CSA indexer distillation on gfx950.
//
// For one token (b,t) the heads' scores against the token's top-k pool rows,
//     c[h,k] = scale * <q[b,t,h,:], pool[b, idx[b,t,k], :]>,
// are one [H x D] x [D x K] product whose right operand is gathered through idx.  The
// target is the conditional, on those rows, of each head's joint softmax over
// [window keys | selected rows | sink]; heads are summed and the row L1-renormalised
// with a float32-tiny floor (Primus PR "perf(deepseek-v4): fuse and enable the indexer
// distillation loss": PR body "Why the target was wrong" and the joint-softmax commit;
// the pool is indexed inside the kernel, so no [B,S,K,D] gather is materialised).
//
// Mapping.  One workgroup per token, NW waves.  The token's queries (all heads) are
// staged once in LDS in MFMA fragment order.  The valid slots of the row are compacted
// (stable, slot order) into a list in LDS; 16-slot tiles of that list are dealt
// round-robin to the waves, so invalid (-1) slots cost no MFMA work wherever they sit.
// Each wave streams its rows' fragments straight from L2/HBM (each lane reads 16
// contiguous bytes of one pool row per 32-wide D chunk) and accumulates
//     C[slot][head] (16x16 tiles) = pool_row . q_head
// for all heads, keeping every score of its slots in registers.  The per-head maximum
// and sum (log2 domain) need two cross-lane steps plus one LDS exchange between waves;
// the head sum of p[h,k] = exp(c[h,k] - full_h) is a 16-lane DPP reduction.  Nothing but
// the target row is written.
#include <float.h>

#include "sd_device.hpp"
#include "sd_internal.hpp"

namespace sd {
namespace {

template <int DT, int HT, int KT, int NW>
__global__ __launch_bounds__(NW * 64) void distill_target_kernel(
    const void *__restrict__ q, const void *__restrict__ pool, const int32_t *__restrict__ idx,
    const float *__restrict__ nc_lse, int S, int H, int D, int N, int K, float scale_log2, float l1_floor,
    float *__restrict__ target) {
    using frag_t = typename Elem<DT>::frag_t;
    extern __shared__ __align__(16) unsigned char smem[];
    const int nch = D >> 5;
    frag_t *qs = reinterpret_cast<frag_t *>(smem);                 // [HT][nch][64]
    int32_t *crow = reinterpret_cast<int32_t *>(qs + (size_t)HT * nch * 64);  // [K] pool row per compacted slot
    int32_t *cslot = crow + K;                                      // [K] slot index per compacted slot
    float *red_a = reinterpret_cast<float *>(cslot + K);            // [NW][16*HT]
    float *red_b = red_a + NW * 16 * HT;                            // [NW][16*HT]
    float *red_t = red_b + NW * 16 * HT;                            // [NW]
    int *wcnt = reinterpret_cast<int *>(red_t + NW);                // [NW]

    // Latest tokens have the most valid slots: start them first.
    const int64_t bt = (int64_t)gridDim.x - 1 - blockIdx.x;
    const int b = (int)(bt / S);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int32_t *idr = idx + bt * K;
    float *Tr = target + bt * K;

    // 1. Stable compaction of the valid slots; invalid slots get target 0 here.
    int base = 0;
    for (int k0 = 0; k0 < K; k0 += NW * 64) {
        const int k = k0 + tid;
        const int v = k < K ? idr[k] : -1;
        const bool ok = k < K && v >= 0 && v < N;
        if (k < K && !ok) Tr[k] = 0.f;
        const uint64_t bal = __ballot(ok);
        const int pre = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        if (lane == 0) wcnt[w] = __popcll(bal);
        __syncthreads();
        int off = base, tot = 0;
        for (int i = 0; i < NW; ++i) {
            const int c = wcnt[i];
            off += i < w ? c : 0;
            tot += c;
        }
        if (ok) {
            crow[off + pre] = v;
            cslot[off + pre] = k;
        }
        base += tot;
        __syncthreads();
    }
    const int nvalid = base;
    if (nvalid == 0) return;  // empty row: already all zeros

    // 2. Stage the token's queries (all heads; padded heads are zero) in fragment order.
    {
        const size_t qrow = (size_t)bt * H * D;
        const int upr = D >> 3;
        for (int u = tid; u < 16 * HT * upr; u += NW * 64) {
            const int h = u / upr, cu = u - h * upr;
            qs[((h >> 4) * nch + (cu >> 2)) * 64 + (h & 15) + 16 * (cu & 3)] =
                h < H ? load_frag<DT>(q, qrow + (size_t)h * D + 8 * cu) : zero_frag<DT>();
        }
    }
    __syncthreads();

    // 3. Scores of this wave's slot tiles: tiles w, w+NW, w+2NW, ... of the compacted list.
    const int ntiles = (nvalid + 15) >> 4;
    const int my = ntiles > w ? (ntiles - w + NW - 1) / NW : 0;
    size_t off[KT];
#pragma unroll
    for (int l = 0; l < KT; ++l) {
        const int pos = 16 * (w + l * NW) + (lane & 15);
        const int r = (l < my && pos < nvalid) ? crow[pos] : crow[0];
        off[l] = ((size_t)b * N + r) * D + 8 * (lane >> 4);
    }
    f32x4 acc[KT][HT];
#pragma unroll
    for (int l = 0; l < KT; ++l)
#pragma unroll
        for (int h = 0; h < HT; ++h) acc[l][h] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int c = 0; c < nch; ++c) {
        frag_t bq[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) bq[ht] = qs[(ht * nch + c) * 64 + lane];
#pragma unroll
        for (int l = 0; l < KT; ++l) {
            if (l < my) {
                const frag_t a = load_frag<DT>(pool, off[l] + 32 * c);
#pragma unroll
                for (int ht = 0; ht < HT; ++ht) acc[l][ht] = mfma_frag<DT>(a, bq[ht], acc[l][ht]);
            }
        }
    }

    // 4. Per-head maximum over the row's valid slots (log2 domain).
    const int prow = 4 * (lane >> 4);
    float mx[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) mx[ht] = -INFINITY;
#pragma unroll
    for (int l = 0; l < KT; ++l)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = l < my && 16 * (w + l * NW) + prow + i < nvalid;
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                const float x = ok ? acc[l][ht][i] * scale_log2 : -INFINITY;
                acc[l][ht][i] = x;
                mx[ht] = fmaxf(mx[ht], x);
            }
        }
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        mx[ht] = cols4_max(mx[ht]);
        if (lane < 16) red_a[w * 16 * HT + ht * 16 + lane] = mx[ht];
    }
    __syncthreads();
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        float m = -INFINITY;
        for (int i = 0; i < NW; ++i) m = fmaxf(m, red_a[i * 16 * HT + ht * 16 + (lane & 15)]);
        mx[ht] = m;
    }

    // 5. Per-head sum of exp2(c - max); keep the exponentials in the accumulators.
    float sm[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) sm[ht] = 0.f;
#pragma unroll
    for (int l = 0; l < KT; ++l)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                const float e = fast_exp2(acc[l][ht][i] - mx[ht]);
                acc[l][ht][i] = e;
                sm[ht] += e;
            }
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        sm[ht] = cols4_sum(sm[ht]);
        if (lane < 16) red_b[w * 16 * HT + ht * 16 + lane] = sm[ht];
    }
    __syncthreads();

    // Joint denominator: full_h = log(sum_k exp(c_hk) + exp(nc_lse_h)); a head's weight
    // on the compressed part is exp(c_max_h - full_h) times its exp2(c - c_max) values.
    float wgt[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const int h = ht * 16 + (lane & 15);
        float s = 0.f;
        for (int i = 0; i < NW; ++i) s += red_b[i * 16 * HT + ht * 16 + (lane & 15)];
        const float clse = mx[ht] + fast_log2(s);
        float full = clse;
        if (nc_lse != nullptr && h < H) full = logaddexp2(clse, nc_lse[bt * H + h] * kLog2e);
        wgt[ht] = h < H ? fast_exp2(mx[ht] - full) : 0.f;
    }

    // 6. Head sum m_k (16-lane row reduction) and the row total.
    float m[KT][4];
    float part = 0.f;
#pragma unroll
    for (int l = 0; l < KT; ++l)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float v = 0.f;
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) v += acc[l][ht][i] * wgt[ht];
            v = row16_sum(v);
            m[l][i] = v;
            part += v;  // invalid slots hold exactly 0
        }
    part = cols4_sum(part);
    if (lane == 0) red_t[w] = part;
    __syncthreads();
    float tot = 0.f;
    for (int i = 0; i < NW; ++i) tot += red_t[i];
    const float den = fmaxf(tot, l1_floor);

    // 7. Scatter the row back to slot order.
    const int isel = lane & 15;
    if (isel < 4) {
#pragma unroll
        for (int l = 0; l < KT; ++l) {
            const int pos = 16 * (w + l * NW) + prow + isel;
            if (l < my && pos < nvalid) {
                const float v = isel == 0 ? m[l][0] : isel == 1 ? m[l][1] : isel == 2 ? m[l][2] : m[l][3];
                Tr[cslot[pos]] = v / den;
            }
        }
    }
}

template <int DT, int HT, int KT, int NW>
hipError_t launch3(const void *q, const void *pool, const int32_t *idx, const float *nc_lse, int B, int S, int H,
                   int D, int N, int K, float scale, float l1_floor, float *target, hipStream_t stream) {
    const size_t lds = (size_t)HT * (D / 32) * 64 * sizeof(typename Elem<DT>::frag_t) + (size_t)2 * K * 4 +
                       (size_t)2 * NW * 16 * HT * 4 + (size_t)NW * 8;
    const float fl = l1_floor > 0.f ? l1_floor : FLT_MIN;
    if (lds > 65536) {  // opt in to more than 64 KiB of LDS per workgroup (gfx950 has 160 KiB per CU)
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&distill_target_kernel<DT, HT, KT, NW>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((distill_target_kernel<DT, HT, KT, NW>), dim3((unsigned)((int64_t)B * S)), dim3(NW * 64),
                       lds, stream, q, pool, idx, nc_lse, S, H, D, N, K, scale * kLog2e, fl, target);
    return hipGetLastError();
}

template <int DT, int HT>
hipError_t launch2(const void *q, const void *pool, const int32_t *idx, const float *nc_lse, int B, int S, int H,
                   int D, int N, int K, float scale, float l1_floor, float *target, hipStream_t stream) {
#define SD_T(KT, NW) launch3<DT, HT, KT, NW>(q, pool, idx, nc_lse, B, S, H, D, N, K, scale, l1_floor, target, stream)
    if (K <= 16) return SD_T(1, 1);
    if (K <= 64) return SD_T(1, 4);
    if (K <= 128) return SD_T(2, 4);
    if (K <= 256) return SD_T(4, 4);
    if (K <= 512) return SD_T(8, 4);
    return SD_T(8, 8);
#undef SD_T
}

template <int DT>
hipError_t launch1(const void *q, const void *pool, const int32_t *idx, const float *nc_lse, int B, int S, int H,
                   int D, int N, int K, float scale, float l1_floor, float *target, hipStream_t stream) {
    if (H <= 16) return launch2<DT, 1>(q, pool, idx, nc_lse, B, S, H, D, N, K, scale, l1_floor, target, stream);
    if (H <= 32) return launch2<DT, 2>(q, pool, idx, nc_lse, B, S, H, D, N, K, scale, l1_floor, target, stream);
    return launch2<DT, 4>(q, pool, idx, nc_lse, B, S, H, D, N, K, scale, l1_floor, target, stream);
}

}  // namespace

hipError_t launch_distill_target(const void *q, const void *pool, const int32_t *idx, const float *nc_lse,
                                 int B, int S, int H, int D, int N, int K, float scale, float l1_floor,
                                 int dtype, float *target, hipStream_t stream) {
    if (dtype == 0) return launch1<0>(q, pool, idx, nc_lse, B, S, H, D, N, K, scale, l1_floor, target, stream);
    return launch1<1>(q, pool, idx, nc_lse, B, S, H, D, N, K, scale, l1_floor, target, stream);
}

}  // namespace sd
