// window_lse.hip -- banded sliding-window + sink log-sum-exp on gfx950.
//
// Computes, per token t and head h, the log-mass of the non-compressed part of the
// CSA layer's joint softmax: the W window keys ending at t (same packed segment) plus
// the per-head sink (Primus PR "perf(deepseek-v4): fuse and enable the indexer
// distillation loss", commit adding the sliding-window LSE kernel: scores stay on chip
// and only the key band a block of queries spans is loaded).
//
// Mapping.  A workgroup owns 4 consecutive tokens of one batch row, one wave per token.
// The key band those tokens span (16-key tiles covering [t0-W+1, t0+3]) is staged in
// LDS one D-chunk at a time, already in MFMA fragment order, and shared by the four
// waves.  Each wave contracts its token's queries (all heads, read straight from HBM
// once) against the band tiles its own window touches:
//     C[key][head] += kwin[key, d-chunk] . q[t, head, d-chunk]     (16x16 tiles)
// so a lane ends up holding one head column and 4 keys per tile; the masked online
// maximum and sum over keys therefore stay in registers and only need two cross-lane
// steps.  The queries are the only HBM stream; everything else is reused from L2/LDS.
#include <algorithm>

#include "sd_device.hpp"
#include "sd_internal.hpp"

namespace sd {
namespace {

constexpr int kWinTok = 4;  // tokens (waves) per workgroup

// Number of 16-key tiles the window [max(0, t-W+1), t] of one token can touch.
__host__ __device__ constexpr int win_tiles(int W) { return (W + 14) / 16 + 1; }

template <int DT, int HT, int NBT, int NSUB>
__global__ __launch_bounds__(kWinTok * 64) void window_lse_kernel(
    const void *__restrict__ q, const void *__restrict__ kwin, const float *__restrict__ sink,
    const int32_t *__restrict__ seg, int S, int H, int D, int W, float scale_log2, float *__restrict__ nc_lse) {
    using frag_t = typename Elem<DT>::frag_t;
    extern __shared__ __align__(16) unsigned char smem[];

    const int b = blockIdx.y;
    const int t0 = blockIdx.x * kWinTok;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int t = t0 + w;
    const bool active = t < S;

    // Key band of the workgroup, in 16-key tiles.
    const int tlast = min(t0 + kWinTok - 1, S - 1);
    const int tile0 = max(t0 - W + 1, 0) >> 4;
    const int nb = (tlast >> 4) - tile0 + 1;
    const int nbmax = win_tiles(W + kWinTok - 1);
    frag_t *band = reinterpret_cast<frag_t *>(smem);                     // [nbmax][NSUB][64]
    int32_t *segband = reinterpret_cast<int32_t *>(band + (size_t)nbmax * NSUB * 64);  // [nbmax*16]

    if (seg) {
        for (int i = tid; i < nb * 16; i += kWinTok * 64) {
            const int key = tile0 * 16 + i;
            segband[i] = key < S ? seg[(size_t)b * S + key] : INT32_MIN;
        }
    }
    const int seg_t = (seg && active) ? seg[(size_t)b * S + t] : 0;

    // This wave's tiles inside the band.
    const int kf = max(t - W + 1, 0);
    const int wfirst = (kf >> 4) - tile0;
    const int wn = active ? (t >> 4) - (kf >> 4) + 1 : 0;  // <= NBT

    f32x4 acc[NBT][HT];
#pragma unroll
    for (int j = 0; j < NBT; ++j)
#pragma unroll
        for (int h = 0; h < HT; ++h) acc[j][h] = f32x4{0.f, 0.f, 0.f, 0.f};

    const size_t qrow = ((size_t)b * S + (active ? t : 0)) * H * (size_t)D;
    const int upr = NSUB * 4;  // 8-element units per key row in one chunk
    for (int dc0 = 0; dc0 < D; dc0 += NSUB * 32) {
        // This wave's query fragments for the chunk (issued before the band load).
        frag_t qf[NSUB][HT];
#pragma unroll
        for (int s = 0; s < NSUB; ++s)
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                const int h = ht * 16 + (lane & 15);
                const int d = dc0 + 32 * s + 8 * (lane >> 4);
                qf[s][ht] = (active && h < H && d < D) ? load_frag<DT>(q, qrow + (size_t)h * D + d) : zero_frag<DT>();
            }
        __syncthreads();  // the previous chunk's band is no longer read
        for (int u = tid; u < nb * 16 * upr; u += kWinTok * 64) {
            const int row = u / upr, cu = u - row * upr;
            const int key = tile0 * 16 + row;
            const int d = dc0 + 8 * cu;
            band[((row >> 4) * NSUB + (cu >> 2)) * 64 + (row & 15) + 16 * (cu & 3)] =
                (key < S && d < D) ? load_frag<DT>(kwin, ((size_t)b * S + key) * D + d) : zero_frag<DT>();
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
            if (dc0 + 32 * s >= D) break;
#pragma unroll
            for (int j = 0; j < NBT; ++j) {
                if (j < wn) {
                    const frag_t a = band[((wfirst + j) * NSUB + s) * 64 + lane];
#pragma unroll
                    for (int ht = 0; ht < HT; ++ht) acc[j][ht] = mfma_frag<DT>(a, qf[s][ht], acc[j][ht]);
                }
            }
        }
    }
    if (!active) return;

    // Masked log-sum-exp over the window keys (log2 domain), then the sink.
    const int kbase = 16 * (tile0 + wfirst) + 4 * (lane >> 4);
    const int lo = t - W + 1;
    float mx[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) mx[ht] = -INFINITY;
#pragma unroll
    for (int j = 0; j < NBT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = kbase + 16 * j + i;
            bool ok = j < wn && key >= lo && key <= t;
            if (seg) ok = ok && segband[key - 16 * tile0] == seg_t;
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                const float x = ok ? acc[j][ht][i] * scale_log2 : -INFINITY;
                acc[j][ht][i] = x;
                mx[ht] = fmaxf(mx[ht], x);
            }
        }
    float sm[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        mx[ht] = cols4_max(mx[ht]);
        sm[ht] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < NBT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) sm[ht] += fast_exp2(acc[j][ht][i] - mx[ht]);
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        sm[ht] = cols4_sum(sm[ht]);
        const int h = ht * 16 + (lane & 15);
        float lse2 = mx[ht] + fast_log2(sm[ht]);
        if (sink && h < H) lse2 = logaddexp2(lse2, sink[h] * kLog2e);
        if (lane < 16 && h < H) nc_lse[((size_t)b * S + t) * H + h] = lse2 * kLn2;
    }
}

// ---------------------------------------------------------------------------------
// bf16 fast path (D % 64 == 0).  A workgroup owns TOK = 2 consecutive tokens x HG head
// tiles (one 16-head tile per wave: 2 x 4 = 8 waves at H = 64); wave w handles token
// w / HG and head tile w % HG.  D is walked in stages of 64 elements (128 bytes of every
// row).  Per stage the workgroup stages, with direct loads into LDS that each move 8
// rows x 128 bytes (fully coalesced):
//   * the key band its tokens span (16-key tiles covering [t0-W+1, t0+1]; from L2),
//     double buffered, one stage ahead;
//   * the queries of its 2 tokens, double buffered, one stage ahead; each wave's two
//     query loads of a stage are issued between its MFMAs.
// Rows are stored with their 16-byte segments XOR-swizzled by (row >> 1) & 7, so the
// 16-row MFMA fragment reads hit distinct LDS banks.  A workgroup needs about 73 KB of
// LDS at W = 128, so two share a CU and each covers the other's load waits (the stage
// loop ends every stage with a full wait and a bare barrier).  Every wave computes the same NBT tiles
// from its first window tile; keys outside the token's window are masked, so the loop
// has no branches.
constexpr int kTokMfma = 2;

__device__ __forceinline__ uint32_t sw_pos(int r, int x) {  // byte offset of row r, segment x
    return (uint32_t)(r * 128 + ((x ^ ((r >> 1) & 7)) << 4));
}

template <int NBT>
__global__ __launch_bounds__(1024) void window_lse_mfma_kernel(
    const void *__restrict__ q, const void *__restrict__ kwin, const float *__restrict__ sink,
    const int32_t *__restrict__ seg, int S, int H, int D, int W, int HG, int nballoc, float scale_log2,
    float *__restrict__ nc_lse) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int b = blockIdx.y;
    const int t0 = blockIdx.x * kTokMfma;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int nwaves = blockDim.x >> 6;
    const int tok = w / HG, hg = w - tok * HG;
    const int t = t0 + tok;
    const bool active = t < S;
    const int HP = HG * 16;  // padded head count

    const int tlast = min(t0 + kTokMfma - 1, S - 1);
    const int tile0 = max(t0 - W + 1, 0) >> 4;
    const int nb = (tlast >> 4) - tile0 + 1;  // band tiles actually loaded
    const int band_bytes = nballoc * 16 * 128;
    const int qst_bytes = kTokMfma * HP * 128;
    unsigned char *band = smem;                   // [2][nballoc*16 rows][128 B]
    unsigned char *qst = smem + 2 * band_bytes;   // [2][TOK*HP rows][128 B]
    int32_t *segband = reinterpret_cast<int32_t *>(qst + 2 * qst_bytes);  // [nballoc*16]

    const rsrc_t kr = make_rsrc(reinterpret_cast<const char *>(kwin) + (size_t)b * S * D * 2, (uint32_t)((size_t)S * D * 2));
    const int nqtok = min(kTokMfma, S - t0);
    const rsrc_t qr = make_rsrc(reinterpret_cast<const char *>(q) + ((size_t)b * S + t0) * H * D * 2,
                                (uint32_t)(nqtok * H * D * 2));
    const int r_in = lane >> 3;
    // Key band of D stage st into band buffer st&1; instruction m covers band rows 8m..8m+7.
    auto stage_band = [&](int st) {
        unsigned char *dst = band + (st & 1) * band_bytes;
        for (int m = w; m < 2 * nb; m += nwaves) {
            const int r = 8 * m + r_in;
            const int x = (lane & 7) ^ ((r >> 1) & 7);  // lands at segment lane&7 of the swizzled row
            const int key = tile0 * 16 + r;
            const uint32_t voff = key < S ? (uint32_t)((key * D + st * 64 + 8 * x) * 2) : 0x80000000u;
            buf_load_lds16(kr, dst + m * 1024, voff);
        }
    };
    // Queries of D stage st into query buffer st%3; row = tok*HP + head.
    // Each wave issues exactly two of the TOK*HP/8 = 2*TOK*HG instructions (there are
    // TOK*HG waves): k = 0, 1.
    auto stage_q_one = [&](int st, int k) {
        unsigned char *dst = qst + (st & 1) * qst_bytes;
        const int m = w + k * nwaves;
        const int r = 8 * m + r_in;
        const int x = (lane & 7) ^ ((r >> 1) & 7);
        const int tk = r / HP, hd = r - tk * HP;
        const uint32_t voff = hd < H ? (uint32_t)(((tk * H + hd) * D + st * 64 + 8 * x) * 2) : 0x80000000u;
        buf_load_lds16(qr, dst + m * 1024, voff);
    };
    auto stage_q = [&](int st) {
        stage_q_one(st, 0);
        stage_q_one(st, 1);
    };
    if (seg) {
        for (int i = tid; i < nb * 16; i += blockDim.x) {
            const int key = tile0 * 16 + i;
            segband[i] = key < S ? seg[(size_t)b * S + key] : INT32_MIN;
        }
    }
    const int seg_t = (seg && active) ? seg[(size_t)b * S + t] : 0;

    // This wave's first window tile inside the band.
    const int kf = max(t - W + 1, 0);
    const int wfirst = active ? (kf >> 4) - tile0 : 0;

    f32x4 acc[NBT];
#pragma unroll
    for (int j = 0; j < NBT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The swizzle only depends on the row within a 16-row tile, so tile j's fragment sits
    // at a fixed base plus 2048*j bytes (an immediate offset).
    const int rq = tok * HP + hg * 16 + (lane & 15);
    const int rb = wfirst * 16 + (lane & 15);
    // MFMAs of stage st.  With qst_next >= 0 the wave's two query loads of that stage are
    // issued in the middle of the two chunks' MFMA runs, so the workgroup's loads reach the
    // memory pipeline spread over the stage instead of as one burst after the barrier.
    auto compute = [&](int st, int qst_next) {
        const unsigned char *bsrc = band + (st & 1) * band_bytes;
        const unsigned char *qsrc = qst + (st & 1) * qst_bytes;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int x = 4 * c + (lane >> 4);
            const u32x4 bq = *reinterpret_cast<const u32x4 *>(qsrc + sw_pos(rq, x));
            const unsigned char *fb = bsrc + sw_pos(rb, x);
            u32x4 a = *reinterpret_cast<const u32x4 *>(fb);
#pragma unroll
            for (int j = 0; j < NBT; ++j) {
                if (j == NBT / 2 && qst_next >= 0) {
                    __builtin_amdgcn_sched_barrier(0);
                    stage_q_one(qst_next, c);
                    __builtin_amdgcn_sched_barrier(0);
                }
                u32x4 an = a;
                if (j + 1 < NBT) an = *reinterpret_cast<const u32x4 *>(fb + 2048 * (j + 1));
                acc[j] = mfma_frag<0>(a, bq, acc[j]);
                a = an;
            }
        }
    };

    const int nst = D >> 6;
    stage_q(0);
    stage_band(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
        if (st + 1 < nst) stage_band(st + 1);
        compute(st, st + 1 < nst ? st + 1 : -1);  // issues the next query stage between the MFMAs
        // This wave's share of the next stage has landed in LDS and its reads of this stage
        // were consumed by its MFMAs; a bare barrier then publishes the stage.
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
    }
    if (!active) return;

    // Masked log-sum-exp over the window keys (log2 domain), then the sink.
    const int kbase = 16 * (tile0 + wfirst) + 4 * (lane >> 4);
    const int lo = t - W + 1;
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < NBT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = kbase + 16 * j + i;
            bool ok = key >= lo && key <= t;
            if (seg && ok) ok = segband[key - 16 * tile0] == seg_t;
            const float x = ok ? acc[j][i] * scale_log2 : -INFINITY;
            acc[j][i] = x;
            mx = fmaxf(mx, x);
        }
    mx = cols4_max(mx);
    float sm = 0.f;
#pragma unroll
    for (int j = 0; j < NBT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) sm += fast_exp2(acc[j][i] - mx);
    sm = cols4_sum(sm);
    const int head = hg * 16 + (lane & 15);
    float lse2 = mx + fast_log2(sm);
    if (sink && head < H) lse2 = logaddexp2(lse2, sink[head] * kLog2e);
    if (lane < 16 && head < H) nc_lse[((size_t)b * S + t) * H + head] = lse2 * kLn2;
}

template <int NBT>
hipError_t launch_mfma(const void *q, const void *kwin, const float *sink, const int32_t *seg, int B, int S, int H,
                       int D, int W, float scale, float *nc_lse, hipStream_t stream) {
    const int HG = (H + 15) / 16;
    const int nballoc = std::max(win_tiles(W + kTokMfma - 1), NBT + 1);
    const size_t lds = (size_t)2 * nballoc * 16 * 128 + (size_t)2 * kTokMfma * HG * 16 * 128 + (size_t)nballoc * 16 * 4;
    auto kfn = &window_lse_mfma_kernel<NBT>;
    if (lds > (size_t)kLdsBytes) return hipErrorInvalidValue;
    if (lds > 65536) {  // more than the default 64 KiB of LDS per workgroup
        const hipError_t e = allow_full_lds<&window_lse_mfma_kernel<NBT>>();
        if (e != hipSuccess) return e;
    }
    dim3 grid((S + kTokMfma - 1) / kTokMfma, B);
    hipLaunchKernelGGL(kfn, grid, dim3(kTokMfma * HG * 64), lds, stream, q, kwin, sink, seg, S, H, D, W, HG, nballoc,
                       scale * kLog2e, nc_lse);
    return hipGetLastError();
}

hipError_t launch_mfma_w(const void *q, const void *kwin, const float *sink, const int32_t *seg, int B, int S, int H,
                         int D, int W, float scale, float *nc_lse, hipStream_t stream) {
    const int nt = win_tiles(W);
    if (nt <= 2) return launch_mfma<2>(q, kwin, sink, seg, B, S, H, D, W, scale, nc_lse, stream);
    if (nt <= 3) return launch_mfma<3>(q, kwin, sink, seg, B, S, H, D, W, scale, nc_lse, stream);
    if (nt <= 5) return launch_mfma<5>(q, kwin, sink, seg, B, S, H, D, W, scale, nc_lse, stream);
    return launch_mfma<9>(q, kwin, sink, seg, B, S, H, D, W, scale, nc_lse, stream);
}

template <int DT, int HT, int NBT>
hipError_t launch3(const void *q, const void *kwin, const float *sink, const int32_t *seg, int B, int S, int H,
                   int D, int W, float scale, float *nc_lse, hipStream_t stream) {
    constexpr int NSUB = DT == 0 ? 4 : 2;  // D-chunk of 128 bf16 / 64 fp32 elements
    const int nbmax = win_tiles(W + kWinTok - 1);
    const size_t lds = (size_t)nbmax * NSUB * 64 * sizeof(typename Elem<DT>::frag_t) + (size_t)nbmax * 16 * 4;
    dim3 grid((S + kWinTok - 1) / kWinTok, B);
    hipLaunchKernelGGL((window_lse_kernel<DT, HT, NBT, NSUB>), grid, dim3(kWinTok * 64), lds, stream, q, kwin,
                       sink, seg, S, H, D, W, scale * kLog2e, nc_lse);
    return hipGetLastError();
}

template <int DT, int HT>
hipError_t launch2(const void *q, const void *kwin, const float *sink, const int32_t *seg, int B, int S, int H,
                   int D, int W, float scale, float *nc_lse, hipStream_t stream) {
    const int nt = win_tiles(W);
    if (nt <= 2) return launch3<DT, HT, 2>(q, kwin, sink, seg, B, S, H, D, W, scale, nc_lse, stream);
    if (nt <= 3) return launch3<DT, HT, 3>(q, kwin, sink, seg, B, S, H, D, W, scale, nc_lse, stream);
    if (nt <= 5) return launch3<DT, HT, 5>(q, kwin, sink, seg, B, S, H, D, W, scale, nc_lse, stream);
    return launch3<DT, HT, 9>(q, kwin, sink, seg, B, S, H, D, W, scale, nc_lse, stream);
}

template <int DT>
hipError_t launch1(const void *q, const void *kwin, const float *sink, const int32_t *seg, int B, int S, int H,
                   int D, int W, float scale, float *nc_lse, hipStream_t stream) {
    if (H <= 16) return launch2<DT, 1>(q, kwin, sink, seg, B, S, H, D, W, scale, nc_lse, stream);
    if (H <= 32) return launch2<DT, 2>(q, kwin, sink, seg, B, S, H, D, W, scale, nc_lse, stream);
    return launch2<DT, 4>(q, kwin, sink, seg, B, S, H, D, W, scale, nc_lse, stream);
}

}  // namespace

hipError_t launch_window_lse(const void *q, const void *kwin, const float *sink, const int32_t *seg, int B,
                             int S, int H, int D, int W, float scale, int dtype, float *nc_lse,
                             hipStream_t stream) {
    if (dtype == 0 && D % 64 == 0)  // bf16 fast path: 2 tokens x up to 4 head tiles per workgroup
        return launch_mfma_w(q, kwin, sink, seg, B, S, H, D, W, scale, nc_lse, stream);
    if (dtype == 0) return launch1<0>(q, kwin, sink, seg, B, S, H, D, W, scale, nc_lse, stream);
    return launch1<1>(q, kwin, sink, seg, B, S, H, D, W, scale, nc_lse, stream);
}

}  // namespace sd
