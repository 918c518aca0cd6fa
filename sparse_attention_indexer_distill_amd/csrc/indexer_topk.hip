// indexer_topk.hip -- the indexer's masked top-k selection and its gradient, on gfx950.
//
// The step before the distillation target (MaxText PR "Add Indexer Loss [Deepseek v4]"):
// each query keeps the top-k of its student block scores under the causal block mask
// combined with the segment (packing) mask -- a block is visible to token t once it is
// complete at t and all of its tokens belong to t's document -- and the slots it cannot
// fill hold -1.  Kept blocks are written in ascending block order (the set is what the
// target and the KL use; ascending order also makes later row gathers walk memory
// forward), with their scores as the values (the student logits of the KL); a -1 slot's
// value is -inf.  Equal scores prefer the smaller block index; NaN ranks lowest.
//
// Mapping: one wave per (b,t) row, element n of the row on lane n % 64, register n / 64,
// so every load and every ordered prefix runs over 64 consecutive blocks.  Scores map to
// order-preserving 32-bit keys (NaN -> 0, the smallest); the K-th largest visible key is
// found one byte at a time, most significant first: each pass counts the visible keys that
// share the bytes found so far into a 256-bin histogram in the wave's LDS (one atomic add per
// key), and a suffix scan over the bins (DPP, on the VALU) picks the next byte.  At most four
// passes, no sort.
// The backward is the adjoint of the gather values[k] = scores[idx[k]]: a dense row of N
// gradients, built in LDS and streamed out with 16-byte stores.  Outputs are written with
// streaming (non-temporal) stores: nothing reads them back here, and they measured faster.
#include <math.h>

#include "sd_device.hpp"
#include "sd_internal.hpp"

namespace sd {
namespace {

constexpr int kTopkWaves = 4;  // rows per workgroup, one wave each

// Order-preserving key of a score: larger score -> larger key; -0 and +0 share a key; every
// NaN maps to 0, below -inf (whose key is 0x007fffff).
__device__ __forceinline__ uint32_t order_key(float s) {
    uint32_t b = __float_as_uint(s);
    if ((b & 0x7fffffffu) > 0x7f800000u) return 0u;
    if (b == 0x80000000u) b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ int wave_popc(bool p) { return __popcll(__ballot(p)); }

// A wave's LDS accesses execute in issue order, so a lane reads what another lane of the same
// wave stored by an earlier instruction; this keeps the compiler from moving LDS accesses
// across the point and waits for the stores to complete.
__device__ __forceinline__ void wave_lds_order() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
}

// lanes below this one whose predicate is set (exclusive prefix within the wave)
__device__ __forceinline__ int wave_prefix(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Sum of v over this lane and every higher lane (inclusive suffix sum), on the VALU: a
// Hillis-Steele scan inside each 16-lane row with DPP row shifts (lanes past the row's end
// read 0), then the totals of the higher rows, read as scalars, are added.
__device__ __forceinline__ int wave_suffix_sum(int v, int lane) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x101, 0xf, 0xf, true);  // row_shl:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x102, 0xf, 0xf, true);  // row_shl:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x104, 0xf, 0xf, true);  // row_shl:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x108, 0xf, 0xf, true);  // row_shl:8
    const int r1 = __builtin_amdgcn_readlane(v, 16), r2 = __builtin_amdgcn_readlane(v, 32),
              r3 = __builtin_amdgcn_readlane(v, 48);  // totals of rows 1, 2, 3
    const int row = lane >> 4;
    return v + (row < 1 ? r1 : 0) + (row < 2 ? r2 : 0) + (row < 3 ? r3 : 0);
}

// E: registers per lane (N <= 64 E).
template <int E>
__global__ __launch_bounds__(kTopkWaves * 64) void indexer_topk_kernel(
    const float *__restrict__ scores, const int32_t *__restrict__ seg, int64_t rows, int S, int N, int K, int ratio,
    int32_t *__restrict__ idx_out, float *__restrict__ val_out) {
    __shared__ __align__(16) uint32_t hist_all[kTopkWaves][2][256];
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kTopkWaves + (threadIdx.x >> 6);
    if (row >= rows) return;  // waves never meet at a workgroup barrier: each owns its histograms
    uint32_t(*hists)[256] = hist_all[threadIdx.x >> 6];  // two, used by alternate passes
    const int64_t b = row / S;
    const int t = (int)(row - b * S);
    const int ncomplete = (t + 1) / ratio;           // blocks complete at t
    const int nc = ncomplete < N ? ncomplete : N;
    const float *sc = scores + row * N;
    const int32_t *sg = seg ? seg + b * S : nullptr;
    const int32_t st = sg ? sg[t] : 0;

    uint32_t key[E];
    bool vis[E];
    float val[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int n = 64 * e + lane;
        bool v = n < nc;
        if (v && sg) {
            for (int i = 0; i < ratio; ++i) v = v && sg[ratio * n + i] == st;   // whole block in t's document
        }
        val[e] = v ? sc[n] : 0.f;
        vis[e] = v;
        key[e] = v ? order_key(val[e]) : 0u;
    }
    int count = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) count += wave_popc(vis[e]);

    // Threshold tau: the K-th largest visible key, built a byte at a time.  Invariant: the
    // visible keys above the bytes found so far number fewer than K, and `need` of the keys
    // that share them are still to be taken.  When a pass takes its whole bin, the remaining
    // bytes of tau stay 0 and every key >= tau is kept (exactly K of them).
    uint32_t tau = 0u;
    int need = count;  // how many of the keys equal to tau are kept (in ascending block order)
    if (count > K) {
        need = K;
        uint32_t hmask = 0u;
        *reinterpret_cast<u32x4 *>(hists[0] + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4 *>(hists[1] + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
        wave_lds_order();
        for (int shift = 24, pass = 0; shift >= 0; shift -= 8, pass ^= 1) {
            uint32_t *hist = hists[pass];  // zero: cleared before the first pass or after its last use
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (vis[e] && (key[e] & hmask) == tau) atomicAdd(hist + ((key[e] >> shift) & 255u), 1u);
            wave_lds_order();
            const u32x4 h = *reinterpret_cast<const u32x4 *>(hist + 4 * lane);   // bins 4*lane .. 4*lane+3
            // cleared for the pass after next; the next pass's wait orders it before that pass
            *reinterpret_cast<u32x4 *>(hist + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
            const int own = (int)(h[0] + h[1] + h[2] + h[3]);
            const int suf = wave_suffix_sum(own, lane);  // keys in the bins of this and every higher lane
            // the byte's lane: the highest one whose suffix still reaches `need` (suf never
            // grows with the lane, and lane 0's suffix is every counted key, at least `need`)
            const int L = __popcll(__ballot(suf >= need)) - 1;
            const int above = __builtin_amdgcn_readlane(suf - own, L);   // keys in bins above lane L's four
            const u32x4 hl = {(uint32_t)__builtin_amdgcn_readlane((int)h[0], L),
                              (uint32_t)__builtin_amdgcn_readlane((int)h[1], L),
                              (uint32_t)__builtin_amdgcn_readlane((int)h[2], L),
                              (uint32_t)__builtin_amdgcn_readlane((int)h[3], L)};
            int cum = above, dig = 4 * L, inbin = 0;
#pragma unroll
            for (int j = 3; j >= 0; --j) {
                if (cum + (int)hl[j] >= need) {
                    dig = 4 * L + j;
                    inbin = (int)hl[j];
                    break;
                }
                cum += (int)hl[j];
            }
            need -= cum;  // keys above the chosen bin are all taken
            tau |= (uint32_t)dig << shift;
            hmask |= 255u << shift;
            if (need == inbin) {  // the whole bin is taken: keep every key >= tau (lower bytes 0)
                need = K;
                break;
            }
        }
    }

    int32_t *io = idx_out + row * K;
    float *vo = val_out ? val_out + row * K : nullptr;
    int tie_base = 0, pos_base = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        bool sel = vis[e];
        if (count > K) {
            const bool tie = vis[e] && key[e] == tau;
            const uint64_t tm = __ballot(tie);
            sel = vis[e] && (key[e] > tau || (tie && tie_base + wave_prefix(tm) < need));
            tie_base += __popcll(tm);
        }
        const uint64_t sm = __ballot(sel);
        if (sel) {
            const int pos = pos_base + wave_prefix(sm);
            __builtin_nontemporal_store(64 * e + lane, io + pos);
            if (vo) __builtin_nontemporal_store(val[e], vo + pos);
        }
        pos_base += __popcll(sm);
    }
    for (int k = pos_base + lane; k < K; k += 64) {  // slots left over
        __builtin_nontemporal_store(-1, io + k);
        if (vo) __builtin_nontemporal_store(-INFINITY, vo + k);
    }
}

// dscores[row, n] = sum of dval[row, k] over the valid slots k holding n, in slot order; 0 for
// every other block.  Slot indices are first written into the wave's LDS row as tags: if every
// valid slot reads its own tag back, the row's slots are distinct and each block receives
// one gradient by a plain store; otherwise the gradients are added one slot at a time.
// KE > 0: the row's K <= 64 KE slots and gradients are loaded once into registers (slot
// 64 e + lane in register e); KE == 0 reads them from memory in each pass (any K).
template <int KE>
__global__ __launch_bounds__(kTopkWaves * 64) void indexer_topk_bwd_kernel(
    const float *__restrict__ dval, const int32_t *__restrict__ idx, int64_t rows, int N, int K,
    float *__restrict__ dscores) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kTopkWaves + w;
    if (row >= rows) return;  // waves never meet at a workgroup barrier: each owns its LDS row
    uint32_t *tag = reinterpret_cast<uint32_t *>(smem) + (size_t)w * N;
    float *buf = reinterpret_cast<float *>(tag);
    const int32_t *ir = idx + row * K;
    const float *dr = dval + row * K;
    constexpr int R = KE > 0 ? KE : 1;
    int sn[R];
    float sgv[R];
    if constexpr (KE > 0) {
#pragma unroll
        for (int e = 0; e < KE; ++e) {
            const int k = 64 * e + lane;
            sn[e] = k < K ? ir[k] : -1;
            sgv[e] = k < K ? dr[k] : 0.f;
        }
    }
    // slot k of this lane's e-th step and its block (-1 when invalid or past K)
    auto slot = [&](int e, int k) -> int {
        int n;
        if constexpr (KE > 0) n = sn[e];
        else n = k < K ? ir[k] : -1;
        return n >= 0 && n < N ? n : -1;
    };
    const int steps = KE > 0 ? KE : (K + 63) / 64;

    for (int n = lane; n < N; n += 64) tag[n] = 0xffffffffu;
    wave_lds_order();
    for (int e = 0; e < steps; ++e) {
        const int k = 64 * e + lane, n = slot(e, k);
        if (n >= 0) tag[n] = (uint32_t)k;
    }
    wave_lds_order();
    bool dup = false;
    for (int e = 0; e < steps; ++e) {
        const int k = 64 * e + lane, n = slot(e, k);
        if (n >= 0) dup = dup || tag[n] != (uint32_t)k;
    }
    const bool any_dup = __ballot(dup) != 0;
    wave_lds_order();
    for (int n = lane; n < N; n += 64) buf[n] = 0.f;
    wave_lds_order();
    for (int e = 0; e < steps; ++e) {
        const int k = 64 * e + lane, n = slot(e, k);
        float g;
        if constexpr (KE > 0) g = sgv[e];
        else g = k < K ? dr[k] : 0.f;
        if (!any_dup) {
            if (n >= 0) buf[n] = g;
        } else {
            for (int j = 0; j < 64; ++j) {  // slot order within the step
                if (lane == j && n >= 0) buf[n] += g;
                wave_lds_order();
            }
        }
    }
    wave_lds_order();
    float *o = dscores + row * N;
    if ((N & 3) == 0) {
        for (int n = 4 * lane; n < N; n += 256)
            __builtin_nontemporal_store(*reinterpret_cast<const f32x4 *>(buf + n), reinterpret_cast<f32x4 *>(o + n));
    } else {
        for (int n = lane; n < N; n += 64) o[n] = buf[n];
    }
}

template <int E>
hipError_t launch_topk(const float *scores, const int32_t *seg, int64_t rows, int S, int N, int K, int ratio,
                       int32_t *idx, float *values, hipStream_t stream) {
    const unsigned grid = (unsigned)((rows + kTopkWaves - 1) / kTopkWaves);
    hipLaunchKernelGGL(indexer_topk_kernel<E>, dim3(grid), dim3(kTopkWaves * 64), 0, stream, scores, seg, rows, S,
                       N, K, ratio, idx, values);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_topk(const float *scores, const int32_t *seg, int B, int S, int N, int K, int ratio,
                               int32_t *idx, float *values, hipStream_t stream) {
    const int64_t rows = (int64_t)B * S;
    if (N <= 64) return launch_topk<1>(scores, seg, rows, S, N, K, ratio, idx, values, stream);
    if (N <= 128) return launch_topk<2>(scores, seg, rows, S, N, K, ratio, idx, values, stream);
    if (N <= 256) return launch_topk<4>(scores, seg, rows, S, N, K, ratio, idx, values, stream);
    if (N <= 512) return launch_topk<8>(scores, seg, rows, S, N, K, ratio, idx, values, stream);
    if (N <= 1024) return launch_topk<16>(scores, seg, rows, S, N, K, ratio, idx, values, stream);
    if (N <= 2048) return launch_topk<32>(scores, seg, rows, S, N, K, ratio, idx, values, stream);
    return launch_topk<64>(scores, seg, rows, S, N, K, ratio, idx, values, stream);
}

hipError_t launch_indexer_topk_bwd(const float *dvalues, const int32_t *idx, int B, int S, int N, int K,
                                   float *dscores, hipStream_t stream) {
    const int64_t rows = (int64_t)B * S;
    const unsigned grid = (unsigned)((rows + kTopkWaves - 1) / kTopkWaves);
    const size_t lds = (size_t)kTopkWaves * N * sizeof(float);  // <= 64 KiB for N <= 4096
#define SD_TB(KE) hipLaunchKernelGGL(indexer_topk_bwd_kernel<KE>, dim3(grid), dim3(kTopkWaves * 64), lds, stream, \
                                     dvalues, idx, rows, N, K, dscores)
    if (K <= 64) SD_TB(1);
    else if (K <= 128) SD_TB(2);
    else if (K <= 256) SD_TB(4);
    else if (K <= 512) SD_TB(8);
    else if (K <= 1024) SD_TB(16);
    else SD_TB(0);
#undef SD_TB
    return hipGetLastError();
}

}  // namespace sd
