// distill_kl.hip -- fused KL(target || softmax(student logits)) with its gradient.
//
// One wave per (b,t) row.  The student softmax runs over the row's valid slots only;
// the forward value and the analytic gradient (sum T) * softmax(z) - T come out of the
// same pass, so nothing is saved between forward and backward (Primus PR
// "perf(deepseek-v4): fuse and enable the indexer distillation loss", commit fusing
// the KL tail with an analytic backward; MaxText PR "Add Indexer Loss [Deepseek v4]",
// review comments: log-softmax KL without epsilon, exact gradient Q - P).
//
// The row is read once from HBM into registers (T, z and idx in one round trip, 16-byte
// loads when K % 4 == 0), all reductions are xor-butterflies inside the wave, and the
// per-row KL plus a per-block (sum, count) partial are written.  A one-block finalize
// kernel adds the partials in a fixed order, so the loss statistics are bitwise
// reproducible.  (A last-block-reduces variant in the same launch needs device-scope
// fences per block, which write back and invalidate L2 and cost far more than the
// second launch.)
#include <atomic>
#include <mutex>

#include "sd_device.hpp"
#include "sd_internal.hpp"

namespace sd {
namespace {

constexpr int kKlRowsPerBlock = 8;

// Loads of one row: V = 4 consecutive slots per lane and chunk (16-byte loads, K % 4 == 0)
// or V = 1 (any K).  Lane l holds slots V*l + 64*V*c + j.  T, z and idx are loaded
// unconditionally in one round trip (all three are K-long rows); validity is applied
// afterwards.  The gradient row is written with streaming (non-temporal) stores: nothing
// reads it back here, and they measured faster.
template <int V>
struct RowIO;
template <>
struct RowIO<1> {
    static __device__ __forceinline__ void load(const float *p, int k, int K, float *o) { o[0] = k < K ? p[k] : 0.f; }
    static __device__ __forceinline__ void load(const int32_t *p, int k, int K, int *o) { o[0] = k < K ? p[k] : -1; }
    static __device__ __forceinline__ void store(float *p, int k, int K, const float *v) {  // streaming store
        if (k < K) __builtin_nontemporal_store(v[0], p + k);
    }
};
template <>
struct RowIO<4> {
    static __device__ __forceinline__ void load(const float *p, int k, int K, float *o) {
        if (k < K) {
            const f32x4 x = *reinterpret_cast<const f32x4 *>(p + k);
            o[0] = x[0]; o[1] = x[1]; o[2] = x[2]; o[3] = x[3];
        } else {
            o[0] = o[1] = o[2] = o[3] = 0.f;
        }
    }
    static __device__ __forceinline__ void load(const int32_t *p, int k, int K, int *o) {
        if (k < K) {
            const u32x4 x = *reinterpret_cast<const u32x4 *>(p + k);
            o[0] = (int)x[0]; o[1] = (int)x[1]; o[2] = (int)x[2]; o[3] = (int)x[3];
        } else {
            o[0] = o[1] = o[2] = o[3] = -1;
        }
    }
    static __device__ __forceinline__ void store(float *p, int k, int K, const float *v) {  // streaming store
        if (k < K) __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4 *>(p + k));
    }
};

// CH chunks of 64*V slots per row (K <= 64*V*CH).
template <int V, int CH>
__global__ __launch_bounds__(kKlRowsPerBlock * 64) void distill_kl_kernel(
    const float *__restrict__ target, const float *__restrict__ logits, const int32_t *__restrict__ idx,
    int64_t rows, int K, int N, float grad_scale, float *__restrict__ kl_rows, float *__restrict__ dlogits,
    float *__restrict__ partials) {
    constexpr int E = V * CH;
    __shared__ float red_s[kKlRowsPerBlock], red_c[kKlRowsPerBlock];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kKlRowsPerBlock + w;
    float rs = 0.f, rc = 0.f;
    if (row < rows) {
        const float *Tr = target + row * K;
        const float *zr = logits + row * K;
        const int32_t *ir = idx + row * K;
        float tv[E], zv[E];
        int iv[E];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int k = V * lane + 64 * V * c;
            RowIO<V>::load(ir, k, K, iv + V * c);
            RowIO<V>::load(Tr, k, K, tv + V * c);
            RowIO<V>::load(zr, k, K, zv + V * c);
        }
        // log2 domain: y = z * log2(e)
        float ymax = -INFINITY, sumT = 0.f;
        bool vv[E];
        bool any = false;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            vv[e] = iv[e] >= 0 && iv[e] < N;  // slots past K carry -1
            tv[e] = vv[e] ? tv[e] : 0.f;
            zv[e] = vv[e] ? zv[e] * kLog2e : -INFINITY;
            ymax = fmaxf(ymax, zv[e]);
            sumT += tv[e];
            any = any || vv[e];
        }
        float *dr = dlogits ? dlogits + row * K : nullptr;
        if (__ballot(any) != 0) {
            ymax = wave_max(ymax);
            sumT = wave_sum(sumT);
            float qv[E];  // softmax numerators 2^(y - ymax) (0 at invalid slots)
            float se = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                qv[e] = fast_exp2(zv[e] - ymax);
                se += qv[e];
            }
            se = wave_sum(se);
            const float lse2 = ymax + fast_log2(se);  // log2-domain LSE of the valid logits
            const float rse = 1.f / se;
            float kl2 = 0.f;  // KL in log2 units: T (log2 T - log2 Q) with log2 Q = y - lse2
#pragma unroll
            for (int e = 0; e < E; ++e) {
                kl2 += (vv[e] && tv[e] > 0.f) ? tv[e] * (log2_full(tv[e]) - (zv[e] - lse2)) : 0.f;
                zv[e] = grad_scale * (sumT * (qv[e] * rse) - tv[e]);  // gradient (0 at invalid slots)
            }
            const float kl = wave_sum(kl2) * kLn2;
            if (dr) {
#pragma unroll
                for (int c = 0; c < CH; ++c) RowIO<V>::store(dr, V * lane + 64 * V * c, K, zv + V * c);
            }
            if (lane == 0) kl_rows[row] = kl;
            rs = kl;
            rc = 1.f;
        } else {
            if (dr) {
                float zero[V] = {};
#pragma unroll
                for (int c = 0; c < CH; ++c) RowIO<V>::store(dr, V * lane + 64 * V * c, K, zero);
            }
            if (lane == 0) kl_rows[row] = 0.f;
        }
    }
    if (lane == 0) {
        red_s[w] = rs;
        red_c[w] = rc;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float s = 0.f, c = 0.f;
#pragma unroll
        for (int i = 0; i < kKlRowsPerBlock; ++i) {
            s += red_s[i];
            c += red_c[i];
        }
        partials[2 * (size_t)blockIdx.x] = s;
        partials[2 * (size_t)blockIdx.x + 1] = c;
    }
}

// Adds the per-block partials in a fixed order (one block of 4 waves): each thread sums a
// strided set of 16-byte (sum, count, sum, count) loads in order, each wave reduces with
// a fixed xor butterfly, and wave 0 adds the 4 wave totals after the single barrier.
__global__ __launch_bounds__(256) void distill_kl_finalize(const float *__restrict__ partials, int nblk,
                                                           float *__restrict__ stats) {
    __shared__ float ws[4], wc[4];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    float s = 0.f, c = 0.f;
    const int npair2 = nblk >> 1;  // partials are 8-byte aligned pairs: two per 16-byte load
    for (int i = tid; i < npair2; i += 256) {
        const f32x4 v = reinterpret_cast<const f32x4 *>(partials)[i];
        s += v[0] + v[2];
        c += v[1] + v[3];
    }
    if ((nblk & 1) && tid == 0) {
        s += partials[2 * (size_t)(nblk - 1)];
        c += partials[2 * (size_t)(nblk - 1) + 1];
    }
    s = wave_sum(s);
    c = wave_sum(c);
    if (lane == 0) {
        ws[w] = s;
        wc[w] = c;
    }
    __syncthreads();
    if (tid == 0) {
        stats[0] = (ws[0] + ws[1]) + (ws[2] + ws[3]);
        stats[1] = (wc[0] + wc[1]) + (wc[2] + wc[3]);
    }
}

template <int V, int CH>
hipError_t launch_e(const float *target, const float *logits, const int32_t *idx, int64_t rows, int K, int N,
                    float grad_scale, float *kl_rows, float *dlogits, float *stats, float *partials, int nblk,
                    hipStream_t stream) {
    hipLaunchKernelGGL((distill_kl_kernel<V, CH>), dim3(nblk), dim3(kKlRowsPerBlock * 64), 0, stream, target, logits,
                       idx, rows, K, N, grad_scale, kl_rows, dlogits, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(distill_kl_finalize, dim3(1), dim3(256), 0, stream, partials, nblk, stats);
    return hipGetLastError();
}

}  // namespace

// Per-block partials of the allocation-free entry point: one fixed array per GPU, in the
// library's device memory for the life of the process.  Host code never passes the array's
// name to a kernel (in host code it names a host-side stand-in); it resolves the device
// address with hipGetSymbolAddress once per device and passes that.
__device__ __align__(256) float scratch[kNoAllocMaxRows / 8 * 2];

namespace {

static_assert(kKlRowsPerBlock == 8, "scratch holds one (sum, count) pair per 8-row block");
constexpr int kMaxDevices = 64;
std::atomic<float *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (resolved on the first call per device,
// with that device current).
hipError_t scratch_for_current_device(float **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    float *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            void *addr = nullptr;
            e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (addr == nullptr) return hipErrorInvalidSymbol;
            p = reinterpret_cast<float *>(addr);
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

size_t kl_workspace_bytes(int B, int S, int K) {
    (void)K;
    const int64_t rows = (int64_t)B * S;
    const int64_t nblk = (rows + kKlRowsPerBlock - 1) / kKlRowsPerBlock;
    return (size_t)nblk * 2 * sizeof(float);
}

hipError_t launch_distill_kl(const float *target, const float *logits, const int32_t *idx, int B, int S, int K,
                             int N, float grad_scale, float *kl_rows, float *dlogits, float *stats, void *workspace,
                             hipStream_t stream) {
    const int64_t rows = (int64_t)B * S;
    const int nblk = (int)((rows + kKlRowsPerBlock - 1) / kKlRowsPerBlock);
    float *partials = reinterpret_cast<float *>(workspace);
#define SD_K(V, C) launch_e<V, C>(target, logits, idx, rows, K, N, grad_scale, kl_rows, dlogits, stats, partials, nblk, stream)
    if (K % 4 == 0) {  // 16-byte rows and loads
        if (K <= 256) return SD_K(4, 1);
        if (K <= 512) return SD_K(4, 2);
        if (K <= 1024) return SD_K(4, 4);
        if (K <= 2048) return SD_K(4, 8);
        return SD_K(4, 16);
    }
    if (K <= 64) return SD_K(1, 1);
    if (K <= 128) return SD_K(1, 2);
    if (K <= 256) return SD_K(1, 4);
    if (K <= 512) return SD_K(1, 8);
    if (K <= 1024) return SD_K(1, 16);
    if (K <= 2048) return SD_K(1, 32);
    return SD_K(1, 64);
#undef SD_K
}

hipError_t launch_distill_kl_noalloc(const float *target, const float *logits, const int32_t *idx, int B, int S,
                                     int K, int N, float grad_scale, float *kl_rows, float *dlogits, float *stats,
                                     hipStream_t stream) {
    float *partials = nullptr;
    const hipError_t e = scratch_for_current_device(&partials);
    if (e != hipSuccess) return e;
    // every partial the finalize reads is written by this call's first kernel: nothing to clear
    return launch_distill_kl(target, logits, idx, B, S, K, N, grad_scale, kl_rows, dlogits, stats, partials, stream);
}

}  // namespace sd
