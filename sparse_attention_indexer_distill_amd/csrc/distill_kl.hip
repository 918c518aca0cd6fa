// distill_kl.hip -- fused KL(target || softmax(student logits)) with its gradient.
//
// One wave per (b,t) row.  The student softmax runs over the row's valid slots only;
// the forward value and the analytic gradient (sum T) * softmax(z) - T come out of the
// same pass, so nothing is saved between forward and backward (Primus PR
// "perf(deepseek-v4): fuse and enable the indexer distillation loss", commit fusing
// the KL tail with an analytic backward; MaxText PR "Add Indexer Loss [Deepseek v4]",
// review comments: log-softmax KL without epsilon, exact gradient Q - P).
//
// The row is read once from HBM into registers (each lane holds slots lane + 64e), all
// reductions are xor-butterflies inside the wave, and the per-row KL plus a per-block
// (sum, count) partial are written.  A one-block finalize kernel adds the partials in a
// fixed order, so the loss statistics are bitwise reproducible.
#include "sd_device.hpp"
#include "sd_internal.hpp"

namespace sd {
namespace {

constexpr int kKlRowsPerBlock = 4;

template <int EPL>
__global__ __launch_bounds__(kKlRowsPerBlock * 64) void distill_kl_kernel(
    const float *__restrict__ target, const float *__restrict__ logits, const int32_t *__restrict__ idx,
    int64_t rows, int K, int N, float grad_scale, float *__restrict__ kl_rows, float *__restrict__ dlogits,
    float *__restrict__ partials) {
    __shared__ float red_s[kKlRowsPerBlock], red_c[kKlRowsPerBlock];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kKlRowsPerBlock + w;
    float rs = 0.f, rc = 0.f;
    if (row < rows) {
        const float *Tr = target + row * K;
        const float *zr = logits + row * K;
        const int32_t *ir = idx + row * K;
        float tv[EPL], zv[EPL];
        bool vv[EPL];
        float zmax = -INFINITY, sumT = 0.f;
        bool any = false;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const int k = lane + 64 * e;
            const int id = k < K ? ir[k] : -1;
            vv[e] = k < K && id >= 0 && id < N;
            tv[e] = vv[e] ? Tr[k] : 0.f;
            zv[e] = vv[e] ? zr[k] : -INFINITY;
            zmax = fmaxf(zmax, zv[e]);
            sumT += tv[e];
            any = any || vv[e];
        }
        if (__ballot(any) != 0) {
            zmax = wave_max(zmax);
            sumT = wave_sum(sumT);
            float se = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) se += vv[e] ? expf(zv[e] - zmax) : 0.f;
            se = wave_sum(se);
            const float lse = zmax + logf(se);
            float kl = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                kl += (vv[e] && tv[e] > 0.f) ? tv[e] * (logf(tv[e]) - (zv[e] - lse)) : 0.f;
            kl = wave_sum(kl);
            if (dlogits) {
                float *dr = dlogits + row * K;
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    const int k = lane + 64 * e;
                    if (k < K) dr[k] = vv[e] ? grad_scale * (sumT * expf(zv[e] - lse) - tv[e]) : 0.f;
                }
            }
            if (lane == 0) kl_rows[row] = kl;
            rs = kl;
            rc = 1.f;
        } else {
            if (dlogits) {
                float *dr = dlogits + row * K;
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    const int k = lane + 64 * e;
                    if (k < K) dr[k] = 0.f;
                }
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

__global__ __launch_bounds__(256) void distill_kl_finalize(const float *__restrict__ partials, int nblk,
                                                           float *__restrict__ stats) {
    __shared__ float ss[256], sc[256];
    float s = 0.f, c = 0.f;
    for (int i = threadIdx.x; i < nblk; i += 256) {
        s += partials[2 * (size_t)i];
        c += partials[2 * (size_t)i + 1];
    }
    ss[threadIdx.x] = s;
    sc[threadIdx.x] = c;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) {
            ss[threadIdx.x] += ss[threadIdx.x + o];
            sc[threadIdx.x] += sc[threadIdx.x + o];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        stats[0] = ss[0];
        stats[1] = sc[0];
    }
}

template <int EPL>
hipError_t launch_e(const float *target, const float *logits, const int32_t *idx, int64_t rows, int K, int N,
                    float grad_scale, float *kl_rows, float *dlogits, float *stats, float *partials, int nblk,
                    hipStream_t stream) {
    hipLaunchKernelGGL((distill_kl_kernel<EPL>), dim3(nblk), dim3(kKlRowsPerBlock * 64), 0, stream, target, logits,
                       idx, rows, K, N, grad_scale, kl_rows, dlogits, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(distill_kl_finalize, dim3(1), dim3(256), 0, stream, partials, nblk, stats);
    return hipGetLastError();
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
#define SD_K(E) launch_e<E>(target, logits, idx, rows, K, N, grad_scale, kl_rows, dlogits, stats, partials, nblk, stream)
    if (K <= 64) return SD_K(1);
    if (K <= 128) return SD_K(2);
    if (K <= 256) return SD_K(4);
    if (K <= 512) return SD_K(8);
    if (K <= 1024) return SD_K(16);
    if (K <= 2048) return SD_K(32);
    return SD_K(64);
#undef SD_K
}

}  // namespace sd
