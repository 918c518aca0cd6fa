// sd_device.hpp -- device-side building blocks for the gfx950 (CDNA4) kernels.
//
// Fragment convention used by every kernel.  The contraction dimension D is walked in
// chunks of 32 elements.  In chunk c, lane l of a wave holds, for one 16-row operand
// tile, the 8 consecutive elements d = 32c + 8*(l/16) + j (j = 0..7) of row l%16.  For
// bf16 this is exactly the A/B operand of v_mfma_f32_16x16x32_bf16; for fp32 the same 8
// elements feed eight v_mfma_f32_16x16x4_f32 steps (element j in step j), so the pairing
// of A and B elements is identical in both cases.  The 16x16 fp32 result of either form
// sits in lane l as rows 4*(l/16)+i (i = 0..3) of column l%16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sd {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element-type traits: DT is the public dtype code (0 = bf16, 1 = fp32).
template <int DT> struct Elem;
template <> struct Elem<0> {
    using frag_t = u32x4;  // 8 x bf16 = 16 bytes
    static constexpr int bytes = 2;
};
template <> struct Elem<1> {
    using frag_t = f32x8;  // 8 x fp32 = 32 bytes
    static constexpr int bytes = 4;
};

template <int DT>
__device__ __forceinline__ typename Elem<DT>::frag_t load_frag(const void *base, size_t elem_off) {
    using F = typename Elem<DT>::frag_t;
    return *reinterpret_cast<const F *>(reinterpret_cast<const char *>(base) + elem_off * Elem<DT>::bytes);
}

template <int DT>
__device__ __forceinline__ typename Elem<DT>::frag_t zero_frag() {
    typename Elem<DT>::frag_t z;
#pragma unroll
    for (int i = 0; i < (int)(sizeof(z) / 4); ++i) reinterpret_cast<uint32_t *>(&z)[i] = 0u;
    return z;
}

// acc += A(16 rows x 32 k) * B(32 k x 16 cols) for one fragment pair.
template <int DT>
__device__ __forceinline__ f32x4 mfma_frag(typename Elem<DT>::frag_t a, typename Elem<DT>::frag_t b, f32x4 acc);

template <>
__device__ __forceinline__ f32x4 mfma_frag<0>(u32x4 a, u32x4 b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x4 mfma_frag<1>(f32x8 a, f32x8 b, f32x4 acc) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], acc, 0, 0, 0);
    return acc;
}

// ---- cross-lane reductions -------------------------------------------------------
// Sum over the 16 lanes of a DPP row (lanes sharing l/16); every lane gets the total.
__device__ __forceinline__ float row16_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));  // row_ror:8
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xf, 0xf, false));  // row_ror:4
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xf, 0xf, false));  // row_ror:2
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xf, 0xf, false));  // row_ror:1
    return v;
}

// Combine the four DPP rows holding the same column (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float cols4_max(float v) {
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}
__device__ __forceinline__ float cols4_sum(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// exp2 / log2 on the hardware transcendental unit.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// log2(2^a + 2^b), with -inf handled.
__device__ __forceinline__ float logaddexp2(float a, float b) {
    float m = fmaxf(a, b);
    if (m == -INFINITY) return -INFINITY;
    return m + fast_log2(fast_exp2(a - m) + fast_exp2(b - m));
}

}  // namespace sd
