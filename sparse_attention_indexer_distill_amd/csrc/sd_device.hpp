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

// ---- buffer loads ------------------------------------------------------------------
// Raw buffer resources give 32-bit per-lane byte offsets and hardware bounds checking:
// any access at or beyond `bytes` reads as zero.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

// Device-scope (sc1) load: served by L2 without allocating in the CU's L1.  Used for row
// gathers, which have no L1 reuse and whose 1 KB-strided rows otherwise pile into a few L1
// sets (tag-conflict stalls).
__device__ __forceinline__ u32x4 buf_load16_l2(rsrc_t r, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 16 /* sc1 */);
}

// One fragment (8 elements) of a row at byte offset `byte_off`.
template <int DT>
__device__ __forceinline__ typename Elem<DT>::frag_t buf_load_frag(rsrc_t r, uint32_t byte_off);
template <>
__device__ __forceinline__ u32x4 buf_load_frag<0>(rsrc_t r, uint32_t byte_off) {
    return buf_load16_l2(r, byte_off);
}
template <>
__device__ __forceinline__ f32x8 buf_load_frag<1>(rsrc_t r, uint32_t byte_off) {
    const f32x4 lo = __builtin_bit_cast(f32x4, buf_load16_l2(r, byte_off));
    const f32x4 hi = __builtin_bit_cast(f32x4, buf_load16_l2(r, byte_off + 16));
    return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Direct buffer -> LDS load of 16 bytes per lane: lane l's bytes land at lds + 16*l.
// `lds` must be wave-uniform.  Completion is tracked by vmcnt (wait before reading).
__device__ __forceinline__ void buf_load_lds16(rsrc_t r, void *lds, uint32_t byte_off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)lds, 16, byte_off, 0, 0, 0);
}

// A fragment stored in LDS as NH = sizeof(frag)/16 planes of 64 lanes x 16 bytes.
template <int DT>
__device__ __forceinline__ typename Elem<DT>::frag_t lds_frag(const u32x4 *units, int unit);
template <>
__device__ __forceinline__ u32x4 lds_frag<0>(const u32x4 *units, int unit) {
    return units[unit];
}
template <>
__device__ __forceinline__ f32x8 lds_frag<1>(const u32x4 *units, int unit) {
    const f32x4 lo = __builtin_bit_cast(f32x4, units[unit]);
    const f32x4 hi = __builtin_bit_cast(f32x4, units[unit + 64]);
    return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// ---- coalesced row gathers ---------------------------------------------------------
// The memory pipeline merges the addresses of CONSECUTIVE lanes: a 16-row x 64-byte load
// whose 4 consecutive lanes share a row streams at ~27 B/clk/CU on gfx950, but the
// MFMA operand layout (lane l on row l%16) spreads each row over lanes 16 apart and runs
// at ~15.5 B/clk/CU for the same bytes.  So rows are loaded "quad-major" -- lane L holds
// row L/4, 16-byte segment L%4 of the chunk -- and moved into the fragment layout (lane
// l: row l%16, segment l/16) with one ds_bpermute per dword (source lane 4*(l%16)+l/16).
__device__ __forceinline__ uint32_t quad_row_lane(int lane) { return (uint32_t)(lane >> 2); }
__device__ __forceinline__ uint32_t quad_seg_bytes(int lane) { return (uint32_t)(16 * (lane & 3)); }
__device__ __forceinline__ int quad_to_frag_addr(int lane) { return (4 * (lane & 15) + (lane >> 4)) << 2; }
__device__ __forceinline__ u32x4 quad_to_frag(u32x4 v, int addr) {
    u32x4 r;
#pragma unroll
    for (int d = 0; d < 4; ++d) r[d] = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)v[d]);
    return r;
}

// ---- coalesced gather of 16-row operand tiles (bf16) ------------------------------
// A 16x16x32 operand tile puts 4 lanes on each row (64 bytes of a row per load), which
// costs one 128-byte L2 request per row and half-uses it.  Instead, the two chunks of a
// 128-byte line (chunks 2p and 2p+1) of a 16-row tile are fetched with two loads that
// each cover 8 rows x 128 bytes:
//     load lo: lane (r = l/16, x = l%16) holds row x%8,     16-byte segment r + 4*(x/8)
//     load hi: lane (r, x)               holds row 8 + x%8, segment r + 4*(x/8)
// The fragment of chunk 2p (segments 0..3) is lo for x < 8 and hi rotated by 8 lanes
// within the 16-lane row for x >= 8; chunk 2p+1 (segments 4..7) is lo rotated by 8 for
// x < 8 and hi for x >= 8.  Byte offset of a lane's segment inside the line:
__device__ __forceinline__ uint32_t pair_seg_bytes(int lane) { return (uint32_t)(16 * ((lane >> 4) + 4 * ((lane >> 3) & 1))); }

// In place: lo becomes the fragment of chunk 2p, hi the fragment of chunk 2p+1
// (low_half: lane%16 < 8).  row_ror:8 never leaves the 16-lane row, so bound_ctrl
// costs nothing and spares the move of an "old" value: two VALU ops per dword.
__device__ __forceinline__ uint32_t ror8(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, true);  // row_ror:8
}
__device__ __forceinline__ void pair_to_frags(u32x4 &lo, u32x4 &hi, bool low_half) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const uint32_t rl = ror8(lo[v]), rh = ror8(hi[v]);
        lo[v] = low_half ? lo[v] : rh;
        hi[v] = low_half ? rl : hi[v];
    }
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
