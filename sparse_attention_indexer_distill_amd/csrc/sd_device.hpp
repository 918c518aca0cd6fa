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

// Device-scope (sc1) load: served by L2 without allocating in the CU's L1.  Used for row
// gathers, which have no L1 reuse and whose 1 KB-strided rows otherwise pile into a few L1
// sets (tag-conflict stalls).
__device__ __forceinline__ u32x4 buf_load16_l2(rsrc_t r, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 16 /* sc1 */);
}
// The same with a wave-uniform part of the offset in the instruction's scalar offset, so no
// vector add is spent on it.
__device__ __forceinline__ u32x4 buf_load16_l2s(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 16 /* sc1 */);
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

// ---- coalesced row gathers ---------------------------------------------------------
// The memory pipeline merges the addresses of CONSECUTIVE lanes: a 16-row x 64-byte load
// whose 4 consecutive lanes share a row streams at ~27 B/clk/CU on gfx950, but the
// MFMA operand layout (lane l on row l%16) spreads each row over lanes 16 apart and runs
// at ~15.5 B/clk/CU for the same bytes.  So rows are loaded "quad-major" -- lane L holds
// row L/4 -- and moved into the fragment layout (lane l: row l%16, segment l/16) with one
// ds_bpermute per dword.  Within a quad the upper half-wave (rows 8..15) takes the four
// segments in the order 2,3,0,1: the permute's source lanes, 4*(l%16) + ((l/16) ^ 2*(row
// >= 8)), are then distinct modulo 32 in each half-wave, which keeps the permute free of
// LDS bank conflicts (the plain order 4*(l%16) + l/16 hits every bank twice).
__device__ __forceinline__ uint32_t quad_row_lane(int lane) { return (uint32_t)(lane >> 2); }
__device__ __forceinline__ uint32_t quad_seg_bytes(int lane) { return (uint32_t)(16 * ((lane & 3) ^ ((lane >> 4) & 2))); }
__device__ __forceinline__ int quad_to_frag_addr(int lane) {
    return (4 * (lane & 15) + ((lane >> 4) ^ ((lane >> 2) & 2))) << 2;
}
__device__ __forceinline__ u32x4 quad_to_frag(u32x4 v, int addr) {
    u32x4 r;
#pragma unroll
    for (int d = 0; d < 4; ++d) r[d] = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)v[d]);
    return r;
}

// ---- 128-byte row pieces (bf16) -------------------------------------------------------
// With 8 consecutive lanes on a row, one load covers 8 rows x 128 bytes (two 32-element
// chunks, 2p and 2p+1) and streams at ~48 B/clk/CU, against ~27 for 16 rows x 64 bytes.
// A 16-row tile takes two such loads:
//     lo: lane L holds row L/8,     16-byte segment s(L) of the piece
//     hi: lane L holds row 8 + L/8, segment s(L) ^ 4
// with s(L) = (L%8) ^ 2*(L >= 32): the 8 lanes of a row still cover its whole 128-byte line, so
// both loads coalesce the same.  Because hi's segments are lo's with the chunk bit flipped, a
// lane holds chunk 2p data in exactly one of the two registers: lanes with L%8 < 4 in lo, the
// others in hi.  One select per dword therefore gathers each chunk into one register,
//     A = L%8 < 4 ? lo : hi   (chunk 2p, all 16 rows)      B = L%8 < 4 ? hi : lo   (chunk 2p+1)
// and one ds_bpermute per dword moves (row r, segment g) to fragment lane 16g + r.  Source
// lanes (r8 = r%8, hb = r/8, x = 2*(r8 >= 4)), distinct modulo 32 within each half-wave, so
// the permute is free of LDS bank conflicts:
//     f0: 8*r8 + 4*hb + (g ^ x)        f1: 8*r8 + 4*(1-hb) + (g ^ x)
__device__ __forceinline__ int pair_row_lane(int lane) { return lane >> 3; }
__device__ __forceinline__ uint32_t pair_seg_bytes(int lane) { return (uint32_t)(16 * ((lane & 7) ^ ((lane >> 4) & 2))); }
__device__ __forceinline__ uint32_t pair_seg_bytes_hi(int lane) { return pair_seg_bytes(lane) ^ 64u; }

struct PairAddr {
    int a0, a1;  // byte addresses for ds_bpermute
};
__device__ __forceinline__ PairAddr pair_frag_addr(int lane) {
    const int r = lane & 15, g = lane >> 4, r8 = r & 7, hb = r >> 3, gx = g ^ (2 * (r8 >> 2));
    return PairAddr{(8 * r8 + 4 * hb + gx) << 2, (8 * r8 + 4 * (1 - hb) + gx) << 2};
}
__device__ __forceinline__ void pair_frags(const u32x4 &lo, const u32x4 &hi, u32x4 &f0, u32x4 &f1, PairAddr pa,
                                           bool lo_first) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const int A = (int)(lo_first ? lo[d] : hi[d]);
        const int B = (int)(lo_first ? hi[d] : lo[d]);
        f0[d] = (uint32_t)__builtin_amdgcn_ds_bpermute(pa.a0, A);
        f1[d] = (uint32_t)__builtin_amdgcn_ds_bpermute(pa.a1, B);
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

// Cross-row exchanges on the VALU (gfx950 v_permlane16_swap / v_permlane32_swap, no LDS
// traffic).  With both operands equal to v, the pair returned in lane l is
// {v[l & ~16], v[l | 16]} (16-lane swap) or {v[l & 31], v[l | 32]} (32-lane swap): the lane's
// own value and its partner's at xor 16 or xor 32, in the same order in both partners, so
// both get bitwise equal results.
__device__ __forceinline__ void xrow16(float v, float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v),
                                                    false, false);
    a = __builtin_bit_cast(float, (uint32_t)r[0]);
    b = __builtin_bit_cast(float, (uint32_t)r[1]);
}
__device__ __forceinline__ void xrow32(float v, float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v),
                                                    false, false);
    a = __builtin_bit_cast(float, (uint32_t)r[0]);
    b = __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Combine the four DPP rows holding the same column (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float cols4_max(float v) {
    float a, b;
    xrow16(v, a, b);
    xrow32(fmaxf(a, b), a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float cols4_sum(float v) {
    float a, b;
    xrow16(v, a, b);
    xrow32(a + b, a, b);
    return a + b;
}

// Value of DPP row R (lanes 16R + l%16) of v in every lane, for R = 0..3.
__device__ __forceinline__ void rows_bcast(float v, float (&out)[4]) {
    float e, o;
    xrow16(v, e, o);           // rows 0/2 and rows 1/3 of v, by half
    xrow32(e, out[0], out[2]);
    xrow32(o, out[1], out[3]);
}

// Butterfly over the 16 lanes of a DPP row with partners x^8, x^7, x^2, x^1 (row_ror:8,
// row_half_mirror, quad_perm [2,3,0,1], quad_perm [1,0,3,2]); the pairings generate the
// whole row, and each pair adds or compares the same two values, so every lane of the row
// ends with the same result.
template <bool MAX>
__device__ __forceinline__ float row16_butterfly(float v) {
    float p;
    p = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));
    v = MAX ? fmaxf(v, p) : v + p;
    p = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xf, 0xf, false));
    v = MAX ? fmaxf(v, p) : v + p;
    p = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4e, 0xf, 0xf, false));
    v = MAX ? fmaxf(v, p) : v + p;
    p = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xb1, 0xf, 0xf, false));
    v = MAX ? fmaxf(v, p) : v + p;
    return v;
}

__device__ __forceinline__ float wave_max(float v) { return cols4_max(row16_butterfly<true>(v)); }
__device__ __forceinline__ float wave_sum(float v) { return cols4_sum(row16_butterfly<false>(v)); }

// exp2 / log2 on the hardware transcendental unit.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// log2 of a positive finite value, exact for subnormal inputs too: v_log_f32 takes no
// subnormal operands, so values below 2^-126 are scaled by 2^32 first (an exact power-of-two
// scaling) and 32 is subtracted from the result.
__device__ __forceinline__ float log2_full(float x) {
    const bool sub = x < 1.17549435e-38f;
    return fast_log2(sub ? x * 4294967296.0f : x) - (sub ? 32.0f : 0.0f);
}

// log2(2^a + 2^b), with -inf handled.
__device__ __forceinline__ float logaddexp2(float a, float b) {
    float m = fmaxf(a, b);
    if (m == -INFINITY) return -INFINITY;
    return m + fast_log2(fast_exp2(a - m) + fast_exp2(b - m));
}

}  // namespace sd
