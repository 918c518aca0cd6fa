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
// staged once in LDS.  The valid slots of the row are compacted (stable, slot order) into
// a list in LDS; 16-slot tiles of that list are dealt to the waves (in pairs when the window
// part is computed here too, else round-robin), so invalid (-1) slots cost no MFMA work
// wherever they sit.  Each wave gathers its rows from L2 in
// 128-byte pieces (8 consecutive lanes on a row, the layout the memory pipeline merges),
// regroups them into MFMA operand fragments with one select and one ds_bpermute per dword, and
// accumulates
//     C[slot][head] (16x16 tiles) = pool_row . q_head
// for all heads, keeping every score of its slots in registers.  The epilogue has one
// barrier: per-wave head statistics cross waves through LDS, the row's joint mass follows
// from them without a second exchange, and the head sum of p[h,k] = exp(c[h,k] - full_h)
// is a 16-lane DPP transpose-reduction.  Nothing but the target row is written.
#include <float.h>
#include <math.h>

#include "sd_device.hpp"
#include "sd_internal.hpp"

namespace sd {
namespace {

// Queries of one token in LDS.
// bf16: pair-major -- the 16 heads x 64 elements of (chunk pair p, head tile ht) fill the
//   2 KB block p*HT + ht; head r of the tile owns the 128 bytes at 128r, holding its eight
//   16-byte segments x (chunk 2p: x = 0..3, chunk 2p+1: x = 4..7) at slot x ^ ((r>>1)&7).
//   A fragment read (lane l: head l%16, segment 4*(c%2) + l/16) is then free of LDS bank
//   conflicts (measured; the 64-byte-row layouts tried before paid 4 extra cycles per
//   read), and all blocks sit at constant offsets from two per-lane bases (one per chunk
//   parity).  An odd chunk count stages a zero chunk to complete the last pair.
// fp32: head row h at byte h*RS (RS = D*4 + 16); fragment unit (ht, c) at row
//   16*ht + l%16, byte (32c + 8*(l/16))*4.
__device__ __forceinline__ int qrow_stride(int D, int EB) { return D * EB + 16; }
__device__ __forceinline__ int q_lane_bytes(int lane, int parity) {
    const int r = lane & 15;
    return 128 * r + 16 * ((4 * parity + (lane >> 4)) ^ ((r >> 1) & 7));
}
template <int HT>
__device__ __forceinline__ int q_bytes(int DT, int D) {
    return DT == 0 ? 2048 * HT * (((D >> 5) + 1) >> 1) : 16 * HT * qrow_stride(D, 4);
}

// bf16 fragment of block u (= pair*HT + ht) from a lane base qb + q_lane_bytes(lane, parity).
__device__ __forceinline__ u32x4 q_unit(const unsigned char *qlane, int u) {
    return *reinterpret_cast<const u32x4 *>(qlane + (u << 11));
}

template <int DT, int HT>
__device__ __forceinline__ typename Elem<DT>::frag_t q_frag(const unsigned char *qb, int RS, int ht, int c, int lane) {
    if constexpr (DT == 0) {
        return q_unit(qb + q_lane_bytes(lane, c & 1), (c >> 1) * HT + ht);
    } else {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(qb + (ht * 16 + (lane & 15)) * RS + (32 * c + 8 * (lane >> 4)) * 4);
        const f32x4 lo = __builtin_bit_cast(f32x4, p[0]), hi = __builtin_bit_cast(f32x4, p[1]);
        return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
}


// Scores of MY slot tiles against all heads, streaming D in 32-element chunks.  The
// gathered pool fragments (buffer loads) and the query fragments (LDS) of chunk c+1 are
// in flight while chunk c's MFMAs run.  MY is a compile-time count, so the loop has no
// per-tile branches.
//
// cr rotates the chunk order (chunk c is D-chunk (c + cr) mod nch): waves of a token and
// tokens in flight start at different offsets of their rows, which spreads the gathers
// over the L2 channels (7% at D = 512).  The sum order stays fixed per (token, wave).
template <int DT, int HT, int MY, int KT>
__device__ __forceinline__ void score_tiles(f32x4 (&acc)[KT][HT], const unsigned char *__restrict__ qb, int RS, rsrc_t pool,
                                            const uint32_t (&off)[KT], int nch, int cr, int lane) {
    using frag_t = typename Elem<DT>::frag_t;
    constexpr uint32_t CB = 32 * Elem<DT>::bytes;  // bytes of one 32-element chunk of a row
    frag_t a0[MY], a1[MY], b0[HT], b1[HT];
    auto rot = [&](int c) {
        const int cc = c + cr;
        return cc >= nch ? cc - nch : cc;
    };
    auto load_a = [&](frag_t(&a)[MY], int c) {
#pragma unroll
        for (int l = 0; l < MY; ++l) a[l] = buf_load_frag<DT>(pool, off[l] + (uint32_t)rot(c) * CB);
    };
    auto load_b = [&](frag_t(&bq)[HT], int c) {
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) bq[ht] = q_frag<DT, HT>(qb, RS, ht, rot(c), lane);
    };
    const int paddr = quad_to_frag_addr(lane);
    auto mma = [&](frag_t(&a)[MY], const frag_t(&bq)[HT]) {
        if constexpr (DT == 0) {  // bf16 rows were loaded quad-major
#pragma unroll
            for (int l = 0; l < MY; ++l) a[l] = quad_to_frag(a[l], paddr);
        }
#pragma unroll
        for (int l = 0; l < MY; ++l)
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) acc[l][ht] = mfma_frag<DT>(a[l], bq[ht], acc[l][ht]);
    };
    const int c0 = nch & 1;  // an odd chunk count runs its first chunk unpipelined
    if (c0) {
        load_a(a0, 0);
        load_b(b0, 0);
        mma(a0, b0);
    }
    if (c0 >= nch) return;
    load_a(a0, c0);
    load_b(b0, c0);
    int c = c0;
    for (; c + 2 < nch; c += 2) {  // steady state: no branches between loads and MFMAs
        load_a(a1, c + 1);
        load_b(b1, c + 1);
        mma(a0, b0);
        load_a(a0, c + 2);
        load_b(b0, c + 2);
        mma(a1, b1);
    }
    load_a(a1, c + 1);  // last pair
    load_b(b1, c + 1);
    mma(a0, b0);
    mma(a1, b1);
}

// fp32 scores in passes of at most two tiles.  Each head tile's query fragment is read
// from LDS just before its MFMAs through a two-deep ring, so two tiles' row fragments (double
// buffered over chunks), two query fragments and the accumulators stay within the 128
// VGPRs a wave has when 16 waves share a workgroup.
template <int HT, int MY, int KT>
__device__ __forceinline__ void score_f32(f32x4 (&acc)[KT][HT], const unsigned char *__restrict__ qb, int RS,
                                          rsrc_t pool, const uint32_t (&off)[KT], int nch, int lane) {
    constexpr uint32_t CB = 32 * 4;  // bytes of one 32-element fp32 chunk of a row
#pragma unroll
    for (int l0 = 0; l0 < MY; l0 += 2) {
        f32x8 a0[2], a1[2];
        auto load = [&](f32x8(&a)[2], int c) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
                if (l0 + t < MY) a[t] = buf_load_frag<1>(pool, off[l0 + t] + (uint32_t)c * CB);
        };
        auto mma = [&](const f32x8(&a)[2], int c) {
            f32x8 b[2];
            b[0] = q_frag<1, HT>(qb, RS, 0, c, lane);
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                if (ht + 1 < HT) b[(ht + 1) & 1] = q_frag<1, HT>(qb, RS, ht + 1, c, lane);
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    if (l0 + t < MY) acc[l0 + t][ht] = mfma_frag<1>(a[t], b[ht & 1], acc[l0 + t][ht]);
            }
        };
        load(a0, 0);
        int c = 0;
        for (; c + 1 < nch; c += 2) {
            load(a1, c + 1);
            mma(a0, c);
            if (c + 2 < nch) load(a0, c + 2);
            mma(a1, c + 1);
        }
        if (c < nch) mma(a0, c);
    }
}

template <int HT, int KT, int MY = KT>
__device__ __forceinline__ void score_dispatch_f32(int my, f32x4 (&acc)[KT][HT], const unsigned char *__restrict__ qb,
                                                   int RS, rsrc_t pool, const uint32_t (&off)[KT], int nch, int lane) {
    if (my == MY) {
        score_f32<HT, MY, KT>(acc, qb, RS, pool, off, nch, lane);
    } else if constexpr (MY > 1) {
        score_dispatch_f32<HT, KT, MY - 1>(my, acc, qb, RS, pool, off, nch, lane);
    }
}

// bf16 scores from 128-byte row pieces (two chunks per load pair; see pair_frags).  The
// tiles are scored PT at a time, so only PT tiles' raw loads and fragments are live next
// to the accumulators; the loads of piece p + DEPTH are issued as soon as piece p has been
// permuted (DEPTH pieces in flight, in a ring of raw registers), and each query fragment is
// read from LDS once per chunk and pass.  With an odd chunk count the last piece is half
// used (its upper 64 bytes belong to the next row, or fall past the buffer end and read as
// zero).  cr rotates the piece order per wave and token, which spreads the gathers over the
// L2 channels.
// SOFF (even chunk counts only): the piece offset goes in the load's scalar offset.  Every
// access of a load then lies inside one pool row; with an odd chunk count the half-used last
// piece reaches past the row, and those loads keep the whole offset in the vector operand,
// which the buffer's range check covers (reads past the pool's end return zero).
template <int HT, int MY, int KT, int PT, bool SOFF, int DEPTH>
__device__ __forceinline__ void score_pairs(f32x4 (&acc)[KT][HT], const unsigned char *__restrict__ qb,
                                            rsrc_t pool, const uint32_t (&olo)[KT], const uint32_t (&ohi)[KT],
                                            int nch, int cr, int lane) {
    const int np = (nch + 1) >> 1;
    const PairAddr pa = pair_frag_addr(lane);
    const bool lo_first = (lane & 4) == 0;  // this lane's chunk-2p dword is in lo (else in hi)
    const unsigned char *qlane0 = qb + q_lane_bytes(lane, 0), *qlane1 = qb + q_lane_bytes(lane, 1);
    auto rot = [&](int p) {
        const int pp = p + cr;
        return pp >= np ? pp - np : pp;
    };
#pragma unroll
    for (int l0 = 0; l0 < MY; l0 += PT) {
        u32x4 lo[DEPTH][PT], hi[DEPTH][PT];
        auto load = [&](u32x4(&l)[PT], u32x4(&h)[PT], int p) {
            const uint32_t pb = (uint32_t)__builtin_amdgcn_readfirstlane(rot(p) * 128);  // wave-uniform
#pragma unroll
            for (int t = 0; t < PT; ++t) {
                if (l0 + t < MY) {
                    if constexpr (SOFF) {
                        l[t] = buf_load16_l2s(pool, olo[l0 + t], pb);
                        h[t] = buf_load16_l2s(pool, ohi[l0 + t], pb);
                    } else {
                        l[t] = buf_load16_l2(pool, olo[l0 + t] + pb);
                        h[t] = buf_load16_l2(pool, ohi[l0 + t] + pb);
                    }
                }
            }
        };
        auto step = [&](u32x4(&l)[PT], u32x4(&h)[PT], int p) {
            u32x4 f0[PT], f1[PT];
#pragma unroll
            for (int t = 0; t < PT; ++t)
                if (l0 + t < MY) pair_frags(l[t], h[t], f0[t], f1[t], pa, lo_first);
            const int c = 2 * rot(p);
            if (p + DEPTH < np) load(l, h, p + DEPTH);
            if (!SOFF && c + 1 >= nch) {  // half piece (odd chunk counts only): chunk c+1 is the
#pragma unroll                                // zero padding chunk of the staged queries
                for (int t = 0; t < PT; ++t) f1[t] = u32x4{0u, 0u, 0u, 0u};
            }
            // query blocks of the pair: chunk c from the even-parity base, c+1 from the odd one,
            // head tile ht at ht * 2 KB; reads run two ahead
            const int qoff = (c >> 1) * HT << 11;
            const unsigned char *qc0 = qlane0 + qoff, *qc1 = qlane1 + qoff;
            auto qread = [&](int u) { return u < HT ? q_unit(qc0, u) : q_unit(qc1, u - HT); };
            u32x4 bq[2];
            bq[0] = qread(0);
            bq[1] = qread(1);
#pragma unroll
            for (int u = 0; u < 2 * HT; ++u) {
                const u32x4 b = bq[u & 1];
                if (u + 2 < 2 * HT) bq[u & 1] = qread(u + 2);
#pragma unroll
                for (int t = 0; t < PT; ++t)
                    if (l0 + t < MY) acc[l0 + t][u % HT] = mfma_frag<0>(u < HT ? f0[t] : f1[t], b, acc[l0 + t][u % HT]);
            }
        };
#pragma unroll
        for (int s = 0; s < DEPTH; ++s)
            if (s < np) load(lo[s], hi[s], s);
        int p = 0;
        for (; p + DEPTH <= np; p += DEPTH) {  // steady state: ring slot s holds piece p + s
#pragma unroll
            for (int s = 0; s < DEPTH; ++s) step(lo[s], hi[s], p + s);
        }
#pragma unroll
        for (int s = 0; s < DEPTH; ++s)
            if (p + s < np) step(lo[s], hi[s], p + s);
    }
}

template <int HT, int KT, int PT, bool SOFF, int DEPTH, int MY = KT>
__device__ __forceinline__ void score_dispatch_pairs(int my, f32x4 (&acc)[KT][HT], const unsigned char *__restrict__ qb,
                                                     rsrc_t pool, const uint32_t (&olo)[KT],
                                                     const uint32_t (&ohi)[KT], int nch, int cr, int lane) {
    if (my == MY) {
        score_pairs<HT, MY, KT, PT, SOFF, DEPTH>(acc, qb, pool, olo, ohi, nch, cr, lane);
    } else if constexpr (MY > 1) {
        score_dispatch_pairs<HT, KT, PT, SOFF, DEPTH, MY - 1>(my, acc, qb, pool, olo, ohi, nch, cr, lane);
    }
}

template <int DT, int HT, int KT, int MY = KT>
__device__ __forceinline__ void score_dispatch(int my, f32x4 (&acc)[KT][HT], const unsigned char *__restrict__ qb, int RS,
                                               rsrc_t pool, const uint32_t (&off)[KT], int nch, int cr, int lane) {
    if (my == MY) {
        score_tiles<DT, HT, MY, KT>(acc, qb, RS, pool, off, nch, cr, lane);
    } else if constexpr (MY > 1) {
        score_dispatch<DT, HT, KT, MY - 1>(my, acc, qb, RS, pool, off, nch, cr, lane);
    }
}

// Cooperative staging of a token's queries straight from HBM into LDS; heads >= H read as
// zero.  bf16: two instructions per 2 KB block (chunk pair, head tile) of the pair-major
// layout, 8 consecutive lanes on each head's 128 bytes.  fp32: each instruction moves up to
// 1 KB of one head row.  The loads complete asynchronously (vmcnt); wait before reading.
template <int DT, int HT, int NW>
__device__ __forceinline__ void stage_queries(const void *q, int64_t bt, int H, int D, unsigned char *qb, int w,
                                              int lane) {
    constexpr int EB = Elem<DT>::bytes;
    const int rowb = D * EB;
    const rsrc_t qr = make_rsrc(reinterpret_cast<const char *>(q) + (size_t)bt * H * D * EB, (uint32_t)(H * D * EB));
    if constexpr (DT == 0) {
        // two instructions per 2 KB block, 8 heads x 128 bytes each (8 lanes to a row)
        const int nch = D >> 5, npair = (nch + 1) >> 1;
        const int rin = lane >> 3;
        for (int u = w; u < npair * HT * 2; u += NW) {
            const int blk = u >> 1, half = u & 1;
            const int p = blk / HT, r = 8 * half + rin, h = 16 * (blk - p * HT) + r;
            const int x = (lane & 7) ^ ((r >> 1) & 7);  // segment landing at slot lane&7
            const bool ok = h < H && 2 * p + (x >> 2) < nch;  // odd nch: the pair's 2nd chunk is zero
            const uint32_t voff = ok ? (uint32_t)(h * rowb + 128 * p + 16 * x) : 0x80000000u;
            buf_load_lds16(qr, qb + (u << 10), voff);
        }
    } else {
        const int RS = qrow_stride(D, EB);
        const int npiece = (rowb + 1023) >> 10;
        for (int u = w; u < 16 * HT * npiece; u += NW) {
            const int h = u / npiece, o = (u - h * npiece) << 10;
            if (o + 16 * lane < rowb) {
                const uint32_t voff = h < H ? (uint32_t)(h * rowb + o + 16 * lane) : 0x80000000u;
                buf_load_lds16(qr, qb + h * RS + o, voff);
            }
        }
    }
}

// Stable compaction of the valid slots of a row (slot order kept) by the whole workgroup,
// one barrier.  Invalid slots get target 0 here.  Returns the valid count (uniform).
template <int NW, int KP>
__device__ __forceinline__ int compact_slots(const int32_t *idr, int K, int N, float *Tr, int32_t *crow,
                                             int32_t *cslot, int *wcnt, int tid, int w, int lane) {
    int v[KP];
    bool ok[KP];
    int pre[KP];
#pragma unroll
    for (int pss = 0; pss < KP; ++pss) {
        const int k = pss * NW * 64 + tid;
        v[pss] = k < K ? idr[k] : -1;
    }
#pragma unroll
    for (int pss = 0; pss < KP; ++pss) {
        const int k = pss * NW * 64 + tid;
        ok[pss] = k < K && v[pss] >= 0 && v[pss] < N;
        if (k < K && !ok[pss]) Tr[k] = 0.f;
        const uint64_t bal = __ballot(ok[pss]);
        pre[pss] = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        if (lane == 0) wcnt[pss * NW + w] = __popcll(bal);
    }
    __syncthreads();
    int base = 0;
#pragma unroll
    for (int pss = 0; pss < KP; ++pss) {
        int off = base, tot = 0;
        for (int i = 0; i < NW; ++i) {
            const int c = wcnt[pss * NW + i];
            off += i < w ? c : 0;
            tot += c;
        }
        if (ok[pss]) {
            crow[off + pre[pss]] = v[pss];
            cslot[off + pre[pss]] = pss * NW * 64 + tid;
        }
        base += tot;
    }
    return base;
}

// ---- epilogue of one token, shared by the kernels below ----------------------------
// Wave w holds my slot tiles of the compacted list, its l-th being TileMap::of(l) (the rest of
// acc at -inf); lane (g, x) = (lane/16, lane%16) holds rows 4g+i of each tile for heads 16ht+x.
//
// The fused kernel deals slot tiles to the waves in pairs (tiles 2p, 2p+1 to one wave), so
// each pass of the score loop over two tiles is full and every query fragment read from LDS
// feeds two MFMAs; pairs go to the last wave first, as the first waves hold the window tiles.
// The three-call kernel deals them round-robin (pairs cost it a register spill at 16 waves).
// The l-th tile of wave w is t0 + (l/2) s2 + (l%2) s1.
struct TileMap {
    int t0, s1, s2;
    __device__ __forceinline__ int of(int l) const { return t0 + (l >> 1) * s2 + (l & 1) * s1; }
};

// Round-robin dealing (tiles w, w+NW, w+2NW, ...).
template <int NW>
__device__ __forceinline__ TileMap slot_tiles_rr(int ntiles, int w, int &my) {
    my = ntiles > w ? (ntiles - w + NW - 1) / NW : 0;
    return TileMap{w, NW, 2 * NW};
}

// Pair dealing: the tiles of wave w among ntiles and their count (one at a time for KT = 1).
template <int KT, int NW>
__device__ __forceinline__ TileMap slot_tiles(int ntiles, int w, int &my) {
    if constexpr (KT == 1) {
        my = ntiles > w ? 1 : 0;
        return TileMap{w, 0, 0};
    } else {
        const int p0 = NW - 1 - w;  // this wave's pairs: p0, p0 + NW, ...
        my = 0;
#pragma unroll
        for (int j = 0; j < KT / 2; ++j) {
            const int r = ntiles - 2 * (p0 + NW * j);
            my += r < 0 ? 0 : (r > 2 ? 2 : r);
        }
        return TileMap{2 * p0, 1, 2 * NW};
    }
}

// Per-head maximum and sum of exp2 over this wave's slots (log2 domain, scale > 0),
// published in red_m/red_s laid out [wave][head%16][head tile].  Padding rows of the
// partial last tile (at most one per wave) are set to -inf first, so every later step
// sees only real slots.  On return acc holds exp2(c - mloc).
template <int HT, int KT, int NW>
__device__ __forceinline__ void epi_stats(f32x4 (&acc)[KT][HT], float (&mloc)[HT], int my, int nv, TileMap tm,
                                          int w, int lane, float scale_log2, float *red_m, float *red_s) {
    const int x = lane & 15, prow = 4 * (lane >> 4);
#pragma unroll
    for (int l = 0; l < KT; ++l) {
        const int base = 16 * tm.of(l);
        if (l < my && base + 16 > nv) {  // uniform: the partial tile
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool pad = base + prow + i >= nv;
#pragma unroll
                for (int ht = 0; ht < HT; ++ht) acc[l][ht][i] = pad ? -INFINITY : acc[l][ht][i];
            }
        }
    }
    float sloc[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        float mx = -INFINITY;
#pragma unroll
        for (int l = 0; l < KT; ++l)
            mx = fmaxf(mx, fmaxf(fmaxf(acc[l][ht][0], acc[l][ht][1]), fmaxf(acc[l][ht][2], acc[l][ht][3])));
        mloc[ht] = cols4_max(mx) * scale_log2;  // -inf for a wave without tiles
    }
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const float nm = mloc[ht] == -INFINITY ? 0.f : -mloc[ht];
        float sum = 0.f;
#pragma unroll
        for (int l = 0; l < KT; ++l)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = fast_exp2(fmaf(acc[l][ht][i], scale_log2, nm));
                acc[l][ht][i] = e;
                sum += e;
            }
        sloc[ht] = cols4_sum(sum);
    }
    if (lane < 16) {
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            red_m[(w * 16 + x) * HT + ht] = mloc[ht];
            red_s[(w * 16 + x) * HT + ht] = sloc[ht];
        }
    }
}

// One butterfly step of a 16-lane transpose-reduction: lanes whose bit `bit` is clear keep
// the first half of their n values, the others the second half, each adding what its
// partner (the lane the DPP control reads from, which differs in that bit) sends.
template <int CTRL, int N>
__device__ __forceinline__ void tr_step(float (&v)[16], bool hi) {
#pragma unroll
    for (int k = 0; k < N / 2; ++k) {
        const float a = v[k], b = v[k + N / 2];
        const float keep = hi ? b : a, send = hi ? a : b;
        v[k] = keep + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, send), CTRL,
                                                                            0xf, 0xf, false));
    }
}

// After the barrier that publishes red_m/red_s: the target row of this wave's slots.
//   full_h = log2(sum_k 2^c_hk + 2^(nc_h log2 e))  (lane (g, x) reduces head 16g+x over waves)
//   row total sum_k m_k = sum_h 2^(clse_h - full_h), clse_h = log2 sum_k 2^c_hk, which needs
//   no further exchange between waves
//   T_k = sum_h exp2(c_hk - mloc_h) * 2^(mloc_h - full_h - lmax) / max(total', 2^(floor - lmax))
//   with lmax = max_h (clse_h - full_h) and total' = sum_h 2^(clse_h - full_h - lmax) in [1, H]
// Shifting every head's log-share by the largest one keeps the row total and the weights in
// range however small the row's mass is (below float32 tiny the floor term wins and still
// scales exactly), and the shifted exponents of heads near the largest are exact
// differences of nearby floats, so a row whose target is a single slot still sums to 1
// within an ulp even when the log-masses are large (a sink far above the logits).  The
// head sum is a 16-lane
// transpose-reduction: afterwards lane (g, x) holds T of row 4g + (x%4) of tile x/4 and
// stores it at its slot.  nc: the natural-log nc_lse of head 16*min(g, HT-1)+x (ignored when
// has_nc is false).
template <int HT, int KT, int NW>
__device__ __forceinline__ void epi_target(const f32x4 (&acc)[KT][HT], const float (&mloc)[HT], int my, int nv,
                                           TileMap tm, int lane, int H, bool has_nc, float nc, float floor_log2, const float *red_m,
                                           const float *red_s, const int32_t *cslot, float *Tr) {
    static_assert(KT <= 4 || KT % 4 == 0, "tiles are reduced in groups of four");
    const int x = lane & 15, g = lane >> 4;
    const int gg = g < HT ? g : HT - 1;
    const bool head_ok = g < HT && gg * 16 + x < H;
    float full, lshare;
    {
        float M = -INFINITY;
#pragma unroll 4
        for (int i = 0; i < NW; ++i) M = fmaxf(M, red_m[(i * 16 + x) * HT + gg]);
        float ssum = 0.f;
#pragma unroll 4
        for (int i = 0; i < NW; ++i)
            ssum = fmaf(red_s[(i * 16 + x) * HT + gg], fast_exp2(red_m[(i * 16 + x) * HT + gg] - M), ssum);
        const float clse = M + fast_log2(ssum);
        full = (has_nc && head_ok) ? logaddexp2(clse, nc * kLog2e) : clse;
        lshare = head_ok ? clse - full : -INFINITY;  // log2 of this head's share of the joint mass
    }
    const float lmax = cols4_max(row16_butterfly<true>(lshare));  // finite: some head is valid
    const float tot = cols4_sum(row16_sum(head_ok ? fast_exp2(lshare - lmax) : 0.f));
    // 2^(floor - lmax) overflows to +inf only when the true target underflows to 0 anyway
    const float rden = 1.f / fmaxf(tot, fast_exp2(floor_log2 - lmax));
    float fr[4];
    rows_bcast(full, fr);  // fr[ht]: full of head 16ht + x
    float wgt[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
        wgt[ht] = (ht * 16 + x < H && mloc[ht] != -INFINITY) ? fast_exp2((mloc[ht] - fr[ht]) - lmax) * rden : 0.f;
    // groups of four tiles: one 16-value transpose-reduction each
#pragma unroll
    for (int lg = 0; lg < KT; lg += 4) {
        float v[16];
#pragma unroll
        for (int l = 0; l < 4; ++l)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float sum = 0.f;
                if (lg + l < KT) {
#pragma unroll
                    for (int ht = 0; ht < HT; ++ht) sum = fmaf(acc[lg + l][ht][i], wgt[ht], sum);
                }
                v[4 * l + i] = sum;
            }
        tr_step<0x128, 16>(v, (x & 8) != 0);  // row_ror:8      partner x^8
        tr_step<0x141, 8>(v, (x & 4) != 0);   // row_half_mirror partner x^7
        tr_step<0x4e, 4>(v, (x & 2) != 0);    // quad_perm 2301 partner x^2
        tr_step<0xb1, 2>(v, (x & 1) != 0);    // quad_perm 1032 partner x^1
        const int l = lg + (x >> 2), pos = 16 * tm.of(l) + 4 * g + (x & 3);
        if (l < KT && l < my && pos < nv) Tr[cslot[pos]] = v[0];
    }
}

// Arguments of the target kernels (one struct in the kernel-argument segment).
struct TargetArgs {
    const void *q, *pool;
    const int32_t *idx;
    const float *nc_lse;  // natural-log window+sink LSE per (b,t,h), or NULL (legacy)
    // fused form only: the window part is computed in the kernel
    const void *kwin;
    const float *sink;    // [H] or NULL
    const int32_t *seg;   // [B,S] or NULL
    float *nc_out;        // [B,S,H] or NULL: the window+sink LSE as a by-product
    int W;
    int B, S, H, D, N, K;
    float scale_log2, floor_log2;  // log2 of the L1 floor
    float *target;
};

// Window tiles of token t (16 keys each, from max(0, t-W+1) to t; at most eight for W <= 128).
__device__ __forceinline__ int window_tiles(int W, int t) {
    const int kf = t - W + 1 > 0 ? t - W + 1 : 0;
    return (t - kf + 16) >> 4;
}

// Window part of the joint softmax for token t of batch b, inside the target kernel:
// the LSE over {scale <q_h, kwin_j> : j in [max(0, t-W+1), t], seg[j] == seg[t]} plus the
// sink, per head.  Window tiles of 16 consecutive keys starting at the first key are dealt
// KWT to a wave: wave w scores tiles KWT*w .. KWT*w + KWT-1 together in one pass of the same
// MFMA loop, so a pair reads the staged queries once (half the query reads of one tile per
// wave).
// window_local publishes each wave's masked per-head maximum and sum in red_wm/red_ws
// without waiting; after the epilogue's barrier window_combine reduces them over the waves
// and adds the sink, returning in natural log the value of head 16*min(g, HT-1) + x for
// lane (g, x) -- the layout the epilogue takes its nc values in.
template <int DT, int HT, int NW, int KWT>
__device__ __forceinline__ void window_local(const TargetArgs &a, const unsigned char *qb, int RS, int b, int t, int w,
                                             int lane, float *red_wm, float *red_ws) {
    constexpr int EB = Elem<DT>::bytes;
    const int S = a.S, D = a.D, nch = D >> 5;
    const int kf = t - a.W + 1 > 0 ? t - a.W + 1 : 0;
    const int nwt = window_tiles(a.W, t);
    const int myw = nwt - KWT * w >= KWT ? KWT : (nwt - KWT * w > 0 ? nwt - KWT * w : 0);  // tiles KWT*w + l
    const rsrc_t kr = make_rsrc(reinterpret_cast<const char *>(a.kwin) + (size_t)b * S * D * EB,
                                (uint32_t)((size_t)S * D * EB));
    f32x4 acc[KWT][HT];
#pragma unroll
    for (int l = 0; l < KWT; ++l) {
        const float init = l < myw ? 0.f : -INFINITY;
#pragma unroll
        for (int h = 0; h < HT; ++h) acc[l][h] = f32x4{init, init, init, init};
    }
    if (myw > 0) {
        uint32_t off[KWT];
#pragma unroll
        for (int l = 0; l < KWT; ++l) {
            int r = kf + 16 * (KWT * w + l) + (DT == 0 ? (int)quad_row_lane(lane) : (lane & 15));
            r = r < t ? r : t;  // rows past t are loaded as row t and masked below
            off[l] = DT == 0 ? (uint32_t)(r * D * EB) + quad_seg_bytes(lane)
                             : (uint32_t)((r * D + 8 * (lane >> 4)) * EB);
        }
        if constexpr (DT == 0) {
            score_dispatch<DT, HT, KWT>(myw, acc, qb, RS, kr, off, nch, 0, lane);
        } else {
            score_dispatch_f32<HT, KWT>(myw, acc, qb, RS, kr, off, nch, lane);
        }
    }
    // masked statistics (log2 domain); key j of element (l, i) = kf + 16(KWT w + l) + 4g + i
    const int x = lane & 15, g = lane >> 4;
    const int sg_t = a.seg ? a.seg[(size_t)b * S + t] : 0;
    bool okj[KWT][4];
#pragma unroll
    for (int l = 0; l < KWT; ++l)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = kf + 16 * (KWT * w + l) + 4 * g + i;
            okj[l][i] = l < myw && j <= t && (a.seg == nullptr || a.seg[(size_t)b * S + j] == sg_t);
        }
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        // masked keys become -inf (whatever they hold), so the maximum and the exponentials
        // need no further masks; the maximum is taken before scaling (scale > 0)
#pragma unroll
        for (int l = 0; l < KWT; ++l)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[l][ht][i] = okj[l][i] ? acc[l][ht][i] : -INFINITY;
        float mx = -INFINITY;
#pragma unroll
        for (int l = 0; l < KWT; ++l)
            mx = fmaxf(mx, fmaxf(fmaxf(acc[l][ht][0], acc[l][ht][1]), fmaxf(acc[l][ht][2], acc[l][ht][3])));
        mx = cols4_max(mx) * a.scale_log2;  // -inf when this wave holds no valid key
        const float nm = mx == -INFINITY ? 0.f : -mx;
        float sum = 0.f;
#pragma unroll
        for (int l = 0; l < KWT; ++l)
#pragma unroll
            for (int i = 0; i < 4; ++i) sum += fast_exp2(fmaf(acc[l][ht][i], a.scale_log2, nm));
        sum = cols4_sum(sum);
        if (lane < 16) {
            red_wm[(w * 16 + x) * HT + ht] = mx;
            red_ws[(w * 16 + x) * HT + ht] = sum;
        }
    }
}

template <int HT, int NW>
__device__ __forceinline__ float window_combine(const TargetArgs &a, int lane, const float *red_wm,
                                                const float *red_ws) {
    const int x = lane & 15, g = lane >> 4;
    const int gg = g < HT ? g : HT - 1;
    float M = -INFINITY;
#pragma unroll 4
    for (int i = 0; i < NW; ++i) M = fmaxf(M, red_wm[(i * 16 + x) * HT + gg]);
    float ssum = 0.f;  // key t is always in its own window, so M is finite
#pragma unroll 4
    for (int i = 0; i < NW; ++i) {
        const float mi = red_wm[(i * 16 + x) * HT + gg];
        ssum += mi == -INFINITY ? 0.f : red_ws[(i * 16 + x) * HT + gg] * fast_exp2(mi - M);
    }
    float nc2 = M + fast_log2(ssum);
    const int h = gg * 16 + x;
    if (a.sink != nullptr && h < a.H) nc2 = logaddexp2(nc2, a.sink[h] * kLog2e);
    return nc2 * kLn2;
}

// One workgroup per token (latest tokens first, they hold the most valid slots).  FUSED:
// the window part of the joint softmax is computed here too (window_local) instead of being
// read from nc_lse, so the queries are read from HBM once for the whole target.
// Waves per SIMD the register budget is set for: 4 (128 registers) for up to 16 accumulator
// tiles per wave, 2 (256 registers) for the 32-tile set of eight slot tiles x four head tiles.
template <int DT, int HT, int KT>
constexpr int waves_per_eu() {
    return DT == 0 && KT * HT <= 16 ? 4 : 2;
}

template <int DT, int HT, int KT, int NW, bool FUSED>
__global__ __launch_bounds__(NW * 64, (waves_per_eu<DT, HT, KT>())) void distill_target_kernel(const TargetArgs a) {
    constexpr int EB = Elem<DT>::bytes;
    constexpr int KP = 2;                      // slot passes of NW*64 (K <= 2*NW*64)
    // window tiles per wave (W <= 128): pairs on waves 0-3 with 8 waves (one read of the staged
    // queries per pair), single tiles on waves 0-7 with 16 (one workgroup per CU: balance wins)
    constexpr int KWT = NW >= 16 ? 1 : 2;
    static_assert(!FUSED || NW * KWT >= 8, "the eight window tiles need NW * KWT >= 8");
    extern __shared__ __align__(16) unsigned char smem[];
    const int S = a.S, H = a.H, D = a.D, N = a.N, K = a.K;
    const int nch = D >> 5;
    const int RS = qrow_stride(D, EB);
    unsigned char *qb = smem;                                                  // the token's queries
    int32_t *crow = reinterpret_cast<int32_t *>(smem + q_bytes<HT>(DT, D));   // [K] pool row per compacted slot
    int32_t *cslot = crow + K;                                                // [K] slot index per compacted slot
    float *red_m = reinterpret_cast<float *>(cslot + K);                      // [NW][16][HT] per-wave head max
    float *red_s = red_m + NW * 16 * HT;                                      // [NW][16][HT] per-wave head sum
    int *wcnt = reinterpret_cast<int *>(red_s + NW * 16 * HT);                // [KP][NW] valid-slot counts
    float *red_wm = reinterpret_cast<float *>(wcnt + KP * NW);                // FUSED: [NW][16][HT] window max
    float *red_ws = red_wm + NW * 16 * HT;                                    // FUSED: [NW][16][HT] window sum

    const int64_t bt = (int64_t)gridDim.x - 1 - blockIdx.x;
    const int b = (int)(bt / S);
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    int lane = tid & 63;
    float *Tr = a.target + bt * K;

    // 0./1. Query staging (asynchronous) overlaps the slot compaction.
    stage_queries<DT, HT, NW>(a.q, bt, H, D, qb, w, lane);
    const int nv = compact_slots<NW, KP>(a.idx + bt * K, K, N, Tr, crow, cslot, wcnt, tid, w, lane);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's query loads have landed in LDS
    __syncthreads();                // ... and everyone else's; the compacted list is complete

    // nc value (natural log) of head 16*min(g, HT-1) + x for lane (g, x).  FUSED: the
    // window statistics are published now and combined after the epilogue's barrier.
    float nc = 0.f;
    auto window_done = [&]() {
        nc = window_combine<HT, NW>(a, lane, red_wm, red_ws);
        const int g = lane >> 4, h = 16 * g + (lane & 15);
        if (a.nc_out != nullptr && g < HT && h < H) a.nc_out[bt * H + h] = nc;
    };
    if constexpr (FUSED) {
        window_local<DT, HT, NW, KWT>(a, qb, RS, b, (int)(bt - (int64_t)b * S), w, lane, red_wm, red_ws);
    } else {
        const int h = 16 * ((lane >> 4) < HT ? (lane >> 4) : HT - 1) + (lane & 15);
        if (a.nc_lse != nullptr && h < H) nc = a.nc_lse[bt * H + h];
    }
    if (nv == 0) {                  // empty row: the target is already all zeros
        if constexpr (FUSED) {
            __syncthreads();
            window_done();
        }
        return;
    }

    // 2. Scores of this wave's slot tiles (TileMap) of the compacted list.
    const int ntiles = (nv + 15) >> 4;
    int my;
    const TileMap tm = FUSED ? slot_tiles<KT, NW>(ntiles, w, my) : slot_tiles_rr<NW>(ntiles, w, my);
    const rsrc_t pr = make_rsrc(reinterpret_cast<const char *>(a.pool) + (size_t)b * N * D * EB,
                                (uint32_t)((size_t)N * D * EB));
    // Tiles this wave does not compute stay at -inf: they drop out of the maximum and
    // their exponentials are exactly 0, so the epilogue needs no per-element masks.
    f32x4 acc[KT][HT];
#pragma unroll
    for (int l = 0; l < KT; ++l) {
        const float init = l < my ? 0.f : -INFINITY;
#pragma unroll
        for (int h = 0; h < HT; ++h) acc[l][h] = f32x4{init, init, init, init};
    }
    if constexpr (DT == 0) {
        // bf16: 128-byte row pieces, lanes 8 to a row (see pair_frags)
        uint32_t olo[KT], ohi[KT];
#pragma unroll
        for (int l = 0; l < KT; ++l) {
            const int pos = 16 * tm.of(l) + pair_row_lane(lane);
            const int r0 = (l < my && pos < nv) ? crow[pos] : crow[0];
            const int r1 = (l < my && pos + 8 < nv) ? crow[pos + 8] : crow[0];
            // 24-bit multiplies (rows < 2^24): 32-bit results, no 64-bit register pairs
            olo[l] = __umul24((uint32_t)r0, (uint32_t)(D * EB)) + pair_seg_bytes(lane);
            ohi[l] = __umul24((uint32_t)r1, (uint32_t)(D * EB)) + pair_seg_bytes_hi(lane);
        }
        // tiles per pass: 2 with 128 registers (16 accumulator tiles), 4 with 256 (32 tiles);
        // one piece in flight (a second one does not fit either register budget)
        constexpr int PT = KT * HT >= 32 ? 4 : (KT * HT >= 16 ? 2 : KT);
        constexpr int DEPTH = 1;
        const int np = (nch + 1) >> 1;
        const int cr = (5 * w + (int)(bt % np)) % np;
        if (my > 0) {
            if (nch & 1)
                score_dispatch_pairs<HT, KT, PT, false, DEPTH>(my, acc, qb, pr, olo, ohi, nch, cr, lane);
            else
                score_dispatch_pairs<HT, KT, PT, true, DEPTH>(my, acc, qb, pr, olo, ohi, nch, cr, lane);
        }
    } else {
        // fp32: lane l on row l%16 (fragment layout)
        uint32_t off[KT];
#pragma unroll
        for (int l = 0; l < KT; ++l) {
            const int pos = 16 * tm.of(l) + (lane & 15);
            const int r = (l < my && pos < nv) ? crow[pos] : crow[0];
            off[l] = (uint32_t)((r * D + 8 * (lane >> 4)) * EB);
        }
        if (my > 0) score_dispatch_f32<HT, KT>(my, acc, qb, RS, pr, off, nch, lane);
    }

    // 3.-6. Epilogue: per-head statistics, joint denominators, head sums, normalised scatter.
    // (lane re-derived from an opaque copy: the epilogue's per-lane addresses are then
    // computed here instead of being hoisted above the score loop, where they would
    // compete with its registers)
    {
        int t = threadIdx.x;
        asm volatile("" : "+v"(t));
        lane = t & 63;
    }
    float mloc[HT];
    epi_stats<HT, KT, NW>(acc, mloc, my, nv, tm, w, lane, a.scale_log2, red_m, red_s);
    __syncthreads();
    if constexpr (FUSED) window_done();
    epi_target<HT, KT, NW>(acc, mloc, my, nv, tm, lane, H, FUSED || a.nc_lse != nullptr, nc, a.floor_log2, red_m,
                           red_s, cslot, Tr);
}

template <int DT, int HT, int KT, int NW, bool FUSED>
hipError_t launch3(const TargetArgs &a, hipStream_t stream) {
    const size_t red = (size_t)NW * 16 * HT * 4;
    const size_t qbytes = DT == 0 ? (size_t)2048 * HT * (((a.D >> 5) + 1) >> 1) : (size_t)16 * HT * (a.D * 4 + 16);
    const size_t lds = qbytes + (size_t)8 * a.K + 2 * red + (size_t)2 * NW * 4 + (FUSED ? 2 * red : 0);
    if (lds > (size_t)kLdsBytes) return hipErrorInvalidValue;
    auto kfn = &distill_target_kernel<DT, HT, KT, NW, FUSED>;
    if (lds > 65536) {  // more than the default 64 KiB of LDS per workgroup
        const hipError_t e = allow_full_lds<&distill_target_kernel<DT, HT, KT, NW, FUSED>>();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kfn, dim3((unsigned)((int64_t)a.B * a.S)), dim3(NW * 64), lds, stream, a);
    return hipGetLastError();
}

template <int DT, int HT, bool FUSED>
hipError_t launch2(const TargetArgs &a, hipStream_t stream) {
    const int K = a.K;
    // K <= 16*NW*KT.  The fused form keeps NW >= 4 so each wave holds at most two of the
    // (up to eight) window tiles.
    if constexpr (!FUSED) {
        if (K <= 16) return launch3<DT, HT, 1, 1, FUSED>(a, stream);
    }
    if (K <= 64) return launch3<DT, HT, 1, 4, FUSED>(a, stream);
    if (K <= 128) return launch3<DT, HT, 2, 4, FUSED>(a, stream);
    if (K <= 256) return launch3<DT, HT, 4, 4, FUSED>(a, stream);
    if (K <= 512) return launch3<DT, HT, 4, 8, FUSED>(a, stream);
    return launch3<DT, HT, 4, 16, FUSED>(a, stream);
}

template <int DT, bool FUSED>
hipError_t launch1(const TargetArgs &a, hipStream_t stream) {
    if (a.H <= 16) return launch2<DT, 1, FUSED>(a, stream);
    if (a.H <= 32) return launch2<DT, 2, FUSED>(a, stream);
    return launch2<DT, 4, FUSED>(a, stream);
}

template <bool FUSED>
hipError_t launch0(TargetArgs a, float scale, float l1_floor, int dtype, hipStream_t stream) {
    a.scale_log2 = scale * kLog2e;
    a.floor_log2 = l1_floor > 0.f ? (float)log2((double)l1_floor) : -126.f;  // FLT_MIN = 2^-126
    if (dtype == 0) return launch1<0, FUSED>(a, stream);
    return launch1<1, FUSED>(a, stream);
}

}  // namespace

hipError_t launch_distill_target(const void *q, const void *pool, const int32_t *idx, const float *nc_lse,
                                 int B, int S, int H, int D, int N, int K, float scale, float l1_floor,
                                 int dtype, float *target, hipStream_t stream) {
    TargetArgs a{};
    a.q = q; a.pool = pool; a.idx = idx; a.nc_lse = nc_lse;
    a.B = B; a.S = S; a.H = H; a.D = D; a.N = N; a.K = K;
    a.target = target;
    return launch0<false>(a, scale, l1_floor, dtype, stream);
}

hipError_t launch_distill_target_fused(const void *q, const void *kwin, const float *sink, const int32_t *seg,
                                       const void *pool, const int32_t *idx, int B, int S, int H, int D, int N,
                                       int K, int W, float scale, float l1_floor, int dtype, float *target,
                                       float *nc_out, hipStream_t stream) {
    TargetArgs a{};
    a.q = q; a.pool = pool; a.idx = idx;
    a.kwin = kwin; a.sink = sink; a.seg = seg; a.nc_out = nc_out; a.W = W;
    a.B = B; a.S = S; a.H = H; a.D = D; a.N = N; a.K = K;
    a.target = target;
    return launch0<true>(a, scale, l1_floor, dtype, stream);
}

}  // namespace sd
