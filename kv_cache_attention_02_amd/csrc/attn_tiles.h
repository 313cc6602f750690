// Key-tile planning shared by the attention kernels: per-row allowed key
// intervals of the three mask modes, and the union of a block of rows' ranges
// in 64-key tiles.  Compiled for the device, where the kernels call it, and for
// the host, where the dry-run planner logs every q-tile's ranges for checking.
#pragma once

#include "wmk_internal.h"

namespace wmk {
namespace tiles {

constexpr int BK = 64;  // keys per tile

// The tile ranges a workgroup visits: union over its rows of their allowed key
// ranges, rounded out to whole tiles, sorted and merged (at most 4 ranges).
// Written with fixed slots, a sorting network and selects -- no dynamically
// indexed arrays -- so that it stays in scalar registers (an array would live
// in scratch memory, whose reads wait for the in-flight tile loads).
struct TileRanges {
    int32_t b0, e0, b1, e1, b2, e2, b3, e3;
    int32_t total;
};

constexpr int32_t kNone = 0x7fffffff;  // empty slot

// Key (or row) indices here are never negative: divide them as unsigned.
__host__ __device__ __forceinline__ int32_t udiv(int32_t n, FastDiv d) { return (int32_t)fastdiv((uint32_t)n, d); }

__host__ __device__ __forceinline__ void set_tiles(int32_t& l, int32_t& h, int32_t a, int32_t b) {
    if (b > a) { l = (int32_t)((uint32_t)a / BK); h = (int32_t)(((uint32_t)b + BK - 1) / BK); }
}

__host__ __device__ __forceinline__ void order(int32_t& al, int32_t& ah, int32_t& bl, int32_t& bh) {
    const bool sw = bl < al;
    const int32_t tl = sw ? bl : al, th = sw ? bh : ah;
    bl = sw ? al : bl;
    bh = sw ? ah : bh;
    al = tl;
    ah = th;
}

__host__ __device__ __forceinline__ void emit(TileRanges& r, int k, int32_t b, int32_t e) {
    r.b0 = k == 0 ? b : r.b0; r.e0 = k == 0 ? e : r.e0;
    r.b1 = k == 1 ? b : r.b1; r.e1 = k == 1 ? e : r.e1;
    r.b2 = k == 2 ? b : r.b2; r.e2 = k == 2 ? e : r.e2;
    r.b3 = k == 3 ? b : r.b3; r.e3 = k == 3 ? e : r.e3;
}

// Sort up to four tile ranges (kNone = empty slot) and merge overlapping or
// touching ones.
__host__ __device__ __forceinline__ TileRanges merge_ranges(int32_t l0, int32_t h0, int32_t l1, int32_t h1, int32_t l2,
                                                   int32_t h2, int32_t l3, int32_t h3) {
    order(l0, h0, l1, h1);
    order(l2, h2, l3, h3);
    order(l0, h0, l2, h2);
    order(l1, h1, l3, h3);
    order(l1, h1, l2, h2);
    TileRanges r = {0, 0, 0, 0, 0, 0, 0, 0, 0};
    int k = 0;
    int32_t cb = l0, ce = h0;
#define WMK_MERGE(L_, H_)              \
    if (L_ != kNone) {                 \
        if (L_ <= ce) {                \
            ce = max(ce, H_);          \
        } else {                       \
            emit(r, k, cb, ce);        \
            ++k;                       \
            cb = L_;                   \
            ce = H_;                   \
        }                              \
    }
    WMK_MERGE(l1, h1)
    WMK_MERGE(l2, h2)
    WMK_MERGE(l3, h3)
#undef WMK_MERGE
    if (cb != kNone) emit(r, k, cb, ce);
    r.total = (r.e0 - r.b0) + (r.e1 - r.b1) + (r.e2 - r.b2) + (r.e3 - r.b3);
    return r;
}

template <class Call>
__host__ __device__ __forceinline__ TileRanges tile_ranges(const Call& c, int32_t r0, int32_t r1) {
    // The two masks with at most two ranges, the first starting at key 0, skip
    // the general sort and merge below (scalar work that every wave of the
    // workgroup repeats at each unit's start).
    if (c.mask.mode == kMaskNone) {  // every key: one range
        const int32_t t = (int32_t)(((uint32_t)c.kv_total + BK - 1) / BK);
        return TileRanges{0, t, 0, 0, 0, 0, 0, 0, t};
    }
    if (c.mask.mode == kMaskCross) {  // environment prompt + the local prompts of the tile's chunks
        const int32_t ca = udiv(r0, c.mask.part_div), cb = udiv(r1 - 1, c.mask.part_div);
        const int32_t a = c.mask.env_len + ca * c.mask.chunk_len, b = c.mask.env_len + (cb + 1) * c.mask.chunk_len;
        const int32_t e0 = (int32_t)(((uint32_t)c.mask.env_len + BK - 1) / BK);
        const int32_t b1 = (int32_t)((uint32_t)a / BK), e1 = (int32_t)(((uint32_t)b + BK - 1) / BK);
        if (b <= a) return TileRanges{0, e0, 0, 0, 0, 0, 0, 0, e0};                      // no local prompt
        if (e0 == 0) return TileRanges{b1, e1, 0, 0, 0, 0, 0, 0, e1 - b1};               // no environment prompt
        if (b1 <= e0) return TileRanges{0, e1, 0, 0, 0, 0, 0, 0, e1};                    // one merged range
        return TileRanges{0, e0, b1, e1, 0, 0, 0, 0, e0 + (e1 - b1)};                     // two ranges
    }
    int32_t l0 = kNone, h0 = kNone, l1 = kNone, h1 = kNone, l2 = kNone, h2 = kNone, l3 = kNone, h3 = kNone;
    {
        const int32_t L = c.mask.part_len, cl = c.mask.chunk_len;
        const FastDiv pd = c.mask.part_div, cd = c.mask.chunk_div;
        const int32_t pa = udiv(r0, pd), pb = min(udiv(r1 - 1, pd), c.mask.parts - 1);
        if (pa <= 0 && 0 <= pb) {  // clean rows: block-causal prefix
            const int32_t fb = min(r1, L) - 1;
            set_tiles(l0, h0, 0, min((udiv(fb, cd) + 1) * cl, L));
        }
        if (pa <= 1 && 1 <= pb) {  // noisy rows: earlier clean chunks, own noisy chunk
            const int32_t fa = max(r0, L) - L, fb = min(r1, 2 * L) - L - 1;
            const int32_t ka = udiv(fa, cd), kb = udiv(fb, cd);
            set_tiles(l1, h1, 0, kb * cl);
            set_tiles(l2, h2, L + ka * cl, L + min((kb + 1) * cl, L));
        }
        if (pa <= 2 && 2 <= pb) set_tiles(l3, h3, 2 * L, 3 * L);  // the bidirectional block
    }
    return merge_ranges(l0, h0, l1, h1, l2, h2, l3, h3);
}

__host__ __device__ __forceinline__ int32_t tile_at(const TileRanges& r, int32_t it) {
    const int32_t n0 = r.e0 - r.b0, n1 = n0 + (r.e1 - r.b1), n2 = n1 + (r.e2 - r.b2);
    return it < n0 ? r.b0 + it : it < n1 ? r.b1 + (it - n0) : it < n2 ? r.b2 + (it - n1) : r.b3 + (it - n2);
}

// End (exclusive, in tiles) of the tile range that visit `it` falls in.
__host__ __device__ __forceinline__ int32_t range_end_at(const TileRanges& r, int32_t it) {
    const int32_t n0 = r.e0 - r.b0, n1 = n0 + (r.e1 - r.b1), n2 = n1 + (r.e2 - r.b2);
    return it < n0 ? r.e0 : it < n1 ? r.e1 : it < n2 ? r.e2 : r.e3;
}

// Allowed key ranges of one query row (see wmk.h).
template <class Call>
__host__ __device__ __forceinline__ void row_ranges(const Call& c, int32_t row, int32_t& lo0, int32_t& hi0, int32_t& lo1,
                                           int32_t& hi1) {
    lo1 = 0; hi1 = 0;
    if (c.mask.mode == kMaskNone || row >= c.q_tokens) { lo0 = 0; hi0 = c.kv_total; return; }
    if (c.mask.mode == kMaskCross) {
        const int32_t ch = udiv(row, c.mask.part_div);
        lo0 = 0; hi0 = c.mask.env_len;
        lo1 = c.mask.env_len + ch * c.mask.chunk_len; hi1 = lo1 + c.mask.chunk_len;
        return;
    }
    const int32_t L = c.mask.part_len, cl = c.mask.chunk_len;
    const int32_t part = udiv(row, c.mask.part_div), r = row - part * L, k = udiv(r, c.mask.chunk_div);
    const int32_t e = min((k + 1) * cl, L);
    if (part == 0) { lo0 = 0; hi0 = e; }
    else if (part == 1) { lo0 = 0; hi0 = k * cl; lo1 = L + k * cl; hi1 = L + e; }
    else { lo0 = 2 * L; hi0 = 3 * L; }
}

// Column view of the MoBA mask, for the backward: the query rows that attend
// key j (at most two ranges).  Transpose of row_ranges: clean key of chunk c -> clean rows
// of chunks >= c and noisy rows of chunks > c; noisy key of chunk c -> noisy
// rows of chunk c; block key -> block rows.
__host__ __device__ __forceinline__ void col_ranges(const MaskShape& m, int32_t n, int32_t j, int32_t& lo0,
                                                    int32_t& hi0, int32_t& lo1, int32_t& hi1) {
    lo0 = hi0 = lo1 = hi1 = 0;
    if (j >= n) return;
    const int32_t L = m.part_len, cl = m.chunk_len;
    const int32_t part = udiv(j, m.part_div), c = udiv(j - part * L, m.chunk_div);
    if (part == 0) {
        lo0 = c * cl; hi0 = L;
        lo1 = min(L + (c + 1) * cl, 2 * L); hi1 = m.parts > 1 ? 2 * L : lo1;
    } else if (part == 1) {
        lo0 = L + c * cl; hi0 = L + min((c + 1) * cl, L);
    } else {
        lo0 = 2 * L; hi0 = 3 * L;
    }
}

// Union over keys [c0, c1) of their query ranges, in 64-row tiles (same form as
// tile_ranges for rows).
__host__ __device__ __forceinline__ TileRanges col_tile_ranges(const MaskShape& m, int32_t n, int32_t c0,
                                                               int32_t c1) {
    int32_t l0 = kNone, h0 = kNone, l1 = kNone, h1 = kNone, l2 = kNone, h2 = kNone, l3 = kNone, h3 = kNone;
    const int32_t L = m.part_len, cl = m.chunk_len;
    c1 = min(c1, n);
    if (c1 > c0) {
        const int32_t pa = udiv(c0, m.part_div), pb = udiv(c1 - 1, m.part_div);
        if (pa <= 0 && 0 <= pb) {  // clean keys: from the first key's chunk on, clean and (later) noisy rows
            const int32_t ca = udiv(c0, m.chunk_div);
            set_tiles(l0, h0, ca * cl, L);
            if (m.parts > 1) set_tiles(l1, h1, min(L + (ca + 1) * cl, 2 * L), 2 * L);
        }
        if (pa <= 1 && 1 <= pb) {  // noisy keys: the noisy rows of their chunks
            const int32_t fa = max(c0, L) - L, fb = min(c1, 2 * L) - L - 1;
            set_tiles(l2, h2, L + udiv(fa, m.chunk_div) * cl, L + min((udiv(fb, m.chunk_div) + 1) * cl, L));
        }
        if (pa <= 2 && 2 <= pb) set_tiles(l3, h3, 2 * L, 3 * L);
    }
    return merge_ranges(l0, h0, l1, h1, l2, h2, l3, h3);
}

// j in [lo, hi), without branches.  The masks are written branch-free on
// purpose: with short-circuit && / || per lane, this toolchain (ROCm 7.2
// clang) lowered the in-place select "s = ok ? s : -inf" into divergent
// blocks that overwrote s with -inf for lanes outside the first interval and
// never restored it for lanes inside the second one.
__host__ __device__ __forceinline__ uint32_t in_range(int32_t j, int32_t lo, int32_t hi) {
    return (uint32_t)(j - lo) < (uint32_t)(hi - lo) ? 1u : 0u;
}

}  // namespace tiles
}  // namespace wmk
