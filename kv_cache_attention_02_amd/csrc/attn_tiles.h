// Key-tile planning shared by the attention kernels: per-row allowed key
// intervals of the three mask modes, and the union of a block of rows' ranges
// in 64-key tiles.  Device code only.
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

__device__ __forceinline__ void set_tiles(int32_t& l, int32_t& h, int32_t a, int32_t b) {
    if (b > a) { l = a / BK; h = (b + BK - 1) / BK; }
}

__device__ __forceinline__ void order(int32_t& al, int32_t& ah, int32_t& bl, int32_t& bh) {
    const bool sw = bl < al;
    const int32_t tl = sw ? bl : al, th = sw ? bh : ah;
    bl = sw ? al : bl;
    bh = sw ? ah : bh;
    al = tl;
    ah = th;
}

__device__ __forceinline__ void emit(TileRanges& r, int k, int32_t b, int32_t e) {
    r.b0 = k == 0 ? b : r.b0; r.e0 = k == 0 ? e : r.e0;
    r.b1 = k == 1 ? b : r.b1; r.e1 = k == 1 ? e : r.e1;
    r.b2 = k == 2 ? b : r.b2; r.e2 = k == 2 ? e : r.e2;
    r.b3 = k == 3 ? b : r.b3; r.e3 = k == 3 ? e : r.e3;
}

// Sort up to four tile ranges (kNone = empty slot) and merge overlapping or
// touching ones.
__device__ __forceinline__ TileRanges merge_ranges(int32_t l0, int32_t h0, int32_t l1, int32_t h1, int32_t l2,
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
__device__ __forceinline__ TileRanges tile_ranges(const Call& c, int32_t r0, int32_t r1) {
    int32_t l0 = kNone, h0 = kNone, l1 = kNone, h1 = kNone, l2 = kNone, h2 = kNone, l3 = kNone, h3 = kNone;
    if (c.mask.mode == kMaskNone) {
        set_tiles(l0, h0, 0, c.kv_total);
    } else if (c.mask.mode == kMaskCross) {  // environment prompt + the local prompts of the tile's chunks
        const int32_t ca = r0 / c.mask.part_len, cb = (r1 - 1) / c.mask.part_len;
        set_tiles(l0, h0, 0, c.mask.env_len);
        set_tiles(l1, h1, c.mask.env_len + ca * c.mask.chunk_len, c.mask.env_len + (cb + 1) * c.mask.chunk_len);
    } else {
        const int32_t L = c.mask.part_len, cl = c.mask.chunk_len;
        const int32_t pa = r0 / L, pb = min((r1 - 1) / L, c.mask.parts - 1);
        if (pa <= 0 && 0 <= pb) {  // clean rows: block-causal prefix
            const int32_t fb = min(r1, L) - 1;
            set_tiles(l0, h0, 0, min((fb / cl + 1) * cl, L));
        }
        if (pa <= 1 && 1 <= pb) {  // noisy rows: earlier clean chunks, own noisy chunk
            const int32_t fa = max(r0, L) - L, fb = min(r1, 2 * L) - L - 1;
            const int32_t ka = fa / cl, kb = fb / cl;
            set_tiles(l1, h1, 0, kb * cl);
            set_tiles(l2, h2, L + ka * cl, L + min((kb + 1) * cl, L));
        }
        if (pa <= 2 && 2 <= pb) set_tiles(l3, h3, 2 * L, 3 * L);  // the bidirectional block
    }
    return merge_ranges(l0, h0, l1, h1, l2, h2, l3, h3);
}

__device__ __forceinline__ int32_t tile_at(const TileRanges& r, int32_t it) {
    const int32_t n0 = r.e0 - r.b0, n1 = n0 + (r.e1 - r.b1), n2 = n1 + (r.e2 - r.b2);
    return it < n0 ? r.b0 + it : it < n1 ? r.b1 + (it - n0) : it < n2 ? r.b2 + (it - n1) : r.b3 + (it - n2);
}

// End (exclusive, in tiles) of the tile range that visit `it` falls in.
__device__ __forceinline__ int32_t range_end_at(const TileRanges& r, int32_t it) {
    const int32_t n0 = r.e0 - r.b0, n1 = n0 + (r.e1 - r.b1), n2 = n1 + (r.e2 - r.b2);
    return it < n0 ? r.e0 : it < n1 ? r.e1 : it < n2 ? r.e2 : r.e3;
}

// Allowed key ranges of one query row (see wmk.h).
template <class Call>
__device__ __forceinline__ void row_ranges(const Call& c, int32_t row, int32_t& lo0, int32_t& hi0, int32_t& lo1,
                                           int32_t& hi1) {
    lo1 = 0; hi1 = 0;
    if (c.mask.mode == kMaskNone || row >= c.q_tokens) { lo0 = 0; hi0 = c.kv_total; return; }
    if (c.mask.mode == kMaskCross) {
        const int32_t ch = row / c.mask.part_len;
        lo0 = 0; hi0 = c.mask.env_len;
        lo1 = c.mask.env_len + ch * c.mask.chunk_len; hi1 = lo1 + c.mask.chunk_len;
        return;
    }
    const int32_t L = c.mask.part_len, cl = c.mask.chunk_len;
    const int32_t part = row / L, r = row - part * L, k = r / cl;
    const int32_t e = min((k + 1) * cl, L);
    if (part == 0) { lo0 = 0; hi0 = e; }
    else if (part == 1) { lo0 = 0; hi0 = k * cl; lo1 = L + k * cl; hi1 = L + e; }
    else { lo0 = 2 * L; hi0 = 3 * L; }
}

// j in [lo, hi), without branches.  The masks are written branch-free on
// purpose: with short-circuit && / || per lane, this toolchain (ROCm 7.2
// clang) lowered the in-place select "s = ok ? s : -inf" into divergent
// blocks that overwrote s with -inf for lanes outside the first interval and
// never restored it for lanes inside the second one.
__device__ __forceinline__ uint32_t in_range(int32_t j, int32_t lo, int32_t hi) {
    return (uint32_t)(j - lo) < (uint32_t)(hi - lo) ? 1u : 0u;
}

}  // namespace tiles
}  // namespace wmk
