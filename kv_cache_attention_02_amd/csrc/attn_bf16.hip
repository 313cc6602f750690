// bf16 attention on the CDNA4 matrix cores (gfx950).
//
// One workgroup = 8 waves = 256 query rows of one head (32 rows per wave); keys
// are visited in tiles of 64.  K and V tiles go from global memory straight
// into LDS (16-byte buffer loads with the LDS-destination form, no staging
// registers) and are shared by the waves; two K and two V buffers, one
// barrier per tile.  Calls whose units walk few key tiles run the same code
// with 4 waves (128 rows) per workgroup and two workgroups per CU, so that one
// workgroup's unit fill overlaps the other's steps.
//
// Per wave, iteration j (software pipelined across tiles):
//   softmax of tile j            fp32, log2 domain: exp2 with scale*log2(e)
//                                folded into one FMA; the reference max moves
//                                (and O, l are rescaled) only when a row max
//                                grows by more than kTau.
//   S^T(j+1) = K(j+1) . Q^T      v_mfma_f32_32x32x16_bf16; K from LDS (A), Q^T
//                                from registers (B, loaded once).  Independent of
//                                the softmax above, so the matrix core runs it
//                                while the VALU does the exponentials.  In the
//                                32x32 accumulator layout lane l owns query l%32
//                                and 16 of each 32-key block; the other 16 sit in
//                                lane l^32 (one permlane32 swap per reduction).
//   O^T += V(j)^T . P(j)^T       P^T is the S^T accumulator rounded to bf16, used
//                                as the B operand as it stands; V^T comes from
//                                the row-major V tile through ds_read_b64_tr_b16
//                                (transposing LDS reads), addressed so that its
//                                key order equals the accumulator's.
//
// LDS tiles are unpadded [key][dim] rows with 16-byte chunks XOR-swizzled per
// row (different swizzles for K and V) so that both read patterns are free of
// bank conflicts.
//
// Masks come from key intervals: every row allows at most two half-open key
// ranges (the whole key range at a chunk step; the MoBA ranges in training).
// A tile that every row of a wave fully allows runs unmasked; any other
// visited tile applies the per-element interval test.  Tiles that no row of
// the workgroup allows are never visited: the workgroup walks only the union of
// its rows' ranges, in tile units.
//
// Split tail: when there are too few units (query tiles of one head)
// to fill the chip, the last units are cut into pieces along their key tiles.
// Each piece writes its unnormalized O and per-row (max, sum) to a workspace;
// attn_merge_kernel, launched after it on the same stream, combines the pieces
// of a unit.  No piece waits on another.
//
// FP8 variant (Q8): Q and K arrive pre-quantized to e4m3 with one fp32 scale per
// block (32 query rows of a wave; one 64-key tile), the K tile already in the
// LDS layout below; S^T = K Q^T runs as v_mfma_scale_f32_32x32x64_f8f6f4 (two
// k-steps of 64 dims instead of eight of 16) and the block scales fold into the
// per-tile exponent multiplier.  Softmax, P and P V are as in the bf16 path.
//
// Sources: chunk attention over [anchors | recent | current] ("Westlake AGI
// Lab's 'World in World' Steers Frozen Video Models", second paragraph); the
// MoBA mask ("Infinite Worlds with Versatile Interactions", causal pretraining
// paragraph; "Mix Forcing: Causal Pre-Training via Mixture Attention for
// Interactive World Models", "Mix the training modes").
#include <math.h>

#include <type_traits>
#include <utility>

#include "attn_tiles.h"
#include "wmk_internal.h"

namespace wmk {

#ifdef WMK_STEP_PROFILE
// Step profile (a separate build, libwmk_stepprof.so): per wave, the shader
// cycles (s_memtime) spent in each phase of the key-tile steps, summed over the
// launch -- [A], [B], the wait for the step's own direct loads, the barrier and
// the issue code before [A] -- plus the step count, the span from the first
// step's start to the last step's end, the unit, that span on the 100 MHz
// real-time counter (s_memrealtime), which gives the shader clock, and the
// cycles from the kernel's entry to the first step (the unit's fill: Q
// fragments, the first tiles, the first scores) and its parts.  Read back with
// wmk_step_profile_read after the launch.  Each timestamp is a scalar memory
// read the following code waits on, so the profiled kernel runs a few percent
// slower than the product build.
__device__ unsigned long long g_step_prof[4096 * 8][16];
extern "C" __attribute__((visibility("default"))) int wmk_step_profile_read(void* host, size_t bytes) {
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_step_prof), bytes, 0, hipMemcpyDeviceToHost);
}
#define WMK_STAMP(x) x = __builtin_amdgcn_s_memtime()
#else
#define WMK_STAMP(x) (void)0
#endif

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int BK = tiles::BK; // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;  // lazy-rescale threshold, log2 units (weights stay <= 256)

// D: head dim; NW: waves per workgroup (8: one workgroup per CU; 4: two per CU,
// for calls of short units, where one workgroup's fill runs beside the other's steps)
template <int D, int NW>
struct Cfg {
    static constexpr int NT = NW * 64;                  // threads per workgroup
    static constexpr int BQ = NW * 32;                  // query rows per workgroup
    static constexpr int CPR = D / 8;                   // 16-byte chunks per key row
    static constexpr int ROWB = D * 2;                  // bytes per key row
    static constexpr int TILEB = BK * ROWB;             // bytes per K (or V) tile
    static constexpr int LPT = TILEB / (NT * 16);       // direct loads per thread per tile
    static constexpr int ROWS_PER_KB = 1024 / ROWB;     // key rows per 1 KB wave load
    static constexpr int DS = D / 16;                   // k-steps of S = K Q^T
    static constexpr int DB = D / 32;                   // 32-row blocks of O^T
    static constexpr int PARTS = LPT >= 2 ? 2 : 1;      // LDS objects per K (or V) buffer
    static constexpr int LPP = LPT / PARTS;             // direct loads per thread into each object
    static constexpr int PART_ROWS = BK / PARTS;        // key rows per LDS object
    static constexpr int PARTB = PART_ROWS * ROWB;      // bytes per LDS object
    static_assert(LPT >= 1 && LPT * NT * 16 == TILEB, "tile must split into whole wave loads");
    static_assert(LPP * PARTS == LPT && PART_ROWS % 32 == 0, "a 32-key block must lie inside one LDS object");
    static_assert(DS >= 2 * LPT, "the K and V loads of a tile are spread over the k-steps of [A]");
};

// 16-byte chunk swizzles (XOR with a per-row constant, so a bijection inside
// each row).  K: 32 rows are read at once at one logical chunk -> the swizzle
// spreads rows over all chunk positions; it depends on row % 16 only.  V: a
// transposing read touches 8 consecutive rows x 64 bytes -> rows r and r+1..3
// go to different 64-byte bank groups; it depends on row % 8 only.  Because of
// that, the per-lane part of every LDS address is fixed and all the rest
// (k-step, key block, buffer) is a compile-time offset.
template <int D, int NW>
__device__ __forceinline__ int swz_k(int row) { return row & 15 & (Cfg<D, NW>::CPR - 1); }
template <int D, int NW>
__device__ __forceinline__ int swz_v(int row) { return (((row & 3) << 2) | ((row >> 2) & 1)) & (Cfg<D, NW>::CPR - 1); }

template <int NS>
struct Params {
    AttnCallN<NS> c;
    AttnPlan p;
};

using tiles::TileRanges;
using tiles::kNone;
using tiles::set_tiles;
using tiles::tile_ranges;
using tiles::tile_at;
using tiles::range_end_at;
using tiles::row_ranges;
using tiles::in_range;

// Span holding key j: base pointers, first and past-the-end key.  Written with
// static indices and selects so that, for a uniform j, it stays in scalar
// registers (dynamic indexing would reload the kernel arguments from memory).
struct SpanSel {
    const char* k;
    const char* v;
    int32_t start, end;
};

template <int N>
__device__ __forceinline__ SpanSel span_sel(const KvSpansN<N>& kv, int32_t j) {
    SpanSel r{(const char*)kv.k[0], (const char*)kv.v[0], 0, kv.end[0]};
#pragma unroll
    for (int x = 0; x < N - 1; ++x) {
        const bool past = (x < kv.n - 1) && (j >= kv.end[x]);
        r.k = past ? (const char*)kv.k[x + 1] : r.k;
        r.v = past ? (const char*)kv.v[x + 1] : r.v;
        r.start = past ? kv.end[x] : r.start;
        r.end = past ? kv.end[x + 1] : r.end;
    }
    return r;
}

// Where the direct loads of one visited key tile come from.  `run` > 0: this
// tile and the next run - 1 visited tiles lie in one tile range and wholly
// inside one span, so each is one uniform base (k, v: the tile's first key row
// of this head) plus per-lane offsets, and the next one is 64 rows further.
// run <= 0: the tile crosses a span end or the last key (per-row lookup).
// Advancing is a few scalar adds except where a run ends.
struct Cursor {
    int32_t tile;
    int32_t run;
    const char* k;
    const char* v;
};

template <class Call>
__device__ __forceinline__ Cursor cursor_at(const Call& c, const TileRanges& tr, int32_t it, int64_t row_bytes,
                                            int64_t head_off) {
    Cursor cu;
    cu.tile = tile_at(tr, it);
    const int32_t j0 = cu.tile * BK;
    const SpanSel sp = span_sel(c.kv, j0);
    cu.run = min(range_end_at(tr, it) - cu.tile, (sp.end - j0) / BK);
    const int64_t base = (int64_t)(j0 - sp.start) * row_bytes + head_off;
    cu.k = sp.k + base;
    cu.v = sp.v + base;
    return cu;
}

template <class Call>
__device__ __forceinline__ void advance(Cursor& cu, const Call& c, const TileRanges& tr, int32_t it_next,
                                        int64_t row_bytes, int64_t head_off) {
    if (cu.run > 1) {
        cu.tile += 1;
        cu.run -= 1;
        cu.k += BK * row_bytes;
        cu.v += BK * row_bytes;
    } else {
        cu = cursor_at(c, tr, it_next, row_bytes, head_off);
    }
}

// This thread's share of the direct tile loads: for each of its LPT wave loads
// of a K (or V) tile, the key row inside the tile it fills and the byte offset
// (from the tile's first key row of this head) of the swizzle-mapped source
// chunk for K and for V.
template <int D, int NW>
struct LoadMap {
    int32_t row[Cfg<D, NW>::LPT];
    uint32_t kg[Cfg<D, NW>::LPT];
    uint32_t vg[Cfg<D, NW>::LPT];
};

template <int D, int NW>
__device__ __forceinline__ LoadMap<D, NW> load_map(int wave, uint32_t row_bytes) {
    using C = Cfg<D, NW>;
    const int lane = threadIdx.x & 63;
    LoadMap<D, NW> m;
#pragma unroll
    for (int i = 0; i < C::LPT; ++i) {
        // load i of every wave fills 1 KB block (i % LPP) * NW + wave of LDS object i / LPP
        const int row = (i / C::LPP) * C::PART_ROWS + ((i % C::LPP) * NW + wave) * C::ROWS_PER_KB +
                        lane / C::CPR;  // key row in the tile
        const int phys = lane % C::CPR;                                           // chunk position it lands in
        m.row[i] = row;
        m.kg[i] = (uint32_t)row * row_bytes + (uint32_t)((phys ^ swz_k<D, NW>(row)) * 16);
        m.vg[i] = (uint32_t)row * row_bytes + (uint32_t)((phys ^ swz_v<D, NW>(row)) * 16);
    }
    return m;
}

// The LDS objects of one K or V buffer: part i holds key rows
// [i * PART_ROWS, (i + 1) * PART_ROWS), each unpadded [row][dim].
template <int D, int NW>
struct Buf {
    char LDS_AS* part[Cfg<D, NW>::PARTS];
    // LDS block that direct load i of `wave` fills
    __device__ __forceinline__ char LDS_AS* load_dst(int i, int wave) const {
        return part[i / Cfg<D, NW>::LPP] + ((i % Cfg<D, NW>::LPP) * NW + wave) * 1024;
    }
    // row kb * 32 + r (0 <= r < 32) of the tile: the object is known at compile
    // time from kb, so the compiler can keep the objects apart
    template <int KB>
    __device__ __forceinline__ char LDS_AS* block_row(int r) const {
        constexpr int P = (KB * 32) / Cfg<D, NW>::PART_ROWS, R0 = (KB * 32) % Cfg<D, NW>::PART_ROWS;
        return part[P] + (R0 + r) * Cfg<D, NW>::ROWB;
    }
};

// Buffer resource over `bytes` bytes from `base` (raw: byte offsets, no
// stride); lanes whose offset falls outside read zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Direct load of 16 bytes per lane at byte offset `off` of buffer `r` into the
// 1 KB block of this wave in LDS object `dst`.  Buffer (not global) loads: the
// compiler counts these only on the vector-memory counter, so waits for LDS
// reads that follow need not drain them.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t off, char LDS_AS* dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void LDS_AS*)dst, 16, off, 0, 0, 0);
}

// Issue the direct loads of the key tile at cursor `cu` into LDS (kbuf and/or
// vbuf).  Common case: the tile lies inside one span, so one buffer resource
// starting at its first row and per-lane constant offsets.  A tile crossing a
// span end (or the last key) loads each span's rows under a lane mask; rows
// past the last key read the last key instead (finite data that the mask
// drops).
template <int D, int NW, class Call>
__device__ __forceinline__ void issue_tile(const Call& c, int32_t head, const Cursor& cu, const LoadMap<D, NW>& m,
                                           int wave, const Buf<D, NW>& kbuf, const Buf<D, NW>& vbuf, bool do_k, bool do_v) {
    using C = Cfg<D, NW>;
    const int64_t row_bytes = (int64_t)c.heads * D * 2;
    const uint32_t tile_bytes = (uint32_t)(BK * row_bytes);  // < 2^31: checked on the host
    if (cu.run > 0) {
        const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(cu.k, tile_bytes);
        const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(cu.v, tile_bytes);
#pragma unroll
        for (int i = 0; i < C::LPT; ++i) {
            if (do_k) dma16(rk, m.kg[i], kbuf.load_dst(i, wave));
            if (do_v) dma16(rv, m.vg[i], vbuf.load_dst(i, wave));
        }
        return;
    }
    // per span touched by the tile: a resource from the span's first row in
    // the tile, and a lane mask for the rows in that span
    const int64_t head_off = (int64_t)head * D * 2;
    const int32_t j0 = cu.tile * BK, j1 = min(j0 + BK, c.kv_total);
#pragma nounroll
    for (int x = 0; x < c.kv.n; ++x) {
        const int32_t sb = x == 0 ? 0 : c.kv.end[x - 1], se = c.kv.end[x];
        if (se <= j0 || sb >= j1) continue;  // tile does not touch span x
        const int32_t r0 = max(j0, sb);      // first key of the span in this tile
        const int64_t base = (int64_t)(r0 - sb) * row_bytes + head_off;
        const __amdgpu_buffer_rsrc_t rk = buffer_rsrc((const char*)c.kv.k[x] + base, tile_bytes);
        const __amdgpu_buffer_rsrc_t rv = buffer_rsrc((const char*)c.kv.v[x] + base, tile_bytes);
#pragma unroll
        for (int i = 0; i < C::LPT; ++i) {
            const int32_t j = min(j0 + m.row[i], c.kv_total - 1);
            if (j >= sb && j < se) {
                // (j - r0) rows below the resource start, at this lane's chunk
                const uint32_t off = (uint32_t)((j - r0) - m.row[i]) * (uint32_t)row_bytes;
                if (do_k) dma16(rk, off + m.kg[i], kbuf.load_dst(i, wave));
                if (do_v) dma16(rv, off + m.vg[i], vbuf.load_dst(i, wave));
            }
        }
    }
}

// Instruction-class masks of sched_group_barrier (AMDGPU backend).
constexpr int kSgValu = 0x0002 | 0x0400;  // VALU, transcendentals included
constexpr int kSgMfma = 0x0008;
constexpr int kSgDsRead = 0x0100;
// Ask the scheduler for `n` instructions of class `mask` next, in this order.
#define sched_group(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Per-lane LDS byte offsets (relative to an LDS object), fixed for the kernel.
template <int D, int NW>
struct LdsAddr {
    uint32_t k[Cfg<D, NW>::DS];  // A operand of S^T, k-step ds: row l32, chunk (2 ds + h) ^ swz
    uint32_t v[Cfg<D, NW>::DB];  // V^T fragment of O block db (t = u = 0, block 0)
};

template <int D, int NW>
__device__ __forceinline__ LdsAddr<D, NW> lds_addr(int lane) {
    using C = Cfg<D, NW>;
    LdsAddr<D, NW> a;
    const int l32 = lane & 31, h = lane >> 5;
#pragma unroll
    for (int ds = 0; ds < C::DS; ++ds)
        a.k[ds] = (uint32_t)(l32 * C::ROWB + (((2 * ds + h) ^ swz_k<D, NW>(l32)) * 16));
    // transposing reads: in a 16-lane group, lane 4e+q names row 4h+e, dims 4q..4q+3
    // of its 16-dim half g&1 (g = lane/16, h = g/2)
    const int g = lane >> 4, e = (lane & 15) >> 2, q = lane & 3, hh = g >> 1;
    const int r = 4 * hh + e;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
        const int d = db * 32 + 16 * (g & 1) + 4 * q;
        a.v[db] = (uint32_t)(r * C::ROWB + (((d >> 3) ^ swz_v<D, NW>(r)) * 16) + (d & 7) * 2);
    }
    return a;
}

// S^T = K Q^T for one tile (two blocks of 32 keys), K from an LDS buffer.
template <int D, int NW>
__device__ __forceinline__ void qk_tile(const Buf<D, NW>& kbuf, const bf16x8* qf, const LdsAddr<D, NW>& la, f32x16* s) {
    using C = Cfg<D, NW>;
    s[0] = f32x16{};
    s[1] = f32x16{};
    const char LDS_AS* b0 = kbuf.template block_row<0>(0);
    const char LDS_AS* b1 = kbuf.template block_row<1>(0);
#pragma unroll
    for (int ds = 0; ds < C::DS; ++ds) {
        const bf16x8 a0 = *(const bf16x8 LDS_AS*)(b0 + la.k[ds]);
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[ds], s[0], 0, 0, 0);
        const bf16x8 a1 = *(const bf16x8 LDS_AS*)(b1 + la.k[ds]);
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[ds], s[1], 0, 0, 0);
    }
}

// V^T fragment (A operand) for O block db, key block KB, k-step t.  Within a
// 16-lane group, lane 4e+q addresses key row (.. + e) at dims 4q..4q+3 of its
// 16-dim half; the transposing read hands lane i dim (i%4) of the rows named by
// lanes i/4, i/4+4, i/4+8, i/4+12, i.e. one dim (db*32 + lane%32) for 4 keys.
// Two reads give the 8 keys of this lane's half: 16t + 8u + 4h + {0..3}, the
// key order of the S^T accumulator registers 8t..8t+7.
template <int D, int NW, int KB>
__device__ __forceinline__ bf16x8 v_frag(const Buf<D, NW>& vbuf, const LdsAddr<D, NW>& la, int db, int t) {
    using C = Cfg<D, NW>;
    const char LDS_AS* base = vbuf.template block_row<KB>(16 * t) + la.v[db];
    const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 LDS_AS*)base);
    const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 LDS_AS*)(base + 8 * C::ROWB));
    const s16x8 v = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// ---- FP8 QK^T (head_dim 128): a K tile of 64 keys x 128 one-byte codes (8 KB)
// in one LDS object; the 16-byte chunks of row r XOR-permuted by (r / 2) % 8, so
// the 16 lanes of a read phase (rows r..r+15, one logical chunk) hit distinct
// banks.  A-operand fragment of key block kb, k-step ks: lane (l32, h) holds row
// 32 kb + l32, dims 64 ks + 32 h .. + 31 (two chunks); the B operand (Q^T) uses
// the same dims per lane, which is all the contraction needs.
constexpr int kD8 = 128;
constexpr int kTile8 = BK * kD8;          // bytes of one K8 tile
constexpr int kDS8 = kD8 / 64;            // k-steps of 64 dims

__device__ __forceinline__ uint32_t k8_off(int l32, int h, int ks, int half) {
    const int chunk = 4 * ks + 2 * h + half;
    return (uint32_t)(l32 * kD8 + ((chunk ^ ((l32 >> 1) & 7)) * 16));
}

// rows 32..63 sit 4 KB further with the same permutation ((32 + r) / 2 % 8 = r / 2 % 8)
template <int KB>
__device__ __forceinline__ i32x8 k8_frag(const char LDS_AS* buf, const uint32_t* off, int ks) {
    const u32x4 a = *(const u32x4 LDS_AS*)(buf + KB * 32 * kD8 + off[2 * ks]);
    const u32x4 b = *(const u32x4 LDS_AS*)(buf + KB * 32 * kD8 + off[2 * ks + 1]);
    return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

// e4m3 x e4m3 -> fp32, unit block scales (E8M0 exponent 127 = 2^0)
__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// S^T = K Q^T for one FP8 tile (two blocks of 32 keys) from an LDS buffer.
__device__ __forceinline__ void qk_tile8(const char LDS_AS* kbuf, const i32x8* qf8, const uint32_t* off, f32x16* s) {
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kDS8; ++ks) {
        s[0] = mfma8(k8_frag<0>(kbuf, off, ks), qf8[ks], s[0]);
        s[1] = mfma8(k8_frag<1>(kbuf, off, ks), qf8[ks], s[1]);
    }
}

// One fp32 read through the vector memory path (counted with the direct loads,
// so the waits for LDS reads that follow need not drain it); 0 when !ok.
__device__ __forceinline__ float load_f32_vmem(const float* ptr, bool ok) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(ptr, ok ? 4u : 0u), 0, 0, 0));
}

// Workspace of the split tail: per piece the unnormalized O (BQ x D fp32) and
// per row (max reference, sum); merged by attn_merge_kernel after the
// attention kernel (stream order makes the pieces visible: no fences, no
// counters -- device-scope fences between pieces on different XCDs cost more
// than the whole tail).
template <int D, int NW>
struct SplitWs {
    static constexpr int BQ = NW * 32;
    static constexpr size_t kO = (size_t)BQ * D;
    static __device__ __forceinline__ float* piece(void* ws, int32_t idx) {
        return (float*)ws + (size_t)idx * (kO + 2 * BQ);
    }
    static __device__ __forceinline__ const float* piece(const void* ws, int32_t idx) {
        return (const float*)ws + (size_t)idx * (kO + 2 * BQ);
    }
};

template <int D, int NS, bool Q8, int NW>
__global__ __launch_bounds__(NW * 64, 2) void attn_bf16_kernel(Params<NS> prm) {
    using C = Cfg<D, NW>;
    constexpr int BQ = C::BQ;
    constexpr int kK8P = kTile8 / (NW * 1024);  // direct loads per thread of a K8 tile
    static_assert(kK8P >= 1 && kK8P * NW * 1024 == kTile8, "a K8 tile splits into whole wave loads");
    static_assert(!Q8 || D == kD8, "FP8 QK^T is built for head_dim 128");
    static_assert(!Q8 || C::PARTB == kTile8, "a K8 tile fills the first LDS object of a K buffer");
    const AttnCallN<NS>& c = prm.c;
    const AttnPlan& p = prm.p;
    // Separate LDS objects, each named statically in the unrolled loop below
    // (buffer stage x part), so the compiler can tell the objects being filled
    // by direct loads from the ones being read -- and the direct loads of one
    // tile from each other -- and adds no waits between them.
    __shared__ __attribute__((aligned(1024))) char k0p0[C::PARTB];
    __shared__ __attribute__((aligned(1024))) char k0p1[C::PARTS > 1 && !Q8 ? C::PARTB : 16];
    __shared__ __attribute__((aligned(1024))) char k1p0[C::PARTB];
    __shared__ __attribute__((aligned(1024))) char k1p1[C::PARTS > 1 && !Q8 ? C::PARTB : 16];
    __shared__ __attribute__((aligned(1024))) char v0p0[C::PARTB];
    __shared__ __attribute__((aligned(1024))) char v0p1[C::PARTS > 1 ? C::PARTB : 16];
    __shared__ __attribute__((aligned(1024))) char v1p0[C::PARTB];
    __shared__ __attribute__((aligned(1024))) char v1p1[C::PARTS > 1 ? C::PARTB : 16];
    __shared__ __attribute__((aligned(1024))) char dummy[NW * 1024];  // sink of loads that fetch nothing
    static_assert(C::PARTS <= 2, "at most two LDS objects per buffer");
    auto mkbuf = [](char* p0, char* p1) {
        Buf<D, NW> b;
        b.part[0] = (char LDS_AS*)p0;
        if constexpr (C::PARTS > 1) b.part[C::PARTS - 1] = (char LDS_AS*)p1;
        return b;
    };
    const Buf<D, NW> kb0 = mkbuf(k0p0, k0p1), kb1 = mkbuf(k1p0, k1p1);
    const Buf<D, NW> vb0 = mkbuf(v0p0, v0p1), vb1 = mkbuf(v1p0, v1p1);

    // ---- which unit (head, q-tile) and which key-tile range this workgroup runs
    [[maybe_unused]] uint64_t pc_entry = 0;
    WMK_STAMP(pc_entry);
    // The kernel arguments the unit's set-up reads, all loaded here: issued
    // together they cost one round trip to the scalar cache, where loads left at
    // their first use (inside the mask-mode and split branches) each waited for
    // their own.
    {
        const int32_t a0 = p.n_units, a1 = p.split_units, a2 = p.splits, a3 = p.xcd_remap, a4 = p.n_groups,
                      a5 = p.n_qtiles, a6 = c.q_tokens, a7 = c.heads, a8 = c.kv_total, a9 = c.kv.n,
                      a10 = c.mask.mode, a11 = c.mask.part_len, a12 = c.mask.chunk_len, a13 = c.mask.parts,
                      a14 = c.mask.env_len;
        const uint32_t b0 = p.splits_div.mul, b1 = p.splits_div.shift, b2 = p.qtiles_div.mul,
                       b3 = p.qtiles_div.shift, b4 = p.heads_div.mul, b5 = p.heads_div.shift,
                       b6 = c.mask.part_div.mul, b7 = c.mask.part_div.shift, b8 = c.mask.chunk_div.mul,
                       b9 = c.mask.chunk_div.shift;
        const float sc = c.scale;
        const void* qp = c.q;
        constexpr int F = NS < kFewSeg ? NS : kFewSeg;  // the spans of the common calls
        const void* sk[kFewSeg] = {};
        const void* sv[kFewSeg] = {};
        int32_t se[kFewSeg] = {};
#pragma unroll
        for (int x = 0; x < F; ++x) {
            sk[x] = c.kv.k[x];
            sv[x] = c.kv.v[x];
            se[x] = c.kv.end[x];
        }
        asm volatile("" ::"s"(a0), "s"(a1), "s"(a2), "s"(a3), "s"(a4), "s"(a5), "s"(a6), "s"(a7), "s"(a8), "s"(a9),
                     "s"(a10), "s"(a11), "s"(a12), "s"(a13), "s"(a14), "s"(b0), "s"(b1), "s"(b2), "s"(b3), "s"(b4),
                     "s"(b5), "s"(b6), "s"(b7), "s"(b8), "s"(b9), "s"(sc), "s"(qp));
        static_assert(kFewSeg == 5, "one asm operand per span field");
        asm volatile("" ::"s"(sk[0]), "s"(sk[1]), "s"(sk[2]), "s"(sk[3]), "s"(sk[4]), "s"(sv[0]), "s"(sv[1]),
                     "s"(sv[2]), "s"(sv[3]), "s"(sv[4]), "s"(se[0]), "s"(se[1]), "s"(se[2]), "s"(se[3]), "s"(se[4]));
    }
    const int32_t b = blockIdx.x;
    const int32_t full_units = p.n_units - p.split_units;
    int32_t u, piece = -1;
    if (b < full_units) {
        if (p.xcd_remap) {
            const int32_t x = b % kNumXcd, j = b / kNumXcd;
            const int32_t per = full_units / kNumXcd, rem = full_units % kNumXcd;
            u = x * per + min(x, rem) + j;
        } else {
            u = b;
        }
    } else {
        const int32_t pb = b - full_units, pu = tiles::udiv(pb, p.splits_div);
        u = full_units + pu;
        piece = pb - pu * p.splits;
    }
    int32_t head, qt;
    if (p.n_groups > 0) {  // longest-first order of q-tiles, all heads of a q-tile together
        const int32_t k = tiles::udiv(u, p.heads_div);
        head = u - k * c.heads;
        int32_t acc = 0;
        qt = 0;
        for (int g = 0; g < p.n_groups; ++g) {
            if (k >= acc && k < acc + p.grp_count[g]) qt = p.grp_start[g] + (k - acc);
            acc += p.grp_count[g];
        }
    } else {
        head = tiles::udiv(u, p.qtiles_div);
        qt = u - head * p.n_qtiles;
    }
    const int32_t r0 = qt * BQ, r1 = min(r0 + BQ, c.q_tokens);
    [[maybe_unused]] uint64_t fl0 = 0;
    WMK_STAMP(fl0);  // the unit is known: the kernel arguments have arrived
    // ---- per-lane query row; its Q fragments are loaded first, so that their
    // memory latency overlaps the planning below (tile ranges, row ranges)
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: keep it scalar
    const int l32 = lane & 31, h = lane >> 5;
    const int32_t row = r0 + wave * 32 + l32;
    const bool row_ok = row < c.q_tokens;
    const bool wave_has_rows = (r0 + wave * 32) < c.q_tokens;
    const int64_t stride = (int64_t)c.heads * D;

    // Q^T fragments (B operand): lane owns query l32, dims ds*16 + h*8 .. +7
    // (FP8: dims 64 ks + 32 h .. + 31 of the wave's quantized 32-row block)
    bf16x8 qf[Q8 ? 1 : C::DS];
    [[maybe_unused]] i32x8 qf8[kDS8];
    float cs0 = c.scale * kLog2e;
    if constexpr (Q8) {
        if (wave_has_rows) {
            const size_t qb = (size_t)(qt * NW + wave) * c.heads + head;
            const uint8_t* qp = p.q8 + qb * 32 * D + l32 * D + h * 32;
#pragma unroll
            for (int ks = 0; ks < kDS8; ++ks) {
                const u32x4 a = *(const u32x4*)(qp + ks * 64), b2 = *(const u32x4*)(qp + ks * 64 + 16);
                qf8[ks] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b2[0], (int)b2[1], (int)b2[2], (int)b2[3]};
            }
            const float sq = p.q8_scale[qb];
            cs0 *= sq > 0.0f ? sq : 1.0f;  // an all-zero block has zero codes: any positive factor
        }
    } else {
        const __bf16* qp = (const __bf16*)c.q + (int64_t)row * stride + (int64_t)head * D + h * 8;
#pragma unroll
        for (int ds = 0; ds < C::DS; ++ds) {
            u32x4 raw = row_ok ? *(const u32x4*)(qp + ds * 16) : u32x4{0u, 0u, 0u, 0u};
            qf[ds] = __builtin_bit_cast(bf16x8, raw);
        }
    }

    const TileRanges tr = tile_ranges(c, r0, r1);
    int32_t it0 = 0, it1 = tr.total;
    if (piece >= 0) {
        // tr.total * splits < 2^31 (the host caps the split count at total / 8)
        it0 = tiles::udiv(tr.total * piece, p.splits_div);
        it1 = tiles::udiv(tr.total * (piece + 1), p.splits_div);
    }

    int32_t lo0, hi0, lo1, hi1;
    row_ranges(c, row, lo0, hi0, lo1, hi1);

    f32x16 o[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) o[db] = f32x16{};
    float m_ref = -INFINITY, l_run = 0.0f;
    // exponent multipliers (scale * log2 e, times the block scales with FP8) of
    // the tile being finished (cs_a) and of the next one (cs_b)
    float cs_a = cs0, cs_b = cs0;
    auto k8_scale = [&](int32_t tile) __attribute__((always_inline)) -> float {
        const float sk = p.k8_scale[(size_t)tile * c.heads + head];
        return sk > 0.0f ? sk : 1.0f;  // an all-zero tile has zero codes: any positive factor
    };
    const LoadMap<D, NW> lm = load_map<D, NW>(wave, (uint32_t)(c.heads * D * 2));
    const LdsAddr<D, NW> la = lds_addr<D, NW>(lane);

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using NotLast = std::integral_constant<bool, false>;
    using Last = std::integral_constant<bool, true>;

    // Pipeline state between tiles: s = S^T(it) (raw dot products, masked),
    // m_ref its exponent reference, pf[0][*] the bf16 weights of its first 32
    // keys (computed early), l_run the weight sum so far (including them).
    f32x16 s[2];
    s[0] = f32x16{};
    s[1] = f32x16{};
    bf16x8 pf0[2];
    const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};

    // Mask S^T of tile `it` in place: nothing to do when every row of the wave
    // allows the whole tile (always, except at the tail, for chunk attention).
    auto mask_tile = [&](int32_t tile) __attribute__((always_inline)) {
        const int32_t j0 = tile * BK;
        if (c.mask.mode == kMaskNone && j0 + BK <= c.kv_total) return;
        const uint32_t lane_full = (row_ok ? 0u : 1u) | ((uint32_t)(lo0 <= j0) & (uint32_t)(j0 + BK <= hi0)) |
                                   ((uint32_t)(lo1 <= j0) & (uint32_t)(j0 + BK <= hi1));
        if (__builtin_amdgcn_ballot_w64(lane_full == 0u) == 0) return;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int32_t j = j0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                const uint32_t ok = in_range(j, lo0, hi0) | in_range(j, lo1, hi1);
                s[kb][r] = ok ? s[kb][r] : -INFINITY;
            }
    };

    // Row max of the (masked) S^T and the new exponent reference: m_ref moves
    // only when a row's tile max exceeds it by more than kTau (p <= 2^kTau).
    // Returns alpha, the factor by which earlier O and l must be scaled.
    auto new_ref = [&]() __attribute__((always_inline)) -> float {
        float mx = s[0][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
        const float mt = pair_max(mx) * cs_a;
        const bool grow = __builtin_amdgcn_ballot_w64(mt > m_ref + kTau) != 0;
        const float m_new = grow ? fmaxf(m_ref, mt) : m_ref;
        const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
        m_ref = m_new;
        return alpha;
    };

    // 8 weights of S^T register block (kb, t) -> bf16, and their sum
    auto weights = [&](auto kb_c, auto t_c, float m_use, float& lsum) __attribute__((always_inline)) -> bf16x8 {
        constexpr int kb = decltype(kb_c)::value, t = decltype(t_c)::value;
        f32x8 e;
#pragma unroll
        for (int r = 0; r < 8; ++r) e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * t + r], cs_a, -m_use));
        const bf16x8 p8 = __builtin_convertvector(e, bf16x8);
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
            const bf16x2 pp = {p8[2 * q2], p8[2 * q2 + 1]};
            lsum = __builtin_amdgcn_fdot2_f32_bf16(pp, one2, lsum, false);
        }
        return p8;
    };

    // ---- prologue: K(it0), V(it0) and K(it0+1) into LDS; S^T(it0) and its first weights
    // Cursors: vcu at the tile whose V is loaded next (it+1 in step it), kcu two ahead.
    const int64_t row_bytes = (int64_t)c.heads * D * 2;
    const int64_t head_off = (int64_t)head * D * 2;
    const uint32_t tile_bytes = (uint32_t)(BK * row_bytes);
    Cursor vcu = cursor_at(c, tr, it0, row_bytes, head_off);
    const int32_t tile0 = vcu.tile;
    Cursor kcu = vcu;
    // FP8: a K tile is one contiguous 8 KB block, copied as it stands (wave w
    // moves bytes [1 KB w, 1 KB (w + 1))); per-lane fragment offsets
    [[maybe_unused]] const uint32_t k8_lane = (uint32_t)(wave * 1024 + lane * 16);
    [[maybe_unused]] uint32_t k8o[2 * kDS8];
    if constexpr (Q8) {
#pragma unroll
        for (int ks = 0; ks < kDS8; ++ks) {
            k8o[2 * ks] = k8_off(l32, h, ks, 0);
            k8o[2 * ks + 1] = k8_off(l32, h, ks, 1);
        }
    }
    auto k8_src = [&](int32_t tile) __attribute__((always_inline)) {
        return p.k8 + ((size_t)tile * c.heads + head) * kTile8;
    };
    [[maybe_unused]] uint64_t fl1 = 0, fl2 = 0, fl3 = 0, fl4 = 0, fl5 = 0;
    WMK_STAMP(fl1);
    if (it0 < it1) {
        if constexpr (Q8) {
#pragma unroll
            for (int j = 0; j < kK8P; ++j)
                dma16(buffer_rsrc(k8_src(vcu.tile), kTile8), k8_lane + j * NW * 1024,
                      kb0.part[0] + (j * NW + wave) * 1024);
            issue_tile<D, NW>(c, head, vcu, lm, wave, kb0, vb0, false, true);
            cs_a = cs0 * k8_scale(vcu.tile);
        } else {
            issue_tile<D, NW>(c, head, vcu, lm, wave, kb0, vb0, true, true);
        }
        advance(vcu, c, tr, it0 + 1, row_bytes, head_off);
        if (it0 + 1 < it1) {
            if constexpr (Q8) {
#pragma unroll
                for (int j = 0; j < kK8P; ++j)
                    dma16(buffer_rsrc(k8_src(vcu.tile), kTile8), k8_lane + j * NW * 1024,
                          kb1.part[0] + (j * NW + wave) * 1024);
                cs_b = cs0 * k8_scale(vcu.tile);
            } else {
                issue_tile<D, NW>(c, head, vcu, lm, wave, kb1, vb1, true, false);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        WMK_STAMP(fl2);
        __syncthreads();
        WMK_STAMP(fl3);
        if (wave_has_rows) {
            if constexpr (Q8) qk_tile8(kb0.part[0], qf8, k8o, s);
            else qk_tile<D, NW>(kb0, qf, la, s);
            mask_tile(tile0);
            new_ref();  // O and l are still zero
            const float m_use = (m_ref == -INFINITY) ? 0.0f : m_ref;
            float lsum = 0.0f;
            pf0[0] = weights(I0{}, I0{}, m_use, lsum);
            pf0[1] = weights(I0{}, I1{}, m_use, lsum);
            l_run = lsum;
        }
        WMK_STAMP(fl4);
        __syncthreads();  // K(it0) is read; the first iteration refills its buffer
        WMK_STAMP(fl5);
    }
    kcu = vcu;
    advance(kcu, c, tr, it0 + 2, row_bytes, head_off);

    // One key tile; ST (compile time) is the buffer holding K(it) and V(it);
    // K(it+1) is in the other K buffer.  Fills K(it+2) into K buffer ST and
    // V(it+1) into the other V buffer while it computes.  LAST: no next tile.
    [[maybe_unused]] uint64_t prof[7] = {};  // step profile: A, B, load wait, barrier, issue, steps, span
    [[maybe_unused]] uint64_t prof_first = 0, real_first = 0, real_last = 0;
    auto step = [&](auto st_tag, auto last_tag, int32_t it) __attribute__((always_inline)) {
        [[maybe_unused]] uint64_t pc_s = 0, pc0 = 0, pc1 = 0, pc2 = 0, pc3 = 0, pc4 = 0;
        WMK_STAMP(pc_s);
        constexpr int ST = decltype(st_tag)::value;
        constexpr bool LAST = decltype(last_tag)::value;
        const Buf<D, NW>& kcur = ST ? kb1 : kb0;
        const Buf<D, NW>& knext = ST ? kb0 : kb1;
        const Buf<D, NW>& vcur = ST ? vb1 : vb0;
        const Buf<D, NW>& vnext = ST ? vb0 : vb1;
        // K(it+2) into kcur and V(it+1) into vnext, both read last in the
        // previous step; spread over the MFMAs of [A] (the tile interface is
        // busy for a while with each direct load, and a wave that issues all of
        // them at once stalls).  A tile crossing a span end is loaded here,
        // per span; its pieces then fetch nothing (zero-size resource) into a
        // dummy block, as do those of a tile past the range.
        const bool k_ok = it + 2 < it1, v_ok = it + 1 < it1;
        const bool k_fast = k_ok && (Q8 || kcu.run > 0), v_fast = v_ok && vcu.run > 0;
        if constexpr (!Q8) {
            if (k_ok && !k_fast) issue_tile<D, NW>(c, head, kcu, lm, wave, kcur, vnext, true, false);
        }
        if (v_ok && !v_fast) issue_tile<D, NW>(c, head, vcu, lm, wave, kcur, vnext, false, true);
        const __amdgpu_buffer_rsrc_t krs =
            Q8 ? buffer_rsrc(k8_src(k_ok ? kcu.tile : 0), k_ok ? (uint32_t)kTile8 : 0u)
               : buffer_rsrc(kcu.k, k_fast ? tile_bytes : 0u);
        const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(vcu.v, v_fast ? tile_bytes : 0u);
        // FP8: the block scale of K(it+2), used from the next step on
        [[maybe_unused]] float sk_next = 1.0f;
        if constexpr (Q8 && !LAST)
            sk_next = load_f32_vmem(p.k8_scale + (size_t)(k_ok ? kcu.tile : 0) * c.heads + head, k_ok);
        auto k_piece = [&](int i) __attribute__((always_inline)) {
            if constexpr (Q8)
                dma16(krs, k8_lane + i * NW * 1024,
                      k_ok ? kcur.part[0] + (i * NW + wave) * 1024 : (char LDS_AS*)dummy + wave * 1024);
            else dma16(krs, lm.kg[i], k_fast ? kcur.load_dst(i, wave) : (char LDS_AS*)dummy + wave * 1024);
        };
        auto v_piece = [&](int i) __attribute__((always_inline)) {
            dma16(vrs, lm.vg[i], v_fast ? vnext.load_dst(i, wave) : (char LDS_AS*)dummy + wave * 1024);
        };
        const int32_t tile_next = vcu.tile;
        vcu = kcu;
        advance(kcu, c, tr, it + 3, row_bytes, head_off);
        if (!wave_has_rows && !LAST) {
#pragma unroll
            for (int i = 0; i < C::LPT; ++i) {
                if (!Q8 || i < kK8P) k_piece(i);
                v_piece(i);
            }
        }

        if (wave_has_rows) {
            WMK_STAMP(pc0);
            // 8 waves: wave priority falls as the step progresses (3 at the start, 2
            // and 1 within [A], 0 halfway through [B]): of the two waves of a SIMD
            // the one behind keeps the higher priority, so both reach the barrier
            // together.  (By age alone, the older wave finished ~500 cycles early
            // every step and waited while the younger one ran alone.)  4 waves: the
            // two waves of a SIMD belong to two workgroups that meet at no barrier,
            // and the priorities only cost (720p cross-attention 2 % faster without).
            if constexpr (NW == 8) __builtin_amdgcn_s_setprio(3);
            const float m_use = (m_ref == -INFINITY) ? 0.0f : m_ref;
            // [A] S^T(it+1) = K(it+1) Q^T on the matrix core, next to the second
            //     half of this tile's weights (pf1) on the VALU.  The order is
            //     written out: K fragments KPF k-steps ahead, and a scheduling
            //     fence after each k-step keeps it.
            constexpr int KPF = 2;
            constexpr int EPS = 16 / C::DS;  // weights of s[1] per k-step
            f32x16 sn0 = f32x16{}, sn1 = f32x16{};
            f32x8 e0, e1;
            if constexpr (!LAST && Q8) {
                // FP8: all four fragments of K(it+1) up front, two k-steps of 64 dims
                const char LDS_AS* kn = knext.part[0];
                i32x8 ka8[kDS8][2];
#pragma unroll
                for (int ks = 0; ks < kDS8; ++ks) {
                    ka8[ks][0] = k8_frag<0>(kn, k8o, ks);
                    ka8[ks][1] = k8_frag<1>(kn, k8o, ks);
                }
                constexpr int EPS8 = 16 / kDS8;
#pragma unroll
                for (int ks = 0; ks < kDS8; ++ks) {
                    sn0 = mfma8(ka8[ks][0], qf8[ks], sn0);
#pragma unroll
                    for (int j = 0; j < kK8P; ++j)
                        if (j % kDS8 == ks) k_piece(j);
#pragma unroll
                    for (int i = 0; i < C::LPT; ++i)
                        if (i * kDS8 / C::LPT == ks) v_piece(i);
#pragma unroll
                    for (int x = 0; x < EPS8; ++x) {
                        const int idx = ks * EPS8 + x;
                        const float v = __builtin_amdgcn_exp2f(__builtin_fmaf(s[1][idx], cs_a, -m_use));
                        if (idx < 8) e0[idx] = v; else e1[idx - 8] = v;
                    }
                    sn1 = mfma8(ka8[ks][1], qf8[ks], sn1);
                    if (ks == kDS8 - 1) __builtin_amdgcn_s_setprio(1);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else if constexpr (!LAST) {
                const char LDS_AS* kn0 = knext.template block_row<0>(0);
                const char LDS_AS* kn1 = knext.template block_row<1>(0);
                bf16x8 ka[KPF + 1][2];
#pragma unroll
                for (int d = 0; d < KPF; ++d) {
                    ka[d][0] = *(const bf16x8 LDS_AS*)(kn0 + la.k[d]);
                    ka[d][1] = *(const bf16x8 LDS_AS*)(kn1 + la.k[d]);
                }
#pragma unroll
                for (int ds = 0; ds < C::DS; ++ds) {
                    if (ds + KPF < C::DS) {
                        ka[(ds + KPF) % (KPF + 1)][0] = *(const bf16x8 LDS_AS*)(kn0 + la.k[ds + KPF]);
                        ka[(ds + KPF) % (KPF + 1)][1] = *(const bf16x8 LDS_AS*)(kn1 + la.k[ds + KPF]);
                    }
                    sn0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ds % (KPF + 1)][0], qf[ds], sn0, 0, 0, 0);
                    // the LPT K pieces and LPT V pieces, alternating, one per SP / 2 k-steps
                    // (8 waves, head_dim 128: K at ds 1, 5; V at 3, 7)
                    constexpr int SP = C::DS / C::LPT;
                    if (ds % SP == SP / 4) k_piece(ds / SP);
                    if (ds % SP == (3 * SP) / 4) v_piece(ds / SP);
#pragma unroll
                    for (int x = 0; x < EPS; ++x) {
                        const int idx = ds * EPS + x;
                        const float v = __builtin_amdgcn_exp2f(__builtin_fmaf(s[1][idx], cs_a, -m_use));
                        if (idx < 8) e0[idx] = v; else e1[idx - 8] = v;
                    }
                    sn1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ds % (KPF + 1)][1], qf[ds], sn1, 0, 0, 0);
                    if (NW == 8 && ds == 3) __builtin_amdgcn_s_setprio(2);
                    if (NW == 8 && ds == 7) __builtin_amdgcn_s_setprio(1);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
#pragma unroll
                for (int idx = 0; idx < 16; ++idx) {
                    const float v = __builtin_amdgcn_exp2f(__builtin_fmaf(s[1][idx], cs_a, -m_use));
                    if (idx < 8) e0[idx] = v; else e1[idx - 8] = v;
                }
            }
            bf16x8 pf1[2];
            pf1[0] = __builtin_convertvector(e0, bf16x8);
            pf1[1] = __builtin_convertvector(e1, bf16x8);
            float lsum = 0.0f;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int q2 = 0; q2 < 4; ++q2) {
                    const bf16x2 pp = {pf1[t][2 * q2], pf1[t][2 * q2 + 1]};
                    lsum = __builtin_amdgcn_fdot2_f32_bf16(pp, one2, lsum, false);
                }
            // keep these weights here: they are only used after the mask branch
            // below, and would otherwise be sunk past it
            asm volatile("" ::"v"(pf1[0]), "v"(pf1[1]), "v"(lsum));
            l_run += lsum;
            WMK_STAMP(pc1);

            // [B] O^T += V(it)^T P(it)^T on the matrix core (V^T fragments VPF
            //     MFMAs ahead), next to the row max of S^T(it+1), the new
            //     reference and the first half of its weights (pn0) on the VALU,
            //     spread over the MFMAs by hand and fenced like [A].
            if constexpr (!LAST) {
                s[0] = sn0;
                s[1] = sn1;
                mask_tile(tile_next);
            }
            constexpr int NPV = 4 * C::DB;   // PV MFMAs: (db, t, kb)
            constexpr int VPF = 3;
            constexpr int RMX = NPV / 4;     // slots of the max reduction
            constexpr int SREF = RMX;        // slot of the new reference
            constexpr int WFIRST = RMX + 1;  // weights in slots WFIRST .. NPV - 2
            constexpr int WSLOTS = NPV - 1 - WFIRST;
            auto vfrag_at = [&](auto i_c) __attribute__((always_inline)) -> bf16x8 {
                constexpr int i = decltype(i_c)::value;
                if constexpr (i % 2 == 0) return v_frag<D, NW, 0>(vcur, la, i / 4, (i / 2) % 2);
                else return v_frag<D, NW, 1>(vcur, la, i / 4, (i / 2) % 2);
            };
            bf16x8 vfr[VPF + 1];
            [&]<int... I>(std::integer_sequence<int, I...>) __attribute__((always_inline)) {
                ((vfr[I] = vfrag_at(std::integral_constant<int, I>{})), ...);
            }(std::make_integer_sequence<int, VPF>{});
            float mx = -INFINITY, alpha = 1.0f, m_next = 0.0f, lsum_n = 0.0f;
            bool grow = false;
            f32x8 w0, w1;
            bf16x8 pn0[2];
            [&]<int... I>(std::integer_sequence<int, I...>) __attribute__((always_inline)) {
                auto slot = [&](auto i_c) __attribute__((always_inline)) {
                    constexpr int i = decltype(i_c)::value;
                    if constexpr (i + VPF < NPV) vfr[(i + VPF) % (VPF + 1)] = vfrag_at(std::integral_constant<int, i + VPF>{});
                    constexpr int db = i / 4, t = (i / 2) % 2, kb = i % 2;
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[i % (VPF + 1)], kb ? pf1[t] : pf0[t], o[db],
                                                                    0, 0, 0);
                    if constexpr (NW == 8 && i == NPV / 2) __builtin_amdgcn_s_setprio(0);
                    if constexpr (!LAST) {
                        if constexpr (i < RMX) {  // row max of S^T(it+1), 32 / RMX values per slot
#pragma unroll
                            for (int r = i * (32 / RMX); r < (i + 1) * (32 / RMX); ++r) mx = fmaxf(mx, s[r / 16][r % 16]);
                        } else if constexpr (i == SREF) {
                            const float mt = pair_max(mx) * cs_b;
                            grow = __builtin_amdgcn_ballot_w64(mt > m_ref + kTau) != 0;
                            const float m_new = grow ? fmaxf(m_ref, mt) : m_ref;
                            alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
                            m_ref = m_new;
                            m_next = (m_new == -INFINITY) ? 0.0f : m_new;
                        } else if constexpr (i >= WFIRST && i < NPV - 1) {  // weights of s[0]
#pragma unroll
                            for (int r = 0; r < 16; ++r)
                                if (WFIRST + r * WSLOTS / 16 == i) {
                                    const float v = __builtin_amdgcn_exp2f(__builtin_fmaf(s[0][r], cs_b, -m_next));
                                    if (r < 8) w0[r] = v; else w1[r - 8] = v;
                                }
                        } else if constexpr (i == NPV - 1) {
                            pn0[0] = __builtin_convertvector(w0, bf16x8);
                            pn0[1] = __builtin_convertvector(w1, bf16x8);
#pragma unroll
                            for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
                                for (int q2 = 0; q2 < 4; ++q2) {
                                    const bf16x2 pp = {pn0[t2][2 * q2], pn0[t2][2 * q2 + 1]};
                                    lsum_n = __builtin_amdgcn_fdot2_f32_bf16(pp, one2, lsum_n, false);
                                }
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                };
                (slot(std::integral_constant<int, I>{}), ...);
            }(std::make_integer_sequence<int, NPV>{});
            if constexpr (!LAST) {
                // keep the next tile's weights in the slots above (they are only
                // used after the branch below, and would otherwise be sunk past it)
                asm volatile("" ::"v"(pn0[0]), "v"(pn0[1]), "v"(lsum_n), "v"(alpha));
                if (grow) {  // rare: a row max grew by more than kTau
#pragma unroll
                    for (int db = 0; db < C::DB; ++db) o[db] *= alpha;
                    l_run *= alpha;
                }
                l_run += lsum_n;
                pf0[0] = pn0[0];
                pf0[1] = pn0[1];
            }
            WMK_STAMP(pc2);
        }
        __builtin_amdgcn_s_waitcnt(0);
        WMK_STAMP(pc3);
        __syncthreads();
        WMK_STAMP(pc4);
#ifdef WMK_STEP_PROFILE
        if (wave_has_rows) {
            prof[0] += pc1 - pc0;
            prof[1] += pc2 - pc1;
            prof[2] += pc3 - pc2;
            prof[3] += pc4 - pc3;
            prof[4] += pc0 - pc_s;
            prof[5] += 1;
            if (prof_first == 0) {
                prof_first = pc_s;
                real_first = __builtin_amdgcn_s_memrealtime();
            }
            prof[6] = pc4 - prof_first;
            if (LAST) real_last = __builtin_amdgcn_s_memrealtime();
        }
#endif
        if constexpr (Q8 && !LAST) {
            cs_a = cs_b;
            cs_b = cs0 * (sk_next > 0.0f ? sk_next : 1.0f);
        }
    };
    int32_t it = it0;
    for (; it + 2 < it1; it += 2) {
        step(I0{}, NotLast{}, it);
        step(I1{}, NotLast{}, it + 1);
    }
    // one or two tiles left (or none)
    if (it + 1 < it1) {
        step(I0{}, NotLast{}, it);
        step(I1{}, Last{}, it + 1);
    } else if (it < it1) {
        step(I0{}, Last{}, it);
    }

#ifdef WMK_STEP_PROFILE
    if (lane == 0 && blockIdx.x < 4096) {
        unsigned long long* e = g_step_prof[blockIdx.x * 8 + wave];  // 8 records per workgroup
        for (int i = 0; i < 7; ++i) e[i] = prof[i];
        e[7] = (unsigned long long)head << 32 | (unsigned long long)qt << 8 | (unsigned long long)(piece < 0 ? 255 : piece);
        e[8] = real_last - real_first;
        e[9] = prof_first - pc_entry;
        e[10] = fl1 - pc_entry;  // unit and ranges, Q fragment loads issued
        e[15] = fl0 - pc_entry;  // of which: until the unit is known (kernel arguments)
        e[11] = fl2 - fl1;       // first tiles issued, wait for them and for Q
        e[12] = fl3 - fl2;       // barrier
        e[13] = fl4 - fl3;       // first S^T, its max and first weights
        e[14] = fl5 - fl4;       // barrier
    }
#endif
    const float l_tot = pair_sum(l_run);
    __bf16* op = (__bf16*)c.out + (int64_t)row * stride + (int64_t)head * D;

    if (piece < 0) {
        if (row_ok) {
            const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
            // log sum exp of the scaled scores: m_ref and the weights are in log2 units
            if (c.lse != nullptr && h == 0)
                c.lse[(size_t)head * c.q_tokens + row] = l_tot > 0.0f ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
            // Lane (l32, h) holds dims 8 g + 4 h .. + 3 of its row for g = 0..3.  Per pair
            // of groups (g0, g1) the lanes l32 and l32 + 32 trade four values, so that
            // each stores 8 adjacent dims (16 bytes): h = 0 dims 8 g0 .. + 7, h = 1
            // dims 8 g1 .. + 7 -- 32 contiguous bytes of the row per store.
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int gp = 0; gp < 2; ++gp) {
                    const int g0 = 2 * gp, g1 = 2 * gp + 1;
                    const f32x4 a0 = {o[db][4 * g0] * inv, o[db][4 * g0 + 1] * inv, o[db][4 * g0 + 2] * inv,
                                      o[db][4 * g0 + 3] * inv};
                    const f32x4 a1 = {o[db][4 * g1] * inv, o[db][4 * g1 + 1] * inv, o[db][4 * g1 + 2] * inv,
                                      o[db][4 * g1 + 3] * inv};
                    const bf16x4 b0 = __builtin_convertvector(a0, bf16x4), b1 = __builtin_convertvector(a1, bf16x4);
                    const uint32_t* p0 = (const uint32_t*)&b0;
                    const uint32_t* p1 = (const uint32_t*)&b1;
                    const uint32_t k0 = h ? p1[0] : p0[0], k1 = h ? p1[1] : p0[1];  // kept
                    const uint32_t s0 = h ? p0[0] : p1[0], s1 = h ? p0[1] : p1[1];  // traded
                    // the swap returns the lane's own word and its partner's; take the other one
                    const auto r0 = __builtin_amdgcn_permlane32_swap(s0, s0, false, false);
                    const auto r1 = __builtin_amdgcn_permlane32_swap(s1, s1, false, false);
                    const uint32_t t0 = r0[0] == s0 ? r0[1] : r0[0], t1 = r1[0] == s1 ? r1[1] : r1[0];
                    const u32x4 w4 = h ? u32x4{t0, t1, k0, k1} : u32x4{k0, k1, t0, t1};
                    *(u32x4*)(op + db * 32 + 8 * (h ? g1 : g0)) = w4;
                }
        }
        return;
    }

    // ---- split tail: publish this piece; attn_merge_kernel combines the pieces
    const int32_t su = u - full_units;
    float* w = SplitWs<D, NW>::piece(p.ws, su * p.splits + piece);
    const int rl = wave * 32 + l32;  // row within the tile
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            *(f32x4*)(w + (size_t)rl * D + db * 32 + 8 * g + 4 * h) =
                f32x4{o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
    if (h == 0) {
        w[SplitWs<D, NW>::kO + 2 * rl] = m_ref;
        w[SplitWs<D, NW>::kO + 2 * rl + 1] = l_tot;
    }
}

// Merge of the split tail: out = sum_q 2^(m_q - M) O_q / sum_q 2^(m_q - M) l_q
// with M = max_q m_q, per row; one thread per (split unit, row, 8 dims).
struct MergeArgs {
    const void* ws;
    __bf16* out;
    float* lse;
    int32_t q_tokens;
    int32_t heads;
    int32_t n_qtiles;
    int32_t full_units;
    int32_t split_units;
    int32_t splits;
};

template <int D, int NW>
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeArgs a) {
    constexpr int BQ = NW * 32;
    constexpr int TPR = D / 8;  // threads per row
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= (int64_t)a.split_units * BQ * TPR) return;
    const int32_t su = (int32_t)(gid / (BQ * TPR)), rem = (int32_t)(gid % (BQ * TPR));
    const int32_t rl = rem / TPR, part = rem % TPR;
    const int32_t u = a.full_units + su;
    const int32_t head = u / a.n_qtiles, qt = u % a.n_qtiles;  // units in head-major order (no MoBA groups)
    const int32_t row = qt * BQ + rl;
    if (row >= a.q_tokens) return;
    float mmax = -INFINITY;
    for (int q = 0; q < a.splits; ++q)
        mmax = fmaxf(mmax, SplitWs<D, NW>::piece(a.ws, su * a.splits + q)[SplitWs<D, NW>::kO + 2 * rl]);
    const float mref = (mmax == -INFINITY) ? 0.0f : mmax;
    f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
    float lt = 0.0f;
    for (int q = 0; q < a.splits; ++q) {
        const float* w = SplitWs<D, NW>::piece(a.ws, su * a.splits + q);
        const float wq = __builtin_amdgcn_exp2f(w[SplitWs<D, NW>::kO + 2 * rl] - mref);
        lt += wq * w[SplitWs<D, NW>::kO + 2 * rl + 1];
        const f32x4* src = (const f32x4*)(w + (size_t)rl * D + part * 8);
        acc0 += wq * src[0];
        acc1 += wq * src[1];
    }
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    if (a.lse != nullptr && part == 0)
        a.lse[(size_t)head * a.q_tokens + row] = lt > 0.0f ? (mref + log2f(lt)) * kLn2 : -INFINITY;
    __bf16* dst = a.out + ((int64_t)row * a.heads + head) * D + part * 8;
    *(bf16x4*)dst = __builtin_convertvector(acc0 * inv, bf16x4);
    *(bf16x4*)(dst + 4) = __builtin_convertvector(acc1 * inv, bf16x4);
}

}  // namespace

int attn_bf16_block_q(int waves) { return waves * 32; }

size_t attn_bf16_split_ws_bytes(int head_dim, int waves, int32_t split_units, int32_t splits) {
    if (split_units <= 0 || splits <= 0) return 0;
    const size_t bq = (size_t)waves * 32;
    return (size_t)split_units * splits * (bq * head_dim + 2 * bq) * sizeof(float);
}

int attn_bf16_blocks_per_cu(int head_dim, int waves) {
    int n = 0;
    hipError_t e;
    if (waves == kWavesShort)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_bf16_kernel<128, kFewSeg, false, kWavesShort>,
                                                         kWavesShort * 64, 0);
    else if (head_dim == 64)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_bf16_kernel<64, kFewSeg, false, kWavesLong>,
                                                         kWavesLong * 64, 0);
    else
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_bf16_kernel<128, kFewSeg, false, kWavesLong>,
                                                         kWavesLong * 64, 0);
    return (e == hipSuccess && n > 0) ? n : 1;
}

template <int NS>
hipError_t launch_spans(const AttnCall& c, const AttnPlan& plan, int32_t blocks, hipStream_t s) {
    Params<NS> prm;
    prm.c.q = c.q;
    prm.c.out = c.out;
    prm.c.q_tokens = c.q_tokens;
    prm.c.heads = c.heads;
    prm.c.head_dim = c.head_dim;
    prm.c.kv_total = c.kv_total;
    prm.c.scale = c.scale;
    prm.c.mask = c.mask;
    prm.c.lse = plan.k8 != nullptr ? nullptr : c.lse;
    for (int x = 0; x < NS; ++x) {
        const bool in = x < c.kv.n;
        prm.c.kv.k[x] = in ? c.kv.k[x] : nullptr;
        prm.c.kv.v[x] = in ? c.kv.v[x] : nullptr;
        prm.c.kv.end[x] = in ? c.kv.end[x] : c.kv_total;
    }
    prm.c.kv.n = c.kv.n;
    prm.p = plan;
    constexpr int L = kWavesLong, S = kWavesShort;
    if (plan.waves == S)  // bf16, head_dim 128 only (checked by the caller)
        hipLaunchKernelGGL((attn_bf16_kernel<128, NS, false, S>), dim3(blocks), dim3(S * 64), 0, s, prm);
    else if (plan.k8 != nullptr)
        hipLaunchKernelGGL((attn_bf16_kernel<128, NS, true, L>), dim3(blocks), dim3(L * 64), 0, s, prm);
    else if (c.head_dim == 64)
        hipLaunchKernelGGL((attn_bf16_kernel<64, NS, false, L>), dim3(blocks), dim3(L * 64), 0, s, prm);
    else
        hipLaunchKernelGGL((attn_bf16_kernel<128, NS, false, L>), dim3(blocks), dim3(L * 64), 0, s, prm);
    return hipGetLastError();
}

hipError_t launch_attn_bf16(const AttnCall& c, const AttnPlan& plan, hipStream_t s) {
    const int32_t blocks = plan.n_units - plan.split_units + plan.split_units * plan.splits;
    if (blocks <= 0) return hipSuccess;
    if (c.kv.n < 0 || c.kv.n > kMaxSeg || (c.head_dim != 64 && c.head_dim != 128)) return hipErrorInvalidValue;
    if (plan.waves != kWavesLong && (plan.waves != kWavesShort || c.head_dim != 128 || plan.k8 != nullptr))
        return hipErrorInvalidValue;
    if (plan.k8 != nullptr && (c.head_dim != 128 || plan.q8 == nullptr || plan.k8_scale == nullptr ||
                               plan.q8_scale == nullptr))
        return hipErrorInvalidValue;
    // one cache run plus up to 4 segments (every call but a retained subset of
    // scattered frames): a span table small enough to stay in scalar registers
    const hipError_t e =
        c.kv.n <= kFewSeg ? launch_spans<kFewSeg>(c, plan, blocks, s) : launch_spans<kMaxSeg>(c, plan, blocks, s);
    if (e != hipSuccess || plan.split_units <= 0) return e;
    MergeArgs m;
    m.ws = plan.ws;
    m.out = (__bf16*)c.out;
    m.lse = plan.k8 != nullptr ? nullptr : c.lse;
    m.q_tokens = c.q_tokens;
    m.heads = c.heads;
    m.n_qtiles = plan.n_qtiles;
    m.full_units = plan.n_units - plan.split_units;
    m.split_units = plan.split_units;
    m.splits = plan.splits;
    const int64_t threads = (int64_t)plan.split_units * plan.waves * 32 * (c.head_dim / 8);
    const dim3 grid((uint32_t)((threads + 255) / 256));
    if (plan.waves == kWavesShort)
        hipLaunchKernelGGL((attn_merge_kernel<128, kWavesShort>), grid, dim3(256), 0, s, m);
    else if (c.head_dim == 64)
        hipLaunchKernelGGL((attn_merge_kernel<64, kWavesLong>), grid, dim3(256), 0, s, m);
    else
        hipLaunchKernelGGL((attn_merge_kernel<128, kWavesLong>), grid, dim3(256), 0, s, m);
    return hipGetLastError();
}

}  // namespace wmk
