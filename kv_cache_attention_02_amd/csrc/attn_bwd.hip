// Backward of the MoBA-masked attention (bf16, head_dim 128) on the CDNA4
// matrix cores: dQ, dK, dV of L = sum(dO * O) for O = softmax(scale Q K^T) V
// under the MoBA mask ("Infinite Worlds with Versatile Interactions", causal
// pretraining paragraph; "Mix Forcing", "Mix the training modes"), with the
// same per-tile skip as the forward: only tiles some row (or column) of a
// workgroup allows are visited.
//
// With the forward's log-sum-exp (lse) and D_i = dO_i . O_i, per head:
//   P = exp(scale Q K^T - lse),  dP = dO V^T,  dS = P * (dP - D),
//   dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K.
// Two kernels, each a loop over 64-row tiles staged in LDS by direct loads
// (double buffered, one barrier per tile), 8 waves x 32 rows of their own:
//   bwd_dq_kernel:   a workgroup owns 256 query rows and walks the key tiles
//                    its rows allow.  S^T = K Q^T and dP^T = V dO^T (lane =
//                    query, as in the forward), dS^T -> bf16, dQ^T += K^T dS^T
//                    with K^T from transposing LDS reads.
//   bwd_dkdv_kernel: a workgroup owns 256 keys and walks the query tiles that
//                    allow them.  S = Q K^T and dP = dO V^T (lane = key), P and
//                    dS -> bf16, dV^T += dO^T P and dK^T += Q^T dS with dO^T,
//                    Q^T from transposing LDS reads.
// A prologue kernel forms D from dO and O.  Every MFMA is
// v_mfma_f32_32x32x16_bf16; accumulators are fp32.
//
// LDS tiles are [64 rows][256 B], the 16-byte chunk c of row r stored at
// c ^ (((r & 3) << 2) | ((r >> 2) & 3)): 16 consecutive rows at one logical
// chunk hit 16 distinct chunk positions (row reads), and the 8 rows x 64 B of a
// transposing read spread over all banks.
#include <math.h>

#include "attn_tiles.h"
#include "wmk_internal.h"

namespace wmk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int NW = 8;            // waves per workgroup
constexpr int NT = NW * 64;      // threads per workgroup
constexpr int HD = 128;          // head_dim
constexpr int ROWB = HD * 2;     // bytes per row of one head
constexpr int TR = 64;           // rows per LDS tile
constexpr int TILEB = TR * ROWB; // 16 KB
constexpr int BR = NW * 32;      // rows a workgroup owns
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// Per-lane LDS byte offsets of the fragment reads, fixed for the kernel (kept
// few: the row-read offset of k-step ds is base + (xr ^ 32 ds), and the second
// transposing read of a k-step sits at (tr0 ^ 32) + 8 rows, because
// swz(r + 8) = swz(r) ^ 2 for r < 8).
struct Frag {
    uint32_t base;     // row read (A operand, row l32 of a 32-row block): row start + the chunk's low bit
    uint32_t xr;       // (swz(l32) & 14) * 16: the chunk bits the k-step's chunk is XORed with
    uint32_t tr0[4];   // transposing read, 32-dim block db, rows +0..7 of a 16-row k-step
};

__device__ __forceinline__ Frag frag_offsets(int lane) {
    Frag f;
    const int l32 = lane & 31, h = lane >> 5;
    // chunk (2 ds + h) ^ swz = (2 ds ^ (swz & 14)) + ((h ^ swz) & 1)
    f.base = (uint32_t)(l32 * ROWB + ((h ^ swz(l32)) & 1) * 16);
    f.xr = (uint32_t)((swz(l32) & 14) * 16);
    // in a 16-lane group, lane 4e+q names row 4hh+e (hh = g/2) at dims 4q..4q+3 of
    // its 16-dim half g&1 (g = lane/16); the read hands lane i dim (i%4) of the
    // rows of lanes i/4, i/4+4, ..: one dim (db*32 + lane%32) for 4 rows
    const int g = lane >> 4, e = (lane & 15) >> 2, q = lane & 3, hh = g >> 1;
    const int r = 4 * hh + e;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const int d = db * 32 + 16 * (g & 1) + 4 * q;
        f.tr0[db] = (uint32_t)(r * ROWB + (((d >> 3) ^ swz(r)) * 16) + (d & 7) * 2);
    }
    return f;
}

// A operand from rows: rows 32 kb + l32, dims 16 ds + 8 h .. + 7.  The eight
// row-read offsets base + (xr ^ 32 ds) are kept as separate values: every
// read is then one of them plus a compile-time offset (the tile object and the
// row block fold into the instruction's immediate).
struct RowOff {
    uint32_t o[8];
};
__device__ __forceinline__ RowOff row_offsets(const Frag& f) {
    RowOff r;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) r.o[ds] = f.base + (f.xr ^ (uint32_t)(32 * ds));
    return r;
}
__device__ __forceinline__ bf16x8 rows_frag(const char LDS_AS* tile, const RowOff& ro, int kb, int ds) {
    return *(const bf16x8 LDS_AS*)(tile + kb * 32 * ROWB + ro.o[ds]);
}

// A operand transposed: dim 32 db + lane%32, the 8 rows 32 kb + 16 t + 8 u + 4 h + {0..3}
// (u = 0, 1) -- the row order of registers 8t .. 8t+7 of a 32x32 accumulator
__device__ __forceinline__ bf16x8 tr_frag(const char LDS_AS* tile, const Frag& f, int kb, int db, int t) {
    const char LDS_AS* base = tile + (kb * 32 + 16 * t) * ROWB;
    const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 LDS_AS*)(base + f.tr0[db]));
    const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 LDS_AS*)(base + 8 * ROWB + (f.tr0[db] ^ 32u)));
    const s16x8 v = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// Keeps a value computed where it is written: an empty asm statement that
// reads and rewrites it, so the optimizer cannot sink its computation past this
// point (next to its use, after the MFMAs it is meant to run beside).
__device__ __forceinline__ void pin(bf16x8& x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// A buffer resource from values the caller knows to be uniform, moved to scalar
// registers explicitly (a clamp done on the VALU would otherwise leave them in
// vector registers, and every load through the resource in a per-lane loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_uniform(const void* base, uint32_t bytes) {
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    return rsrc((const void*)(uintptr_t)(((uint64_t)hi << 32) | lo), __builtin_amdgcn_readfirstlane(bytes));
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t off, char LDS_AS* dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void LDS_AS*)dst, 16, off, 0, 0, 0);
}

// Direct loads of rows [r0, r0 + 64) of one head of a [n][heads][128] bf16
// tensor into an LDS tile (two 16-byte loads per thread); rows past n read 0.
struct TileLoad {
    uint32_t off[2];  // byte offset from the tile's first row of this head
};
__device__ __forceinline__ TileLoad tile_load_map(int tid, uint32_t row_stride) {
    TileLoad m;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = 32 * i + tid / 16, phys = tid % 16;
        m.off[i] = (uint32_t)row * row_stride + (uint32_t)((phys ^ swz(row)) * 16);
    }
    return m;
}
__device__ __forceinline__ void load_tile(const char* src, int32_t r0, int32_t n, int32_t heads, int32_t head,
                                          const TileLoad& m, char LDS_AS* tile, int wave) {
    const uint32_t row_stride = (uint32_t)heads * ROWB;
    const int32_t valid = max(0, min(TR, n - r0));
    const __amdgpu_buffer_rsrc_t r = rsrc_uniform(src + ((size_t)r0 * heads + head) * ROWB, (uint32_t)valid * row_stride);
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(r, m.off[i], tile + i * (TILEB / 2) + wave * 1024);
}

using tiles::col_ranges;
using tiles::col_tile_ranges;

struct BwdArgs {
    const __bf16* q;
    const __bf16* k;
    const __bf16* v;
    const __bf16* dout;
    const float* lse;   // [heads][n], natural log
    const float* dsum;  // [heads][n], D = dO . O
    __bf16* dq;
    __bf16* dk;
    __bf16* dv;
    int32_t n;
    int32_t heads;
    float scale;
    MaskShape mask;
    // launch order of this kernel's tiles, longest walk first (0 groups: natural order)
    int32_t n_groups;
    int32_t grp_start[kMaxGroups];
    int32_t grp_count[kMaxGroups];
};

// exp2 exponent offset of a row: lse in log2 units; a row with no key (lse =
// -inf) gets +inf so that all its weights are 0
__device__ __forceinline__ float lse2_of(float lse) { return lse == -INFINITY ? INFINITY : lse * kLog2e; }

// ---- D_i = sum_d dO_id O_id per (row, head): 16 threads per row and head
__global__ __launch_bounds__(256) void bwd_dsum_kernel(const __bf16* dout, const __bf16* out, float* dsum, int32_t n,
                                                       int32_t heads) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t rh = gid / 16;  // row * heads + head
    const int part = (int)(gid % 16);
    float acc = 0.0f;
    if (rh < (int64_t)n * heads) {
        const u32x4 a = *(const u32x4*)(dout + rh * HD + part * 8);
        const u32x4 b = *(const u32x4*)(out + rh * HD + part * 8);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            acc += __uint_as_float(a[w] << 16) * __uint_as_float(b[w] << 16);
            acc += __uint_as_float(a[w] & 0xffff0000u) * __uint_as_float(b[w] & 0xffff0000u);
        }
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
    if (part == 0 && rh < (int64_t)n * heads) {
        const int32_t row = (int32_t)(rh / heads), head = (int32_t)(rh % heads);
        dsum[(size_t)head * n + row] = acc;
    }
}

// workgroup -> (head, tile of BR rows or keys).  With a group table: the
// tiles longest walk first, all heads of a tile together (a uniform walk length
// per launch position keeps the last round short); without: consecutive tiles
// of one head share an XCD.
__device__ __forceinline__ void unit_of(const BwdArgs& a, int32_t b, int32_t n_tiles, int32_t& head, int32_t& t) {
    if (a.n_groups > 0) {
        const int32_t k = b / a.heads;
        head = b - k * a.heads;
        int32_t acc = 0;
        t = 0;
        for (int g = 0; g < a.n_groups; ++g) {
            if (k >= acc && k < acc + a.grp_count[g]) t = a.grp_start[g] + (k - acc);
            acc += a.grp_count[g];
        }
        return;
    }
    const int32_t units = n_tiles * a.heads;
    const int32_t x = b % kNumXcd, j = b / kNumXcd;
    const int32_t per = units / kNumXcd, rem = units % kNumXcd;
    const int32_t u = x * per + min(x, rem) + j;  // XCD x runs units [x per + min(x, rem), ...)
    head = u / n_tiles;
    t = u % n_tiles;
}

// The tile ranges depend only on the workgroup; say so to the compiler, so
// that the buffer resources built from them stay in scalar registers (the
// direct loads then need no per-lane loop).
__device__ __forceinline__ tiles::TileRanges uniform(tiles::TileRanges r) {
    r.b0 = __builtin_amdgcn_readfirstlane(r.b0);
    r.e0 = __builtin_amdgcn_readfirstlane(r.e0);
    r.b1 = __builtin_amdgcn_readfirstlane(r.b1);
    r.e1 = __builtin_amdgcn_readfirstlane(r.e1);
    r.b2 = __builtin_amdgcn_readfirstlane(r.b2);
    r.e2 = __builtin_amdgcn_readfirstlane(r.e2);
    r.b3 = __builtin_amdgcn_readfirstlane(r.b3);
    r.e3 = __builtin_amdgcn_readfirstlane(r.e3);
    r.total = __builtin_amdgcn_readfirstlane(r.total);
    return r;
}

// The next tile's direct loads, issued in four pieces per thread (rows 0-31
// and 32-63 of the first tensor, then of the second) spread over the first
// MFMA group of a step: a wave that issues them all at once stalls on the
// load interface.
struct NextTile {
    __amdgpu_buffer_rsrc_t r0, r1;
    char LDS_AS* t0;
    char LDS_AS* t1;
    bool ok;
};
__device__ __forceinline__ NextTile next_tile(const tiles::TileRanges& tr, int32_t it, const __bf16* src0,
                                              const __bf16* src1, int32_t n, int32_t heads, int32_t head, char* t0,
                                              char* t1) {
    NextTile x;
    x.ok = it < tr.total;
    const int32_t r0 = x.ok ? tiles::tile_at(tr, it) * TR : 0;
    const uint32_t bytes = x.ok ? (uint32_t)max(0, min(TR, n - r0)) * (uint32_t)heads * ROWB : 0u;
    const size_t off = ((size_t)r0 * heads + head) * ROWB;
    x.r0 = rsrc_uniform((const char*)src0 + off, bytes);
    x.r1 = rsrc_uniform((const char*)src1 + off, bytes);
    x.t0 = (char LDS_AS*)t0;
    x.t1 = (char LDS_AS*)t1;
    return x;
}
__device__ __forceinline__ void next_piece(const NextTile& x, const TileLoad& m, int wave, int i) {
    if (!x.ok) return;
    if (i < 2) dma16(x.r0, m.off[i], x.t0 + i * (TILEB / 2) + wave * 1024);
    else dma16(x.r1, m.off[i - 2], x.t1 + (i - 2) * (TILEB / 2) + wave * 1024);
}

// ---- dQ: a workgroup owns BR query rows of one head
__global__ __launch_bounds__(NT, 2) void bwd_dq_kernel(BwdArgs a) {
    __shared__ __attribute__((aligned(1024))) char k0[TILEB];
    __shared__ __attribute__((aligned(1024))) char k1[TILEB];
    __shared__ __attribute__((aligned(1024))) char v0[TILEB];
    __shared__ __attribute__((aligned(1024))) char v1[TILEB];
    const int32_t n_tiles = (a.n + BR - 1) / BR;
    int32_t head, qt;
    unit_of(a, blockIdx.x, n_tiles, head, qt);
    const int32_t r0 = qt * BR, r1 = min(r0 + BR, a.n);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    const int32_t row = r0 + wave * 32 + l32;
    const bool row_ok = row < a.n;
    const bool wave_has_rows = r0 + wave * 32 < a.n;

    AttnCallN<1> rc{};  // row-interval view of the mask for tiles::row_ranges / tile_ranges
    rc.q_tokens = a.n;
    rc.kv_total = a.n;
    rc.mask = a.mask;
    const tiles::TileRanges tr = uniform(tiles::tile_ranges(rc, r0, r1));
    int32_t lo0, hi0, lo1, hi1;
    tiles::row_ranges(rc, row, lo0, hi0, lo1, hi1);

    const int64_t stride = (int64_t)a.heads * HD;
    bf16x8 qf[8], df[8];
    {
        const __bf16* qp = a.q + (int64_t)row * stride + (int64_t)head * HD + h * 8;
        const __bf16* dp = a.dout + (int64_t)row * stride + (int64_t)head * HD + h * 8;
#pragma unroll
        for (int ds = 0; ds < 8; ++ds) {
            qf[ds] = __builtin_bit_cast(bf16x8, row_ok ? *(const u32x4*)(qp + ds * 16) : u32x4{0u, 0u, 0u, 0u});
            df[ds] = __builtin_bit_cast(bf16x8, row_ok ? *(const u32x4*)(dp + ds * 16) : u32x4{0u, 0u, 0u, 0u});
        }
    }
    const float lse2 = row_ok ? lse2_of(a.lse[(size_t)head * a.n + row]) : INFINITY;
    const float dsr = row_ok ? a.dsum[(size_t)head * a.n + row] : 0.0f;
    const float cs = a.scale * kLog2e;
    const Frag fr = frag_offsets(lane);
    const RowOff ro = row_offsets(fr);
    const TileLoad lm = tile_load_map(threadIdx.x, (uint32_t)(a.heads * ROWB));
    f32x16 dq[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) dq[db] = f32x16{};

    // One key tile, two halves of 32 keys, in this written order (a scheduling
    // fence after each MFMA group keeps it):
    //   A0   S^T, dP^T of half 0 (16 MFMAs; the next tile's loads spread here)
    //   V0   dS^T of half 0 (VALU)
    //   A1   S^T, dP^T of half 1
    //   B0   dQ^T += K^T dS^T of half 0 (8 MFMAs), beside dS^T of half 1
    //   B1   dQ^T += K^T dS^T of half 1
    // Row fragments are read two k-steps ahead, K^T fragments two MFMAs ahead,
    // and the first reads of a group are made in the last steps of the one before.
    // full: every row of the wave allows the whole tile (the mask code is skipped)
    auto step = [&](bool full, int32_t j0, const char* kt_, const char* vt_, const NextTile& nx)
                    __attribute__((always_inline)) {
        const char LDS_AS* kt = (const char LDS_AS*)kt_;
        const char LDS_AS* vt = (const char LDS_AS*)vt_;
        bf16x8 kr[2][8], vr[2][8], kq[2][8];  // fragments, each read once (registers follow liveness)
        auto rows = [&](int kb, int ds) __attribute__((always_inline)) {
            kr[kb][ds] = rows_frag(kt, ro, kb, ds);
            vr[kb][ds] = rows_frag(vt, ro, kb, ds);
        };
        auto trs = [&](int kb, int m) __attribute__((always_inline)) { kq[kb][m] = tr_frag(kt, fr, kb, m >> 1, m & 1); };
        f32x16 s, dp;
        // masked keys get a score of -inf (weight 0); one uniform branch per half
        auto mask = [&](int kb) __attribute__((always_inline)) {
            if (full) return;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int32_t j = j0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                const uint32_t ok = tiles::in_range(j, lo0, hi0) | tiles::in_range(j, lo1, hi1);
                s[r] = ok ? s[r] : -INFINITY;
            }
        };
        // dS^T = P^T (dP^T - D) for accumulator registers 4g .. 4g + 3, in bf16
        auto dsg = [&](int g, bf16x8* dsb) __attribute__((always_inline)) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int r = 4 * g + w;
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], cs, -lse2));
                dsb[r >> 3][r & 7] = (__bf16)(p * (dp[r] - dsr));
            }
        };
        bf16x8 ds0[2], ds1[2];
        // wave priority falls as the tile progresses (3, 2 after A0, 1 after A1,
        // 0 after B0): of the two waves of a SIMD the one behind keeps the
        // higher priority, so both reach the barrier together
        __builtin_amdgcn_s_setprio(3);
        // A0
        rows(0, 0);
        rows(0, 1);
        s = f32x16{};
        dp = f32x16{};
#pragma unroll
        for (int ds = 0; ds < 8; ++ds) {
            if (ds + 2 < 8) rows(0, ds + 2);
            else rows(1, ds - 6);
            s = mfma(kr[0][ds], qf[ds], s);
            dp = mfma(vr[0][ds], df[ds], dp);
            if (ds & 1) next_piece(nx, lm, wave, ds >> 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        // V0
        __builtin_amdgcn_s_setprio(2);
        mask(0);
#pragma unroll
        for (int g = 0; g < 4; ++g) dsg(g, ds0);
        pin(ds0[0]);
        pin(ds0[1]);
        __builtin_amdgcn_sched_barrier(0);
        // A1
        s = f32x16{};
        dp = f32x16{};
#pragma unroll
        for (int ds = 0; ds < 8; ++ds) {
            if (ds + 2 < 8) rows(1, ds + 2);
            else trs(0, ds - 6);
            s = mfma(kr[1][ds], qf[ds], s);
            dp = mfma(vr[1][ds], df[ds], dp);
            __builtin_amdgcn_sched_barrier(0);
        }
        mask(1);
        __builtin_amdgcn_s_setprio(1);
        __builtin_amdgcn_sched_barrier(0);
        // B0 beside V1
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            if (m + 2 < 8) trs(0, m + 2);
            else trs(1, m - 6);
            dq[m >> 1] = mfma(kq[0][m], ds0[m & 1], dq[m >> 1]);
            if (m & 1) {
                dsg(m >> 1, ds1);
                pin(ds1[m >> 2]);
            }
            if (m == 7) __builtin_amdgcn_s_setprio(0);
            __builtin_amdgcn_sched_barrier(0);
        }
        // B1
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            if (m + 2 < 8) trs(1, m + 2);
            dq[m >> 1] = mfma(kq[1][m], ds1[m & 1], dq[m >> 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto run = [&](int32_t it, char* kt, char* vt, char* kn, char* vn) __attribute__((always_inline)) {
        const NextTile nx = next_tile(tr, it + 1, a.k, a.v, a.n, a.heads, head, kn, vn);
        if (wave_has_rows) {
            const int32_t j0 = tiles::tile_at(tr, it) * TR;
            const bool full = __builtin_amdgcn_ballot_w64(!row_ok || ((lo0 <= j0) & (j0 + TR <= hi0)) ||
                                                          ((lo1 <= j0) & (j0 + TR <= hi1))) == ~0ull;
            step(full, j0, kt, vt, nx);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) next_piece(nx, lm, wave, i);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    if (tr.total > 0) {
        const NextTile first = next_tile(tr, 0, a.k, a.v, a.n, a.heads, head, k0, v0);
#pragma unroll
        for (int i = 0; i < 4; ++i) next_piece(first, lm, wave, i);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    for (int32_t it = 0; it < tr.total; it += 2) {
        run(it, k0, v0, k1, v1);
        if (it + 1 >= tr.total) break;
        run(it + 1, k1, v1, k0, v0);
    }

    if (row_ok) {
        __bf16* op = a.dq + (int64_t)row * stride + (int64_t)head * HD;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 v4 = {dq[db][4 * g] * a.scale, dq[db][4 * g + 1] * a.scale, dq[db][4 * g + 2] * a.scale,
                            dq[db][4 * g + 3] * a.scale};
                *(bf16x4*)(op + db * 32 + 8 * g + 4 * h) = __builtin_convertvector(v4, bf16x4);
            }
    }
}

// ---- dK, dV: a workgroup owns BR keys of one head
__global__ __launch_bounds__(NT, 2) void bwd_dkdv_kernel(BwdArgs a) {
    __shared__ __attribute__((aligned(1024))) char q0[TILEB];
    __shared__ __attribute__((aligned(1024))) char q1[TILEB];
    __shared__ __attribute__((aligned(1024))) char d0[TILEB];
    __shared__ __attribute__((aligned(1024))) char d1[TILEB];
    __shared__ __attribute__((aligned(16))) float rowv[2][2][TR];  // [buffer][lse2, D][row of the tile]
    __shared__ __attribute__((aligned(1024))) char vown[BR * ROWB];  // V of the workgroup's keys (B operand of dP)
    const int32_t n_tiles = (a.n + BR - 1) / BR;
    int32_t head, kt;
    unit_of(a, blockIdx.x, n_tiles, head, kt);
    const int32_t c0 = kt * BR;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    const int32_t key = c0 + wave * 32 + l32;
    const bool key_ok = key < a.n;
    const bool wave_has_keys = c0 + wave * 32 < a.n;
    const tiles::TileRanges tr = uniform(col_tile_ranges(a.mask, a.n, c0, c0 + BR));
    int32_t lo0, hi0, lo1, hi1;
    col_ranges(a.mask, a.n, key, lo0, hi0, lo1, hi1);

    const int64_t stride = (int64_t)a.heads * HD;
    // K^T as B operand in registers: lane = key l32, dims 16 ds + 8 h .. + 7; V^T
    // (the same fragments of V) is read from LDS, where this workgroup's V rows
    // stay for the whole loop (registers hold the dK^T, dV^T accumulators)
    bf16x8 kf[8];
    {
        const __bf16* kp = a.k + (int64_t)key * stride + (int64_t)head * HD + h * 8;
#pragma unroll
        for (int ds = 0; ds < 8; ++ds)
            kf[ds] = __builtin_bit_cast(bf16x8, key_ok ? *(const u32x4*)(kp + ds * 16) : u32x4{0u, 0u, 0u, 0u});
    }
    const float cs = a.scale * kLog2e;
    const Frag fr = frag_offsets(lane);
    const RowOff ro = row_offsets(fr);
    const TileLoad lm = tile_load_map(threadIdx.x, (uint32_t)(a.heads * ROWB));
#pragma unroll
    for (int i = 0; i < BR / TR; ++i)
        load_tile((const char*)a.v, c0 + i * TR, a.n, a.heads, head, lm, (char LDS_AS*)vown + i * TILEB, wave);
    const char LDS_AS* vw = (const char LDS_AS*)vown + wave * 32 * ROWB;  // this wave's 32 keys
    f32x16 dk[4], dv[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        dk[db] = f32x16{};
        dv[db] = f32x16{};
    }

    // the tile's row values (lse in log2 units, D) go through registers into LDS
    float rv_l = 0.0f, rv_d = 0.0f;
    auto fetch_rows = [&](int32_t it) __attribute__((always_inline)) {
        const int32_t i = tiles::tile_at(tr, it) * TR + (int32_t)threadIdx.x;
        if (threadIdx.x < TR) {
            rv_l = i < a.n ? lse2_of(a.lse[(size_t)head * a.n + i]) : INFINITY;
            rv_d = i < a.n ? a.dsum[(size_t)head * a.n + i] : 0.0f;
        }
    };
    auto store_rows = [&](int buf) __attribute__((always_inline)) {
        if (threadIdx.x < TR) {
            rowv[buf][0][threadIdx.x] = rv_l;
            rowv[buf][1][threadIdx.x] = rv_d;
        }
    };

    // One query tile as one stream of 64 MFMAs, per 32-row half qb:
    //   S   = Q K^T               (8; Q rows from LDS, K^T in registers)
    //   P   = 2^(S cs - lse)       VALU, rounded to bf16
    //   dV^T += dO^T P            (8; dO^T from transposing reads)
    //   dP  = dO V^T              (8; dO rows and this wave's V rows from LDS)
    //   dS  = P (dP - D)           VALU, in bf16
    //   dK^T += Q^T dS            (8; Q^T from transposing reads)
    // Every fragment is read two MFMAs ahead of its use, across the VALU steps
    // too; a scheduling fence after each MFMA keeps this written order, and the
    // next tile's direct loads are spread over the first S group.  The two
    // halves run as a loop (not unrolled): the mask branch of an unrolled pair
    // costs more registers than the kernel has.
    auto step = [&](bool full, int32_t i0, const char* qt_, const char* dt_, int buf, const NextTile& nx)
                    __attribute__((always_inline)) {
        const char LDS_AS* qt = (const char LDS_AS*)qt_;
        const char LDS_AS* dt = (const char LDS_AS*)dt_;
        bf16x8 fa[32], fb[32];  // fragments of MFMA n of a half (fb: the dP group's B operand)
        auto fetch = [&](int qb, int n) __attribute__((always_inline)) {
            const int ph = (n >> 3) & 3, i = n & 7;
            if (ph == 0) {
                fa[n] = rows_frag(qt, ro, qb, i);
            } else if (ph == 1) {
                fa[n] = tr_frag(dt, fr, qb, i >> 1, i & 1);
            } else if (ph == 2) {
                fa[n] = rows_frag(dt, ro, qb, i);
                fb[n] = rows_frag(vw, ro, 0, i);
            } else {
                fa[n] = tr_frag(qt, fr, qb, i >> 1, i & 1);
            }
        };
        f32x16 s, dp;
        bf16x8 pb[2], dsb[2];
        auto weights = [&](int qb) __attribute__((always_inline)) {
            if (!full) {
                // rows of the half that may not see this lane's key: score -inf.
                // Register r holds row i0 + 32 qb + 4 h + c(r), c(r) = 8 (r/4) + r%4;
                // the test (i - lo) < (hi - lo) (unsigned) is one add of c(r) to a
                // per-step base (pinned, so that the compiler does not keep a
                // hoisted copy of base + c(r) for every r across the loop).
                int32_t b0 = i0 + qb * 32 + 4 * h - lo0, b1 = i0 + qb * 32 + 4 * h - lo1;
                asm volatile("" : "+v"(b0), "+v"(b1));
                const uint32_t n0 = (uint32_t)(hi0 - lo0), n1 = (uint32_t)(hi1 - lo1);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int32_t c = 8 * (r >> 2) + (r & 3);
                    const bool ok = ((uint32_t)(b0 + c) < n0) | ((uint32_t)(b1 + c) < n1);
                    s[r] = ok ? s[r] : -INFINITY;
                }
            }
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                // registers 4g .. 4g+3 hold rows 32 qb + 16 (g/2) + 8 (g%2) + 4 h + {0..3}
                const f32x4 l4 = *(const f32x4*)&rowv[buf][0][qb * 32 + 8 * g + 4 * h];
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    pb[g >> 1][4 * (g & 1) + w] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * g + w], cs, -l4[w]));
            }
            pin(pb[0]);
            pin(pb[1]);
        };
        auto dscores = [&](int qb) __attribute__((always_inline)) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 d4 = *(const f32x4*)&rowv[buf][1][qb * 32 + 8 * g + 4 * h];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const int e = 4 * (g & 1) + w;
                    dsb[g >> 1][e] = (__bf16)((float)pb[g >> 1][e] * (dp[4 * g + w] - d4[w]));
                }
            }
            pin(dsb[0]);
            pin(dsb[1]);
        };
        // wave priority falls as the tile progresses (3; 2 after the dV group of
        // half 0; 1 after half 0; 0 after the dV group of half 1), as in dQ
        __builtin_amdgcn_s_setprio(3);
#pragma nounroll
        for (int qb = 0; qb < 2; ++qb) {
        fetch(qb, 0);
        fetch(qb, 1);
#pragma unroll
        for (int n = 0; n < 32; ++n) {
            const int ph = (n >> 3) & 3, i = n & 7;
            if (n + 2 < 32) fetch(qb, n + 2);
            if (ph == 0) {
                if (i == 0) s = f32x16{};
                s = mfma(fa[n], kf[i], s);
                if (qb == 0 && (i & 1)) next_piece(nx, lm, wave, i >> 1);
            } else if (ph == 1) {
                dv[i >> 1] = mfma(fa[n], pb[i & 1], dv[i >> 1]);
            } else if (ph == 2) {
                if (i == 0) dp = f32x16{};
                dp = mfma(fa[n], fb[n], dp);
            } else {
                dk[i >> 1] = mfma(fa[n], dsb[i & 1], dk[i >> 1]);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (i == 7 && ph == 0) weights(qb);
            if (i == 7 && ph == 2) dscores(qb);
            if (i == 7 && ph == 1) {
                if (qb) __builtin_amdgcn_s_setprio(0);
                else __builtin_amdgcn_s_setprio(2);
            }
            if (i == 7 && ph == 3 && qb == 0) __builtin_amdgcn_s_setprio(1);
            __builtin_amdgcn_sched_barrier(0);
        }
        }
    };
    auto run = [&](int32_t it, char* qt, char* dt, char* qn, char* dn, int buf) __attribute__((always_inline)) {
        const NextTile nx = next_tile(tr, it + 1, a.q, a.dout, a.n, a.heads, head, qn, dn);
        const bool more = it + 1 < tr.total;
        if (more) fetch_rows(it + 1);
        if (wave_has_keys) {
            const int32_t i0 = tiles::tile_at(tr, it) * TR;
            const bool full = __builtin_amdgcn_ballot_w64(!key_ok || ((lo0 <= i0) & (i0 + TR <= hi0)) ||
                                                          ((lo1 <= i0) & (i0 + TR <= hi1))) == ~0ull;
            step(full, i0, qt, dt, buf, nx);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) next_piece(nx, lm, wave, i);
        }
        if (more) store_rows(buf ^ 1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    if (tr.total > 0) {
        const NextTile first = next_tile(tr, 0, a.q, a.dout, a.n, a.heads, head, q0, d0);
#pragma unroll
        for (int i = 0; i < 4; ++i) next_piece(first, lm, wave, i);
        fetch_rows(0);
        store_rows(0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    for (int32_t it = 0; it < tr.total; it += 2) {
        run(it, q0, d0, q1, d1, 0);
        if (it + 1 >= tr.total) break;
        run(it + 1, q1, d1, q0, d0, 1);
    }

    if (key_ok) {
        __bf16* kp = a.dk + (int64_t)key * stride + (int64_t)head * HD;
        __bf16* vp = a.dv + (int64_t)key * stride + (int64_t)head * HD;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 k4 = {dk[db][4 * g] * a.scale, dk[db][4 * g + 1] * a.scale, dk[db][4 * g + 2] * a.scale,
                            dk[db][4 * g + 3] * a.scale};
                f32x4 v4 = {dv[db][4 * g], dv[db][4 * g + 1], dv[db][4 * g + 2], dv[db][4 * g + 3]};
                *(bf16x4*)(kp + db * 32 + 8 * g + 4 * h) = __builtin_convertvector(k4, bf16x4);
                *(bf16x4*)(vp + db * 32 + 8 * g + 4 * h) = __builtin_convertvector(v4, bf16x4);
            }
    }
}

}  // namespace

hipError_t launch_moba_backward(const MobaBwd& b, hipStream_t s) {
    if (b.n <= 0 || b.heads <= 0) return hipErrorInvalidValue;
    BwdArgs a;
    a.q = (const __bf16*)b.q;
    a.k = (const __bf16*)b.k;
    a.v = (const __bf16*)b.v;
    a.dout = (const __bf16*)b.dout;
    a.lse = b.lse;
    a.dsum = b.dsum;
    a.dq = (__bf16*)b.dq;
    a.dk = (__bf16*)b.dk;
    a.dv = (__bf16*)b.dv;
    a.n = b.n;
    a.heads = b.heads;
    a.scale = b.scale;
    a.mask = b.mask;
    const int64_t rows = (int64_t)b.n * b.heads;
    hipLaunchKernelGGL(bwd_dsum_kernel, dim3((uint32_t)((rows * 16 + 255) / 256)), dim3(256), 0, s, (const __bf16*)b.dout,
                       (const __bf16*)b.out, b.dsum, b.n, b.heads);
    const uint32_t units = (uint32_t)(((b.n + BR - 1) / BR) * b.heads);
    a.n_groups = b.n_groups_k;
    for (int g = 0; g < kMaxGroups; ++g) {
        a.grp_start[g] = b.grp_k_start[g];
        a.grp_count[g] = b.grp_k_count[g];
    }
    hipLaunchKernelGGL(bwd_dkdv_kernel, dim3(units), dim3(NT), 0, s, a);
    a.n_groups = b.n_groups_q;
    for (int g = 0; g < kMaxGroups; ++g) {
        a.grp_start[g] = b.grp_q_start[g];
        a.grp_count[g] = b.grp_q_count[g];
    }
    hipLaunchKernelGGL(bwd_dq_kernel, dim3(units), dim3(NT), 0, s, a);
    return hipGetLastError();
}

int moba_bwd_block() { return BR; }

}  // namespace wmk
