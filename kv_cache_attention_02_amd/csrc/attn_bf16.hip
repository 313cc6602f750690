// bf16 attention on the CDNA4 matrix cores (gfx950).
//
// One workgroup = 4 waves = 128 query rows of one head (32 rows per wave); keys
// are visited in tiles of 64, staged in LDS (double-buffered, one barrier per
// tile) and shared by the 4 waves.
//
// Per wave and tile:
//   S^T[key][q] = K . Q^T        v_mfma_f32_32x32x16_bf16, K from LDS (A), Q^T
//                                from registers (B, loaded once).  In the 32x32
//                                accumulator layout lane l owns query l%32 and
//                                16 of the tile's 32 keys per block; the other 16
//                                sit in lane l^32, so a row max or sum is a
//                                register reduction plus one permlane32 swap.
//   online softmax in fp32       exp2 with scale*log2(e) folded into one FMA;
//                                the accumulator is rescaled only when some row
//                                max of the wave grew.
//   O^T[d][q] += V^T . P^T       the S^T accumulator, rounded to bf16, is the B
//                                operand as it stands; V^T comes from LDS, where
//                                it is stored transposed with its keys permuted
//                                to the accumulator's key order.
//
// Masks come from key intervals: every row allows at most two half-open key
// ranges (the whole key range at a chunk step; the MoBA ranges in training).
// A tile that every row of a wave fully allows runs unmasked; any other
// visited tile applies the per-element interval test.  Tiles that no row of
// the workgroup allows are never visited: the workgroup walks only the union of
// its rows' ranges, in tile units.
//
// Sources: chunk attention over [anchors | recent | current] ("Westlake AGI
// Lab's 'World in World' Steers Frozen Video Models", second paragraph); the
// MoBA mask ("Infinite Worlds with Versatile Interactions", causal pretraining
// paragraph; "Mix Forcing: Causal Pre-Training via Mixture Attention for
// Interactive World Models", "Mix the training modes").
#include <math.h>

#include "wmk_internal.h"

namespace wmk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BQ = 128;  // query rows per workgroup
constexpr int BK = 64;   // keys per tile
constexpr int NT = 256;  // threads per workgroup (4 waves)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kTau = 8.0f;  // lazy-rescale threshold, log2 units (weights stay <= 256)

template <int D>
struct Cfg {
    static constexpr int KS = D + 8;           // LDS row stride of K (bf16 elements, 16 B pad)
    static constexpr int VS = BK + 8;          // LDS row stride of V^T
    static constexpr int KE = BK * KS;
    static constexpr int VE = D * VS;
    static constexpr int BUF = KE + VE;        // one pipeline stage
    static constexpr int DS = D / 16;          // k-steps of S = K Q^T
    static constexpr int DB = D / 32;          // 32-row blocks of O^T
    static constexpr int KCH = D / 8;          // 16-byte chunks per row
    static constexpr int KLD = BK * KCH / NT;  // K chunks loaded per thread
    static constexpr int VIT = 16 * KCH;       // V items: (4-key quad, 8-dim chunk)
};

struct Params {
    AttnCall c;
    AttnPlan p;
};

// The tile ranges a workgroup visits: union over its rows of their allowed key
// ranges, rounded out to whole tiles, sorted and merged (at most 4 ranges).
// Written with fixed slots, a sorting network and selects -- no dynamically
// indexed arrays -- so that it stays in scalar registers: an array here would
// live in scratch memory, and every scratch read in the tile loop would wait
// for the in-flight prefetch of the next tile.
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

__device__ __forceinline__ TileRanges tile_ranges(const AttnCall& c, int32_t r0, int32_t r1) {
    int32_t l0 = kNone, h0 = kNone, l1 = kNone, h1 = kNone, l2 = kNone, h2 = kNone, l3 = kNone, h3 = kNone;
    if (!c.moba.enabled) {
        set_tiles(l0, h0, 0, c.kv_total);
    } else {
        const int32_t L = c.moba.part_len, cl = c.moba.chunk_len;
        const int32_t pa = r0 / L, pb = min((r1 - 1) / L, c.moba.parts - 1);
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
    order(l0, h0, l1, h1);
    order(l2, h2, l3, h3);
    order(l0, h0, l2, h2);
    order(l1, h1, l3, h3);
    order(l1, h1, l2, h2);
    TileRanges r = {0, 0, 0, 0, 0, 0, 0, 0, 0};
    int k = 0;
    int32_t cb = l0, ce = h0;
#define WMK_MERGE(L_, H_)                                      \
    if (L_ != kNone) {                                         \
        if (L_ <= ce) {                                        \
            ce = max(ce, H_);                                  \
        } else {                                               \
            emit(r, k, cb, ce);                                \
            ++k;                                               \
            cb = L_;                                           \
            ce = H_;                                           \
        }                                                      \
    }
    WMK_MERGE(l1, h1)
    WMK_MERGE(l2, h2)
    WMK_MERGE(l3, h3)
#undef WMK_MERGE
    if (cb != kNone) emit(r, k, cb, ce);
    r.total = (r.e0 - r.b0) + (r.e1 - r.b1) + (r.e2 - r.b2) + (r.e3 - r.b3);
    return r;
}

__device__ __forceinline__ int32_t tile_at(const TileRanges& r, int32_t it) {
    const int32_t n0 = r.e0 - r.b0, n1 = n0 + (r.e1 - r.b1), n2 = n1 + (r.e2 - r.b2);
    return it < n0 ? r.b0 + it : it < n1 ? r.b1 + (it - n0) : it < n2 ? r.b2 + (it - n1) : r.b3 + (it - n2);
}

// Allowed key ranges of one query row (see wmk.h).
__device__ __forceinline__ void row_ranges(const AttnCall& c, int32_t row, int32_t& lo0, int32_t& hi0, int32_t& lo1,
                                           int32_t& hi1) {
    lo1 = 0; hi1 = 0;
    if (!c.moba.enabled || row >= c.q_tokens) { lo0 = 0; hi0 = c.kv_total; return; }
    const int32_t L = c.moba.part_len, cl = c.moba.chunk_len;
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

// Element offset of key j (head `head`) inside its span, and the span index.
__device__ __forceinline__ int span_of(const KvSpans& kv, int32_t j, int32_t& start) {
    int s = 0;
    start = 0;
#pragma unroll
    for (int x = 0; x < kMaxSeg - 1; ++x)
        if (x < kv.n - 1 && j >= kv.end[x]) { s = x + 1; start = kv.end[x]; }
    return s;
}

template <int D>
struct TileRegs {
    u32x4 k[Cfg<D>::KLD];
    u32x4 v[4];
};

// Per-lane byte offsets of this thread's K and V chunks inside a tile, relative
// to the tile's first key row; constant over the key loop.
template <int D>
struct LaneOffsets {
    uint32_t k[Cfg<D>::KLD];
    uint32_t v[4];
};

template <int D>
__device__ __forceinline__ LaneOffsets<D> lane_offsets(int32_t heads, int32_t head) {
    using C = Cfg<D>;
    const int tid = threadIdx.x;
    const uint32_t row_bytes = (uint32_t)heads * D * 2, head_bytes = (uint32_t)head * D * 2;
    LaneOffsets<D> o;
#pragma unroll
    for (int i = 0; i < C::KLD; ++i)
        o.k[i] = (uint32_t)(tid / C::KCH + i * (NT / C::KCH)) * row_bytes + head_bytes + (tid % C::KCH) * 16;
    const int ch = (tid / 16) % C::KCH, qd = tid % 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) o.v[i] = (uint32_t)(qd * 4 + i) * row_bytes + head_bytes + ch * 16;
    return o;
}

// Global -> registers for key tile `tile`.  Common case: the whole tile lies in
// one span, so every load is a uniform base plus this lane's constant offset.
// A tile that crosses a span end or the last key takes the per-lane path
// (span lookup, zeros past the last key).
template <int D>
__device__ __forceinline__ void load_tile(const AttnCall& c, int32_t head, int32_t tile, const LaneOffsets<D>& lo,
                                          TileRegs<D>& r) {
    using C = Cfg<D>;
    const int tid = threadIdx.x;
    const int64_t row_bytes = (int64_t)c.heads * D * 2;
    const int32_t j0 = tile * BK;
    int32_t s0start;
    const int s0 = span_of(c.kv, j0, s0start);
    if (j0 + BK <= c.kv.end[s0]) {
        const char* kb = (const char*)c.kv.k[s0] + (int64_t)(j0 - s0start) * row_bytes;
        const char* vb = (const char*)c.kv.v[s0] + (int64_t)(j0 - s0start) * row_bytes;
#pragma unroll
        for (int i = 0; i < C::KLD; ++i) r.k[i] = *(const u32x4*)(kb + lo.k[i]);
        if (tid < C::VIT) {
#pragma unroll
            for (int i = 0; i < 4; ++i) r.v[i] = *(const u32x4*)(vb + lo.v[i]);
        }
        return;
    }
    const int64_t stride = (int64_t)c.heads * D;
    {
        const int ch = tid % C::KCH;
#pragma unroll
        for (int i = 0; i < C::KLD; ++i) {
            const int32_t j = j0 + tid / C::KCH + i * (NT / C::KCH);
            int32_t st;
            const int s = span_of(c.kv, j, st);
            const __bf16* base = (const __bf16*)c.kv.k[s];
            r.k[i] = u32x4{0u, 0u, 0u, 0u};
            if (j < c.kv_total) r.k[i] = *(const u32x4*)(base + (int64_t)(j - st) * stride + (int64_t)head * D + ch * 8);
        }
    }
    if (tid < C::VIT) {
        const int ch = tid / 16, qd = tid % 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int32_t j = j0 + qd * 4 + i;
            int32_t st;
            const int s = span_of(c.kv, j, st);
            const __bf16* base = (const __bf16*)c.kv.v[s];
            r.v[i] = u32x4{0u, 0u, 0u, 0u};
            if (j < c.kv_total) r.v[i] = *(const u32x4*)(base + (int64_t)(j - st) * stride + (int64_t)head * D + ch * 8);
        }
    }
}

// Position of key quad qd inside a V^T row: within each group of 16 keys the
// quads are stored in the order 0, 2, 1, 3, so that lanes 0-31 of the PV
// operand read keys {0-3, 8-11} and lanes 32-63 keys {4-7, 12-15} as one
// contiguous 16-byte vector -- the key order of the S^T accumulator rows.
__device__ __forceinline__ int vt_pos(int qd) {
    return (qd >> 2) * 16 + (((qd & 1) << 1) | ((qd >> 1) & 1)) * 4;
}

template <int D>
__device__ __forceinline__ void store_tile(__bf16* buf, const TileRegs<D>& r) {
    using C = Cfg<D>;
    const int tid = threadIdx.x;
    __bf16* Kl = buf;
    __bf16* Vt = buf + C::KE;
    {
        const int ch = tid % C::KCH;
#pragma unroll
        for (int i = 0; i < C::KLD; ++i) {
            const int row = tid / C::KCH + i * (NT / C::KCH);
            *(u32x4*)(Kl + row * C::KS + ch * 8) = r.k[i];
        }
    }
    if (tid < C::VIT) {
        const int ch = tid / 16, qd = tid % 16;
        const int pos = vt_pos(qd);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            // element e of keys 0..3: low (e even) or high (e odd) half of dword e/2
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            const int w = e >> 1;
            const uint32_t lo01 = __builtin_amdgcn_perm(r.v[1][w], r.v[0][w], sel);
            const uint32_t lo23 = __builtin_amdgcn_perm(r.v[3][w], r.v[2][w], sel);
            *(u32x2*)(Vt + (ch * 8 + e) * C::VS + pos) = u32x2{lo01, lo23};
        }
    }
}

__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workspace of the split tail: per split unit a counter, then per piece the
// unnormalized O (BQ x D fp32) and per-row (max, sum).
template <int D>
struct SplitWs {
    static constexpr size_t kO = (size_t)BQ * D;
    static __device__ __forceinline__ int* counters(void* ws) { return (int*)ws; }
    static __device__ __forceinline__ float* piece(void* ws, int32_t n_units, int32_t idx) {
        const size_t head = ((size_t)n_units * sizeof(int) + 255) & ~(size_t)255;
        return (float*)((char*)ws + head) + (size_t)idx * (kO + 2 * BQ);
    }
};

template <int D>
__global__ __launch_bounds__(NT, 2) void attn_bf16_kernel(Params prm) {
    using C = Cfg<D>;
    const AttnCall& c = prm.c;
    const AttnPlan& p = prm.p;
    __shared__ __attribute__((aligned(16))) __bf16 lds[2 * C::BUF];
    __shared__ int s_last;

    // ---- which unit (head, q-tile) and which key-tile range this workgroup runs
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
        const int32_t pb = b - full_units;
        u = full_units + pb / p.splits;
        piece = pb % p.splits;
    }
    int32_t head, qt;
    if (p.n_groups > 0) {  // longest-first order of q-tiles, all heads of a q-tile together
        const int32_t k = u / c.heads;
        head = u % c.heads;
        int32_t acc = 0;
        qt = 0;
        for (int g = 0; g < p.n_groups; ++g) {
            if (k >= acc && k < acc + p.grp_count[g]) qt = p.grp_start[g] + (k - acc);
            acc += p.grp_count[g];
        }
    } else {
        head = u / p.n_qtiles;
        qt = u % p.n_qtiles;
    }
    const int32_t r0 = qt * BQ, r1 = min(r0 + BQ, c.q_tokens);
    const TileRanges tr = tile_ranges(c, r0, r1);
    int32_t it0 = 0, it1 = tr.total;
    if (piece >= 0) {
        it0 = (int32_t)((int64_t)tr.total * piece / p.splits);
        it1 = (int32_t)((int64_t)tr.total * (piece + 1) / p.splits);
    }

    // ---- per-lane query row and its allowed key ranges
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, h = lane >> 5;
    const int32_t row = r0 + wave * 32 + l32;
    const bool row_ok = row < c.q_tokens;
    const bool wave_has_rows = (r0 + wave * 32) < c.q_tokens;
    int32_t lo0, hi0, lo1, hi1;
    row_ranges(c, row, lo0, hi0, lo1, hi1);
    const int64_t stride = (int64_t)c.heads * D;

    // Q^T fragments (B operand): lane owns query l32, dims ds*16 + h*8 .. +7
    bf16x8 qf[C::DS];
    {
        const __bf16* qp = (const __bf16*)c.q + (int64_t)row * stride + (int64_t)head * D + h * 8;
#pragma unroll
        for (int ds = 0; ds < C::DS; ++ds) {
            u32x4 raw = row_ok ? *(const u32x4*)(qp + ds * 16) : u32x4{0u, 0u, 0u, 0u};
            qf[ds] = __builtin_bit_cast(bf16x8, raw);
        }
    }

    f32x16 o[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) o[db] = f32x16{};
    float m_ref = -INFINITY, l_run = 0.0f;
    const float cs = c.scale * kLog2e;

    const LaneOffsets<D> loffs = lane_offsets<D>(c.heads, head);
    TileRegs<D> regs;
    if (it0 < it1) {
        load_tile<D>(c, head, tile_at(tr, it0), loffs, regs);
        store_tile<D>(lds, regs);
    }
    __syncthreads();

    for (int32_t it = it0; it < it1; ++it) {
        const int stage = (it - it0) & 1;
        const bool more = it + 1 < it1;
        if (more) load_tile<D>(c, head, tile_at(tr, it + 1), loffs, regs);

        if (wave_has_rows) {
            const __bf16* Kl = lds + stage * C::BUF;
            const __bf16* Vt = Kl + C::KE;
            const int32_t j0 = tile_at(tr, it) * BK;

            // S^T = K Q^T for two blocks of 32 keys
            f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
            for (int ds = 0; ds < C::DS; ++ds) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16x8 a = *(const bf16x8*)(Kl + (kb * 32 + l32) * C::KS + ds * 16 + h * 8);
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ds], s[kb], 0, 0, 0);
                }
            }

            // mask: skipped when every row of the wave allows the whole tile
            const uint32_t lane_full = (row_ok ? 0u : 1u) | ((uint32_t)(lo0 <= j0) & (uint32_t)(j0 + BK <= hi0)) |
                                       ((uint32_t)(lo1 <= j0) & (uint32_t)(j0 + BK <= hi1));
            if (__builtin_amdgcn_ballot_w64(lane_full == 0u) != 0) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int32_t j = j0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                        const uint32_t ok = in_range(j, lo0, hi0) | in_range(j, lo1, hi1);
                        s[kb][r] = ok ? s[kb][r] : -INFINITY;
                    }
            }

            // online softmax (log2 domain).  m_ref is the reference the
            // exponentials use; it moves (and O, l are rescaled) only when a
            // row's tile max exceeds it by more than kTau, so p <= 2^kTau.
            float mx = s[0][0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
            const float mt = pair_max(mx) * cs;
            if (__builtin_amdgcn_ballot_w64(mt > m_ref + kTau) != 0) {
                const float m_new = fmaxf(m_ref, mt);
                const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
#pragma unroll
                for (int db = 0; db < C::DB; ++db) o[db] *= alpha;
                l_run *= alpha;
                m_ref = m_new;
            }
            const float m_use = (m_ref == -INFINITY) ? 0.0f : m_ref;

            bf16x8 pf[2][2];
            float lsum = 0.0f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    f32x8 e;
#pragma unroll
                    for (int r = 0; r < 8; ++r) e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * t + r], cs, -m_use));
                    pf[kb][t] = __builtin_convertvector(e, bf16x8);
                    // row sum of the bf16 weights the PV product uses
                    const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
                    for (int q2 = 0; q2 < 4; ++q2) {
                        const bf16x2 pp = {pf[kb][t][2 * q2], pf[kb][t][2 * q2 + 1]};
                        lsum = __builtin_amdgcn_fdot2_f32_bf16(pp, one2, lsum, false);
                    }
                }
            }
            l_run += lsum;

            // O^T += V^T P^T
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const bf16x8 a =
                            *(const bf16x8*)(Vt + (db * 32 + l32) * C::VS + (2 * kb + t) * 16 + h * 8);
                        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kb][t], o[db], 0, 0, 0);
                    }
                }
            }
        }

        if (more) store_tile<D>(lds + (stage ^ 1) * C::BUF, regs);
        __syncthreads();
    }

    const float l_tot = pair_sum(l_run);
    __bf16* op = (__bf16*)c.out + (int64_t)row * stride + (int64_t)head * D;

    if (piece < 0) {
        if (row_ok) {
            const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    f32x4 v4 = {o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
                                o[db][4 * g + 3] * inv};
                    *(bf16x4*)(op + db * 32 + 8 * g + 4 * h) = __builtin_convertvector(v4, bf16x4);
                }
        }
        return;
    }

    // ---- split tail: publish this piece, the last piece of the unit merges
    const int32_t su = u - full_units;
    {
        float* w = SplitWs<D>::piece(p.ws, p.split_units, su * p.splits + piece);
        const int rl = wave * 32 + l32;  // row within the tile
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *(f32x4*)(w + (size_t)rl * D + db * 32 + 8 * g + 4 * h) =
                    f32x4{o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
        if (h == 0) {
            w[SplitWs<D>::kO + 2 * rl] = m_ref;
            w[SplitWs<D>::kO + 2 * rl + 1] = l_tot;
        }
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const int prev = atomicAdd(SplitWs<D>::counters(p.ws) + su, 1);
        s_last = (prev == p.splits - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    // merge: thread t handles row t/2, half (t%2) of the dims
    {
        const int rl = threadIdx.x >> 1, half = threadIdx.x & 1;
        const int32_t mrow = r0 + rl;
        float mmax = -INFINITY;
        for (int q = 0; q < p.splits; ++q) {
            const float* w = SplitWs<D>::piece(p.ws, p.split_units, su * p.splits + q);
            mmax = fmaxf(mmax, __builtin_nontemporal_load(w + SplitWs<D>::kO + 2 * rl));
        }
        const float mref = (mmax == -INFINITY) ? 0.0f : mmax;
        float acc[D / 2];
#pragma unroll
        for (int d = 0; d < D / 2; ++d) acc[d] = 0.0f;
        float lt = 0.0f;
        for (int q = 0; q < p.splits; ++q) {
            const float* w = SplitWs<D>::piece(p.ws, p.split_units, su * p.splits + q);
            const float wq = __builtin_amdgcn_exp2f(__builtin_nontemporal_load(w + SplitWs<D>::kO + 2 * rl) - mref);
            lt += wq * __builtin_nontemporal_load(w + SplitWs<D>::kO + 2 * rl + 1);
            const float* src = w + (size_t)rl * D + half * (D / 2);
#pragma unroll
            for (int d = 0; d < D / 2; d += 4) {
                const f32x4 x = __builtin_nontemporal_load((const f32x4*)(src + d));
                acc[d] += wq * x[0];
                acc[d + 1] += wq * x[1];
                acc[d + 2] += wq * x[2];
                acc[d + 3] += wq * x[3];
            }
        }
        if (mrow < c.q_tokens) {
            const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
            __bf16* dst = (__bf16*)c.out + (int64_t)mrow * stride + (int64_t)head * D + half * (D / 2);
#pragma unroll
            for (int d = 0; d < D / 2; d += 4) {
                f32x4 v4 = {acc[d] * inv, acc[d + 1] * inv, acc[d + 2] * inv, acc[d + 3] * inv};
                *(bf16x4*)(dst + d) = __builtin_convertvector(v4, bf16x4);
            }
        }
        if (threadIdx.x == 0) SplitWs<D>::counters(p.ws)[su] = 0;  // leave the counter zeroed
    }
}

__global__ void zero_ints(int* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

}  // namespace

size_t attn_bf16_split_ws_bytes(int head_dim, int32_t split_units, int32_t splits) {
    if (split_units <= 0 || splits <= 0) return 0;
    const size_t head = ((size_t)split_units * sizeof(int) + 255) & ~(size_t)255;
    return head + (size_t)split_units * splits * ((size_t)BQ * head_dim + 2 * BQ) * sizeof(float);
}

int attn_bf16_blocks_per_cu(int head_dim) {
    int n = 0;
    hipError_t e;
    if (head_dim == 64)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_bf16_kernel<64>, NT, 0);
    else
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_bf16_kernel<128>, NT, 0);
    return (e == hipSuccess && n > 0) ? n : 1;
}

hipError_t launch_attn_bf16(const AttnCall& c, const AttnPlan& plan, hipStream_t s) {
    Params prm;
    prm.c = c;
    prm.p = plan;
    const int32_t blocks = plan.n_units - plan.split_units + plan.split_units * plan.splits;
    if (blocks <= 0) return hipSuccess;
    if (plan.split_units > 0) {
        hipLaunchKernelGGL(zero_ints, dim3((plan.split_units + 255) / 256), dim3(256), 0, s, (int*)plan.ws,
                           plan.split_units);
    }
    if (c.head_dim == 64)
        hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(blocks), dim3(NT), 0, s, prm);
    else if (c.head_dim == 128)
        hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(blocks), dim3(NT), 0, s, prm);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace wmk
