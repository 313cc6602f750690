// The C ABI of include/wmk.h: argument checks, host-side cache bookkeeping and
// launch planning.  Bookkeeping is a per-layer frame counter on the host; it
// decides slots and resident prefixes without ever reading the device, so a
// generation loop needs no host/device synchronization (the per-layer host
// syncs that the LingBot-World 2.0 speed-up write-up removes in its
// step-ablation table, "Host syncs" row, do not arise).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "attn_tiles.h"
#include "wmk.h"
#include "wmk_internal.h"

struct wmk_cache {
    wmk_cache_desc d;
    char* k;
    char* v;
    size_t frame_bytes;  // one latent frame of one layer: tpf * heads * head_dim * elem
    size_t layer_bytes;  // (S + W) frames
    std::vector<int64_t> frames;  // per layer: frames appended so far
};

namespace {

thread_local std::string g_err;

wmk_status fail(wmk_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

wmk_status ok() {
    g_err.clear();
    return WMK_OK;
}

size_t elem_size(wmk_dtype t) { return t == WMK_F32 ? 4 : 2; }
bool dtype_ok(int t) { return t == WMK_F32 || t == WMK_BF16; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Test hook: WMK_FAULT_INJECT=1 makes every launch report a refused launch
// before touching the device, so the no-state-change-on-error rule can be
// checked on a machine without a GPU.
bool fault_injected() {
    const char* e = getenv("WMK_FAULT_INJECT");
    return e != nullptr && e[0] == '1';
}

// Test hook: WMK_DRY_RUN=<path> checks and plans every call but launches
// nothing; each planned launch is appended to <path> as one line, so host
// bookkeeping and planning can be checked on a machine without a GPU.
const char* dry_run_path() {
    const char* e = getenv("WMK_DRY_RUN");
    return (e != nullptr && e[0] != '\0') ? e : nullptr;
}

void dry_log(const char* fmt, ...) {
    const char* path = dry_run_path();
    if (path == nullptr) return;
    FILE* f = fopen(path, "a");
    if (f == nullptr) return;
    va_list ap;
    va_start(ap, fmt);
    vfprintf(f, fmt, ap);
    va_end(ap);
    fclose(f);
}

wmk_status check_desc(const wmk_cache_desc* d) {
    if (d == nullptr) return fail(WMK_ERR_NULL, "cache descriptor is NULL");
    if (!dtype_ok(d->dtype)) return fail(WMK_ERR_DTYPE, "dtype %d is not WMK_F32 or WMK_BF16", (int)d->dtype);
    if (d->num_layers < 1 || d->num_heads < 1 || d->tokens_per_frame < 1 || d->sink_frames < 0 ||
        d->window_frames < 1 || d->chunk_frames < 1)
        return fail(WMK_ERR_SHAPE, "cache descriptor has a non-positive field (layers %d heads %d tpf %d S %d W %d cf %d)",
                    d->num_layers, d->num_heads, d->tokens_per_frame, d->sink_frames, d->window_frames,
                    d->chunk_frames);
    if (d->head_dim != 64 && d->head_dim != 128)
        return fail(WMK_ERR_SHAPE, "head_dim %d is not 64 or 128", d->head_dim);
    if (d->num_heads > wmk::kMaxHeads) return fail(WMK_ERR_SHAPE, "num_heads %d > %d", d->num_heads, wmk::kMaxHeads);
    const int64_t slots = (int64_t)d->sink_frames + d->window_frames;
    if (slots * d->tokens_per_frame > INT32_MAX)
        return fail(WMK_ERR_SHAPE, "(S + W) * tokens_per_frame exceeds 2^31 - 1 tokens");
    return WMK_OK;
}

wmk_status check_head(const wmk_head_desc* hd) {
    if (hd == nullptr) return fail(WMK_ERR_NULL, "head descriptor is NULL");
    if (!dtype_ok(hd->dtype)) return fail(WMK_ERR_DTYPE, "dtype %d is not WMK_F32 or WMK_BF16", (int)hd->dtype);
    if (hd->num_heads < 1) return fail(WMK_ERR_SHAPE, "num_heads %d < 1", hd->num_heads);
    if (hd->num_heads > wmk::kMaxHeads) return fail(WMK_ERR_SHAPE, "num_heads %d > %d", hd->num_heads, wmk::kMaxHeads);
    if (hd->head_dim != 64 && hd->head_dim != 128)
        return fail(WMK_ERR_SHAPE, "head_dim %d is not 64 or 128", hd->head_dim);
    return WMK_OK;
}

wmk_status check_scale(float scale) {
    if (!(scale > 0.0f) || !isfinite(scale)) return fail(WMK_ERR_RANGE, "scale %g is not finite and > 0", scale);
    return WMK_OK;
}

// Slot of frame f (first S frames: their own slot; later frames: ring of W).
int64_t slot_of(const wmk_cache_desc& d, int64_t f) {
    return f < d.sink_frames ? f : d.sink_frames + (f - d.sink_frames) % d.window_frames;
}

// Filled slots after F frames: they are always the prefix [0, valid).
int64_t valid_of(const wmk_cache_desc& d, int64_t F) {
    return std::min<int64_t>(F, d.sink_frames) + std::min<int64_t>(std::max<int64_t>(F - d.sink_frames, 0),
                                                                    d.window_frames);
}

// ---- per-device facts used by the planner
struct DeviceInfo {
    int cus = 0;
    int bpc64 = 0, bpc128 = 0, bpc128_short = 0;  // resident workgroups per CU of the bf16 kernels
    int slots(int head_dim, int waves) const {
        return cus * (waves == wmk::kWavesShort ? bpc128_short : head_dim == 64 ? bpc64 : bpc128);
    }
};
std::mutex g_dev_mu;
std::vector<DeviceInfo> g_dev;

DeviceInfo device_info() {
    if (dry_run_path() != nullptr) {  // no device: an MI355X-like 256 CUs, one 8-wave or two 4-wave workgroups each
        DeviceInfo di;
        di.cus = 256;
        di.bpc64 = 1;
        di.bpc128 = 1;
        di.bpc128_short = 2;
        return di;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if ((int)g_dev.size() <= dev) g_dev.resize(dev + 1);
    DeviceInfo& di = g_dev[dev];
    if (di.cus == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        di.cus = cus;
        di.bpc64 = wmk::attn_bf16_blocks_per_cu(64, wmk::kWavesLong);
        di.bpc128 = wmk::attn_bf16_blocks_per_cu(128, wmk::kWavesLong);
        di.bpc128_short = wmk::attn_bf16_blocks_per_cu(128, wmk::kWavesShort);
    }
    return di;
}

constexpr int kBK = 64;
constexpr int kMinTilesPerPiece = 8;

// Split the last, partly filled round of units over the whole GPU when the
// caller gave enough workspace.  Returns the workspace bytes that split needs
// (0 when the call gets no split whatever the workspace).
// kv_tiles: 64-key tiles of the whole key range, a bound on any unit's visits
// (the kernel splits with 32-bit products visits x piece).
size_t plan_split(wmk::AttnPlan& p, int head_dim, int32_t tiles_per_unit, int32_t kv_tiles, void* ws,
                  size_t ws_bytes) {
    p.split_units = 0;
    p.splits = 1;
    p.ws = nullptr;
    if (tiles_per_unit < 2 * kMinTilesPerPiece) return 0;
    const int slots = device_info().slots(head_dim, p.waves);
    if (slots <= 0) return 0;
    const int32_t rounds = p.n_units / slots, tail = p.n_units % slots;
    if (rounds < 1 || tail == 0) return 0;
    int32_t splits = std::min<int32_t>(slots / tail, tiles_per_unit / kMinTilesPerPiece);
    splits = std::min<int32_t>(splits, INT32_MAX / std::max(kv_tiles, 1));
    if (splits < 2) return 0;
    const size_t need = wmk::attn_bf16_split_ws_bytes(head_dim, p.waves, tail, splits);
    // (the pieces store 16-byte vectors: a misaligned workspace is not used)
    if (ws == nullptr || ((uintptr_t)ws & 15) != 0 || need > ws_bytes) return need;
    p.split_units = tail;
    p.splits = splits;
    p.ws = ws;
    return need;
}

// Number of 64-wide tiles the union of the half-open intervals iv covers
// (each rounded out to whole tiles; the kernels' merge rule).
int32_t tiles_of_union(std::vector<std::pair<int32_t, int32_t>> iv) {
    for (auto& x : iv) x = {x.first / kBK, (x.second + kBK - 1) / kBK};
    std::sort(iv.begin(), iv.end());
    int32_t total = 0, cur_b = -1, cur_e = -1;
    for (auto& x : iv) {
        if (x.second <= x.first) continue;
        if (cur_e >= 0 && x.first <= cur_e) {
            cur_e = std::max(cur_e, x.second);
        } else {
            if (cur_e >= 0) total += cur_e - cur_b;
            cur_b = x.first;
            cur_e = x.second;
        }
    }
    if (cur_e >= 0) total += cur_e - cur_b;
    return total;
}

// Key tiles a q-tile of the MoBA sequence visits (same union rule as the kernel).
int32_t moba_rows_cost(const wmk::MaskShape& m, int32_t q_tokens, int32_t r0, int32_t r1) {
    r1 = std::min(r1, q_tokens);
    const int32_t L = m.part_len, cl = m.chunk_len;
    std::vector<std::pair<int32_t, int32_t>> iv;
    for (int32_t part = r0 / L; part <= (r1 - 1) / L && part < m.parts; ++part) {
        const int32_t fa = std::max(r0, part * L) - part * L, fb = std::min(r1, (part + 1) * L) - part * L - 1;
        const int32_t ka = fa / cl, kb = fb / cl;
        if (part == 0) {
            iv.push_back({0, std::min((kb + 1) * cl, L)});
        } else if (part == 1) {
            if (kb > 0) iv.push_back({0, kb * cl});
            iv.push_back({L + ka * cl, L + std::min((kb + 1) * cl, L)});
        } else {
            iv.push_back({2 * L, 3 * L});
        }
    }
    return tiles_of_union(iv);
}

int32_t moba_qtile_cost(const wmk::MaskShape& m, int32_t q_tokens, int32_t qt) {
    const int32_t bq = wmk::attn_bf16_block_q(wmk::kWavesLong);  // MoBA runs the 8-wave kernel
    return moba_rows_cost(m, q_tokens, qt * bq, qt * bq + bq);
}

// Query tiles of 64 rows a block of keys [c0, c1) of the MoBA sequence is
// attended by (the dK/dV kernel's walk: the same union rule, transposed --
// clean key of chunk c: clean rows of chunks >= c and noisy rows of chunks > c;
// noisy key of chunk c: noisy rows of chunk c; block key: block rows).
int32_t moba_ktile_cost(const wmk::MaskShape& m, int32_t n, int32_t c0, int32_t c1) {
    const int32_t L = m.part_len, cl = m.chunk_len;
    c1 = std::min(c1, n);
    std::vector<std::pair<int32_t, int32_t>> iv;
    if (c1 <= c0) return 0;
    const int32_t pa = c0 / L, pb = (c1 - 1) / L;
    if (pa <= 0 && 0 <= pb) {
        const int32_t ca = c0 / cl;
        iv.push_back({ca * cl, L});
        if (m.parts > 1) iv.push_back({std::min(L + (ca + 1) * cl, 2 * L), 2 * L});
    }
    if (pa <= 1 && 1 <= pb) {
        const int32_t fa = std::max(c0, L) - L, fb = std::min(c1, 2 * L) - L - 1;
        iv.push_back({L + (fa / cl) * cl, L + std::min((fb / cl + 1) * cl, L)});
    }
    if (pa <= 2 && 2 <= pb) iv.push_back({2 * L, 3 * L});
    return tiles_of_union(iv);
}

// Longest-first launch order: runs of consecutive tiles with equal cost,
// sorted by decreasing cost (stable).  Returns the number of runs, or 0 (the
// natural order) when there are more runs than the kernels' tables hold.
int32_t plan_groups(const std::vector<int32_t>& cost, int32_t* grp_start, int32_t* grp_count) {
    struct Run { int32_t start, count, cost; };
    std::vector<Run> runs;
    for (int32_t t = 0; t < (int32_t)cost.size(); ++t) {
        if (!runs.empty() && runs.back().cost == cost[t] && runs.back().start + runs.back().count == t)
            runs.back().count++;
        else
            runs.push_back({t, 1, cost[t]});
    }
    if ((int)runs.size() > wmk::kMaxGroups) return 0;
    std::stable_sort(runs.begin(), runs.end(), [](const Run& a, const Run& b) { return a.cost > b.cost; });
    for (size_t i = 0; i < runs.size(); ++i) {
        grp_start[i] = runs[i].start;
        grp_count[i] = runs[i].count;
    }
    return (int32_t)runs.size();
}

// Longest-first launch order of the MoBA forward's q-tiles.
void plan_moba_groups(wmk::AttnPlan& p, const wmk::MaskShape& m, int32_t q_tokens) {
    std::vector<int32_t> cost(p.n_qtiles);
    for (int32_t qt = 0; qt < p.n_qtiles; ++qt) cost[qt] = moba_qtile_cost(m, q_tokens, qt);
    p.n_groups = plan_groups(cost, p.grp_start, p.grp_count);
}

// FP8 QK^T buffers carved from the caller's workspace (see qk8_layout).
struct Qk8Bufs {
    uint8_t* k8;
    float* k8_scale;
    uint8_t* q8;
    float* q8_scale;
};

// strict_ws: the workspace is the library's own fixed scratch; a split that
// does not fit is an error rather than a reason to run unsplit, so the call
// plans exactly as wmk_chunk_attention with an ample workspace would.
wmk_status run_attention(const wmk::AttnCall& call, wmk_dtype dtype, void* ws, size_t ws_bytes,
                         hipStream_t stream, const Qk8Bufs* qk8 = nullptr, bool strict_ws = false) {
    if (fault_injected()) return fail(WMK_ERR_HIP, "launch refused (WMK_FAULT_INJECT)");
    hipError_t e;
    if (dtype == WMK_F32) {
        if (dry_run_path() != nullptr) {
            dry_log("attn dtype=f32 q=%d heads=%d d=%d kv=%d mask=%d\n", call.q_tokens, call.heads, call.head_dim,
                    call.kv_total, call.mask.mode);
            return ok();
        }
        e = wmk::launch_attn_f32(call, stream);
    } else {
        wmk::AttnPlan p;
        memset(&p, 0, sizeof p);
        // every q-tile of a chunk-attention or cross-mask call visits the same
        // number of key tiles: the whole key range, or (cross mask) the
        // environment prompt plus its chunks' local prompts
        const int32_t kv_tiles = (int32_t)(((int64_t)call.kv_total + kBK - 1) / kBK);
        int32_t tiles = kv_tiles;
        if (call.mask.mode == wmk::kMaskCross)
            tiles = (call.mask.env_len + kBK - 1) / kBK + (call.mask.chunk_len + kBK - 1) / kBK;
        p.waves = wmk::kWavesLong;
        if (call.mask.mode != wmk::kMaskMoba && call.head_dim == 128 && qk8 == nullptr &&
            tiles <= wmk::kShortUnitTiles)
            p.waves = wmk::kWavesShort;
        const int32_t bq = wmk::attn_bf16_block_q(p.waves);
        p.n_qtiles = (call.q_tokens + bq - 1) / bq;
        p.n_units = p.n_qtiles * call.heads;
        p.splits = 1;
        if (call.mask.mode == wmk::kMaskMoba) {
            plan_moba_groups(p, call.mask, call.q_tokens);
            p.xcd_remap = 0;
        } else {
            p.xcd_remap = 1;
            const size_t need = plan_split(p, call.head_dim, tiles, kv_tiles, ws, ws_bytes);
            if (strict_ws && need > ws_bytes)
                return fail(WMK_ERR_CAPACITY, "the split tail of this call needs %zu bytes of scratch; the library "
                            "holds %zu", need, ws_bytes);
        }
        p.heads_div = wmk::make_fastdiv((uint32_t)std::max(call.heads, 1));
        p.qtiles_div = wmk::make_fastdiv((uint32_t)std::max(p.n_qtiles, 1));
        p.splits_div = wmk::make_fastdiv((uint32_t)std::max(p.splits, 1));
        if (qk8 != nullptr) {
            p.k8 = qk8->k8;
            p.k8_scale = qk8->k8_scale;
            p.q8 = qk8->q8;
            p.q8_scale = qk8->q8_scale;
        }
        if (dry_run_path() != nullptr) {
            dry_log("attn dtype=bf16 q=%d heads=%d d=%d kv=%d mask=%d bq=%d units=%d qtiles=%d groups=%d "
                    "split_units=%d splits=%d qk8=%d\n", call.q_tokens, call.heads, call.head_dim, call.kv_total,
                    call.mask.mode, bq, p.n_units, p.n_qtiles, p.n_groups, p.split_units, p.splits,
                    qk8 != nullptr ? 1 : 0);
            for (int g = 0; g < p.n_groups; ++g) dry_log("group %d %d\n", p.grp_start[g], p.grp_count[g]);
            for (int x = 0; x < call.kv.n; ++x)
                dry_log("span %d %d %llx %llx\n", x, call.kv.end[x], (unsigned long long)(uintptr_t)call.kv.k[x],
                        (unsigned long long)(uintptr_t)call.kv.v[x]);
            // the key tiles each q-tile's workgroup walks, from the kernels' own planner
            for (int32_t qt = 0; qt < p.n_qtiles; ++qt) {
                const int32_t r0 = qt * bq, r1 = std::min(r0 + bq, call.q_tokens);
                const wmk::tiles::TileRanges tr = wmk::tiles::tile_ranges(call, r0, r1);
                dry_log("tiles %d %d %d %d %d %d %d %d %d %d %d\n", r0, r1, tr.b0, tr.e0, tr.b1, tr.e1, tr.b2, tr.e2,
                        tr.b3, tr.e3, tr.total);
            }
            return ok();
        }
        if (qk8 != nullptr) {
            // quantize Q (blocks of 32 rows) and the key sequence (tiles of 64 keys) first
            const void* qsrc[1] = {call.q};
            const int32_t qend[1] = {call.q_tokens};
            e = wmk::launch_quant_e4m3(qsrc, qend, 1, call.q_tokens, call.heads, call.head_dim, 32, qk8->q8,
                                       qk8->q8_scale, stream);
            if (e == hipSuccess && call.kv_total > 0)
                e = wmk::launch_quant_e4m3(call.kv.k, call.kv.end, call.kv.n, call.kv_total, call.heads,
                                           call.head_dim, 64, qk8->k8, qk8->k8_scale, stream);
            if (e != hipSuccess) return fail(WMK_ERR_HIP, "quantization launch failed: %s", hipGetErrorString(e));
        }
        e = wmk::launch_attn_bf16(call, p, stream);
    }
    if (e != hipSuccess) return fail(WMK_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

const int64_t kNoFrame = -1;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of the FP8 QK^T path, in order: K codes (one 8 KB block per 64-key
// tile and head), their scales, Q codes (one 4 KB block per 32 rows and head),
// their scales -- each 256-byte aligned -- then the split-tail scratch.
size_t qk8_bytes(int32_t heads, int32_t q_tokens, int64_t kv_tokens, Qk8Bufs* b, char* base) {
    const int64_t kt = (kv_tokens + 63) / 64, qb = ((int64_t)q_tokens + 31) / 32;
    size_t off = 0;
    const size_t k8 = off;
    off += align256((size_t)kt * heads * 64 * 128);
    const size_t ks = off;
    off += align256((size_t)kt * heads * 4);
    const size_t q8 = off;
    off += align256((size_t)qb * heads * 32 * 128);
    const size_t qs = off;
    off += align256((size_t)qb * heads * 4);
    if (b != nullptr) {
        b->k8 = (uint8_t*)(base + k8);
        b->k8_scale = (float*)(base + ks);
        b->q8 = (uint8_t*)(base + q8);
        b->q8_scale = (float*)(base + qs);
    }
    return off;
}

// Chunk attention over the resident frames of `layer` (keep == NULL: all of
// them; else the n_keep listed frames) plus the caller's segments.  The cache
// part becomes one span per run of adjacent slots.  The plain paths visit the
// slots in slot order (softmax does not depend on the order of the keys, and
// the whole resident prefix is then one span); the FP8 path visits the
// resident frames in time order -- sinks, then recent frames, oldest first --
// because its 64-key scale blocks are cut along the key sequence, and in time
// order that sequence, and so every block, depends only on which frames are
// resident, not on where the ring has wrapped.
wmk_status chunk_attention_impl(const wmk_cache* c, int32_t layer, const int64_t* keep, int32_t n_keep,
                                const wmk_head_desc* hd, const void* q, int32_t q_tokens, const wmk_kv_segment* seg,
                                int32_t n_seg, void* out, float scale, void* workspace, size_t workspace_bytes,
                                hipStream_t stream, bool qk8 = false, bool strict_ws = false) {
    wmk_status s = check_head(hd);
    if (s != WMK_OK) return s;
    if (qk8 && hd->dtype != WMK_BF16) return fail(WMK_ERR_DTYPE, "FP8 QK^T takes bf16 inputs");
    if (qk8 && hd->head_dim != 128) return fail(WMK_ERR_SHAPE, "FP8 QK^T is built for head_dim 128");
    if (q == nullptr || out == nullptr) return fail(WMK_ERR_NULL, "q and out must not be NULL");
    if (n_seg < 0 || n_seg > wmk::kMaxCallerSeg)
        return fail(WMK_ERR_SHAPE, "n_seg %d outside [0, %d]", n_seg, wmk::kMaxCallerSeg);
    if (n_seg > 0 && seg == nullptr) return fail(WMK_ERR_NULL, "seg is NULL with n_seg %d", n_seg);
    if (q_tokens <= 0) return fail(WMK_ERR_SHAPE, "q_tokens %d <= 0", q_tokens);
    if ((s = check_scale(scale)) != WMK_OK) return s;
    if (!aligned16(q) || !aligned16(out)) return fail(WMK_ERR_ALIGN, "q/out must be 16-byte aligned");
    if (c != nullptr) {
        if (layer < 0 || layer >= c->d.num_layers)
            return fail(WMK_ERR_RANGE, "layer %d outside [0, %d)", layer, c->d.num_layers);
        if (c->d.num_heads != hd->num_heads || c->d.head_dim != hd->head_dim)
            return fail(WMK_ERR_SHAPE, "head descriptor (%d x %d) does not match the cache (%d x %d)",
                        hd->num_heads, hd->head_dim, c->d.num_heads, c->d.head_dim);
        if (c->d.dtype != hd->dtype) return fail(WMK_ERR_DTYPE, "dtype differs from the cache's");
    }
    wmk::AttnCall call;
    memset(&call, 0, sizeof call);
    int64_t total = 0;
    int n = 0;
    if (c != nullptr) {
        const wmk_cache_desc& d = c->d;
        const int32_t slots = d.sink_frames + d.window_frames;
        const int64_t F = c->frames[layer];
        std::vector<char> sel(slots, 0);
        if (keep == nullptr) {
            std::fill(sel.begin(), sel.begin() + valid_of(d, F), 1);
        } else {
            for (int32_t i = 0; i < n_keep; ++i) {
                const int64_t f = keep[i];
                const bool resident = f >= 0 && f < F && (f < d.sink_frames || f >= std::max<int64_t>(d.sink_frames, F - d.window_frames));
                if (!resident) return fail(WMK_ERR_RANGE, "frame %lld is not resident in layer %d", (long long)f, layer);
                const int64_t slot = f < d.sink_frames ? f : d.sink_frames + (f - d.sink_frames) % d.window_frames;
                if (sel[slot]) return fail(WMK_ERR_RANGE, "frame %lld listed twice", (long long)f);
                sel[slot] = 1;
            }
        }
        // the selected slots in visiting order
        std::vector<int32_t> order;
        if (qk8) {
            auto visit = [&](int64_t f) {
                if (sel[slot_of(d, f)]) order.push_back((int32_t)slot_of(d, f));
            };
            for (int64_t f = 0; f < std::min<int64_t>(F, d.sink_frames); ++f) visit(f);
            for (int64_t f = std::max<int64_t>(d.sink_frames, F - d.window_frames); f < F; ++f) visit(f);
        } else {
            for (int32_t a = 0; a < slots; ++a)
                if (sel[a]) order.push_back(a);
        }
        const size_t base = (size_t)layer * c->layer_bytes;
        for (size_t i = 0; i < order.size();) {
            size_t j = i + 1;
            while (j < order.size() && order[j] == order[j - 1] + 1) ++j;
            if (n + n_seg >= wmk::kMaxSeg)
                return fail(WMK_ERR_CAPACITY, "retained frames form more than %d runs of adjacent slots with %d segments",
                            wmk::kMaxSeg - n_seg, n_seg);
            call.kv.k[n] = c->k + base + (size_t)order[i] * c->frame_bytes;
            call.kv.v[n] = c->v + base + (size_t)order[i] * c->frame_bytes;
            total += (int64_t)(j - i) * d.tokens_per_frame;
            call.kv.end[n] = (int32_t)total;  // < 2^31: the cache size check bounds a layer's tokens
            ++n;
            i = j;
        }
    }
    for (int i = 0; i < n_seg; ++i) {
        if (seg[i].k == nullptr || seg[i].v == nullptr) return fail(WMK_ERR_NULL, "segment %d has a NULL k/v", i);
        if (seg[i].tokens <= 0) return fail(WMK_ERR_SHAPE, "segment %d has %d tokens", i, seg[i].tokens);
        if (!aligned16(seg[i].k) || !aligned16(seg[i].v))
            return fail(WMK_ERR_ALIGN, "segment %d k/v must be 16-byte aligned", i);
        total += seg[i].tokens;
        if (total > INT32_MAX) return fail(WMK_ERR_SHAPE, "more than 2^31 - 1 keys");
        call.kv.k[n] = seg[i].k;
        call.kv.v[n] = seg[i].v;
        call.kv.end[n] = (int32_t)total;
        ++n;
    }
    call.kv.n = n;
    call.q = q;
    call.out = out;
    call.q_tokens = q_tokens;
    call.heads = hd->num_heads;
    call.head_dim = hd->head_dim;
    call.kv_total = (int32_t)total;
    call.scale = scale;
    call.mask.mode = wmk::kMaskNone;
    if (!qk8) return run_attention(call, hd->dtype, workspace, workspace_bytes, stream, nullptr, strict_ws);
    Qk8Bufs bufs;
    const size_t need = qk8_bytes(hd->num_heads, q_tokens, total, &bufs, (char*)workspace);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(WMK_ERR_CAPACITY, "FP8 QK^T needs %zu bytes of workspace, got %zu", need, workspace_bytes);
    if (((uintptr_t)workspace & 255) != 0) return fail(WMK_ERR_ALIGN, "workspace must be 256-byte aligned");
    return run_attention(call, hd->dtype, (char*)workspace + need, workspace_bytes - need, stream, &bufs);
}

// Validate a MoBA call and fill its AttnCall (no workspace, no lse).
wmk_status moba_call(const wmk_moba_desc* m, const wmk_head_desc* hd, const void* q, const void* k, const void* v,
                     void* out, float scale, wmk::AttnCall& call) {
    if (m == nullptr) return fail(WMK_ERR_NULL, "MoBA descriptor is NULL");
    wmk_status s = check_head(hd);
    if (s != WMK_OK) return s;
    if (q == nullptr || k == nullptr || v == nullptr || out == nullptr)
        return fail(WMK_ERR_NULL, "q, k, v and out must not be NULL");
    if (m->tokens_per_frame < 1 || m->frames < 1 || m->chunk_frames < 1)
        return fail(WMK_ERR_SHAPE, "MoBA descriptor has a non-positive field");
    if (m->bidir_block != 0 && m->bidir_block != 1) return fail(WMK_ERR_SHAPE, "bidir_block %d not 0 or 1", m->bidir_block);
    const int64_t L = (int64_t)m->frames * m->tokens_per_frame;
    const int64_t total = (2 + m->bidir_block) * L;
    if (total > INT32_MAX) return fail(WMK_ERR_SHAPE, "sequence of %lld tokens exceeds 2^31 - 1", (long long)total);
    if ((s = check_scale(scale)) != WMK_OK) return s;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(WMK_ERR_ALIGN, "q/k/v/out must be 16-byte aligned");
    memset(&call, 0, sizeof call);
    call.kv.k[0] = k;
    call.kv.v[0] = v;
    call.kv.end[0] = (int32_t)total;
    call.kv.n = 1;
    call.q = q;
    call.out = out;
    call.q_tokens = (int32_t)total;
    call.heads = hd->num_heads;
    call.head_dim = hd->head_dim;
    call.kv_total = (int32_t)total;
    call.scale = scale;
    call.mask.mode = wmk::kMaskMoba;
    call.mask.part_len = (int32_t)L;
    call.mask.chunk_len = std::min(m->chunk_frames, m->frames) * m->tokens_per_frame;
    call.mask.parts = 2 + m->bidir_block;
    wmk::set_mask_divisors(call.mask);
    return WMK_OK;
}

}  // namespace

#pragma GCC visibility push(default)
extern "C" {

size_t wmk_cache_bytes(const wmk_cache_desc* d) {
    if (check_desc(d) != WMK_OK) return 0;
    return (size_t)d->num_layers * (size_t)(d->sink_frames + d->window_frames) * (size_t)d->tokens_per_frame *
           (size_t)d->num_heads * (size_t)d->head_dim * elem_size(d->dtype);
}

wmk_status wmk_cache_init(const wmk_cache_desc* d, void* k_dev, void* v_dev, size_t capacity_bytes,
                          wmk_cache** out) {
    wmk_status s = check_desc(d);
    if (s != WMK_OK) return s;
    if (k_dev == nullptr || v_dev == nullptr || out == nullptr)
        return fail(WMK_ERR_NULL, "k_dev, v_dev and out must not be NULL");
    if (!aligned16(k_dev) || !aligned16(v_dev)) return fail(WMK_ERR_ALIGN, "cache buffers must be 16-byte aligned");
    const size_t need = wmk_cache_bytes(d);
    if (capacity_bytes < need)
        return fail(WMK_ERR_CAPACITY, "capacity %zu bytes < %zu bytes needed per K/V buffer", capacity_bytes, need);
    wmk_cache* c = new (std::nothrow) wmk_cache;
    if (c == nullptr) return fail(WMK_ERR_CAPACITY, "out of host memory");
    c->d = *d;
    c->k = (char*)k_dev;
    c->v = (char*)v_dev;
    c->frame_bytes = (size_t)d->tokens_per_frame * d->num_heads * d->head_dim * elem_size(d->dtype);
    c->layer_bytes = c->frame_bytes * (size_t)(d->sink_frames + d->window_frames);
    c->frames.assign(d->num_layers, 0);
    *out = c;
    return ok();
}

void wmk_cache_destroy(wmk_cache* c) { delete c; }

namespace {

// The copies of one append: the frames still resident after it (sinks and the
// last W non-sink frames; the others would be overwritten by this same call
// and are skipped) in runs of adjacent slots, each run one K and one V range
// from k_new/v_new into `layer`.  At most 3 runs (sinks, window up to the ring
// end, wrapped window).  Returns the number of ranges, or -1 if they do not
// fit one launch.
int append_ranges(const wmk_cache* c, int32_t layer, int64_t F, const void* k_new, const void* v_new,
                  int32_t n_frames, wmk::CopyRange* r) {
    const wmk_cache_desc& d = c->d;
    const int64_t keep_from = F + n_frames - d.window_frames;
    int nr = 0;
    int64_t run_f = -1, run_slot = -1, run_len = 0;
    bool too_many = false;
    auto flush = [&]() {
        if (run_len == 0) return;
        if (nr + 2 > wmk::kMaxCopy) {
            too_many = true;
            return;
        }
        const size_t src_off = (size_t)(run_f - F) * c->frame_bytes;
        const size_t dst_off = (size_t)layer * c->layer_bytes + (size_t)run_slot * c->frame_bytes;
        const int64_t bytes = run_len * (int64_t)c->frame_bytes;
        r[nr++] = {(const char*)k_new + src_off, c->k + dst_off, bytes};
        r[nr++] = {(const char*)v_new + src_off, c->v + dst_off, bytes};
        run_len = 0;
    };
    for (int64_t f = F; f < F + n_frames; ++f) {
        if (!(f < d.sink_frames || f >= keep_from)) continue;
        const int64_t s = slot_of(d, f);
        if (run_len > 0 && f == run_f + run_len && s == run_slot + run_len) {
            ++run_len;
        } else {
            flush();
            run_f = f;
            run_slot = s;
            run_len = 1;
        }
    }
    flush();
    return too_many ? -1 : nr;
}

void dry_log_ranges(const wmk_cache* c, const void* k_new, const wmk::CopyRange* r, int nr) {
    for (int i = 0; i < nr; i += 2)
        dry_log(" %lld:%lld:%lld", (long long)((const char*)r[i].src - (const char*)k_new),
                (long long)((char*)r[i].dst - c->k), (long long)r[i].bytes);
    dry_log("\n");
}

}  // namespace

wmk_status wmk_cache_append_evict(wmk_cache* c, int32_t layer, const void* k_new, const void* v_new,
                                  int32_t n_frames, hipStream_t stream) {
    if (c == nullptr || k_new == nullptr || v_new == nullptr)
        return fail(WMK_ERR_NULL, "cache, k_new and v_new must not be NULL");
    const wmk_cache_desc& d = c->d;
    if (layer < 0 || layer >= d.num_layers)
        return fail(WMK_ERR_RANGE, "layer %d outside [0, %d)", layer, d.num_layers);
    if (n_frames <= 0) return fail(WMK_ERR_SHAPE, "n_frames %d <= 0", n_frames);
    if ((int64_t)n_frames * d.tokens_per_frame > INT32_MAX)
        return fail(WMK_ERR_SHAPE, "n_frames * tokens_per_frame exceeds 2^31 - 1");
    if (!aligned16(k_new) || !aligned16(v_new)) return fail(WMK_ERR_ALIGN, "k_new/v_new must be 16-byte aligned");

    const int64_t F = c->frames[layer];
    wmk::CopyRange r[wmk::kMaxCopy];
    const int nr = append_ranges(c, layer, F, k_new, v_new, n_frames, r);
    if (nr < 0) return fail(WMK_ERR_SHAPE, "append maps to more slot ranges than one launch copies");
    if (fault_injected()) return fail(WMK_ERR_HIP, "launch refused (WMK_FAULT_INJECT)");
    if (dry_run_path() != nullptr) {
        dry_log("append layer=%d F=%lld n=%d ranges=%d", layer, (long long)F, n_frames, nr / 2);
        dry_log_ranges(c, k_new, r, nr);
        c->frames[layer] = F + n_frames;
        return ok();
    }
    const hipError_t e = wmk::launch_copy_ranges(r, nr, stream);
    if (e != hipSuccess) return fail(WMK_ERR_HIP, "append launch failed: %s", hipGetErrorString(e));
    c->frames[layer] = F + n_frames;
    return ok();
}

wmk_status wmk_cache_append_evict_layers(wmk_cache* c, int32_t first_layer, int32_t n_layers, const void* k_new,
                                         const void* v_new, int32_t n_frames, hipStream_t stream) {
    if (c == nullptr || k_new == nullptr || v_new == nullptr)
        return fail(WMK_ERR_NULL, "cache, k_new and v_new must not be NULL");
    const wmk_cache_desc& d = c->d;
    if (n_layers <= 0) return fail(WMK_ERR_SHAPE, "n_layers %d <= 0", n_layers);
    if (first_layer < 0 || first_layer >= d.num_layers || n_layers > d.num_layers - first_layer)
        return fail(WMK_ERR_RANGE, "layers [%d, %d) outside [0, %d)", first_layer, first_layer + n_layers,
                    d.num_layers);
    if (n_frames <= 0) return fail(WMK_ERR_SHAPE, "n_frames %d <= 0", n_frames);
    if ((int64_t)n_frames * d.tokens_per_frame > INT32_MAX)
        return fail(WMK_ERR_SHAPE, "n_frames * tokens_per_frame exceeds 2^31 - 1");
    if (!aligned16(k_new) || !aligned16(v_new)) return fail(WMK_ERR_ALIGN, "k_new/v_new must be 16-byte aligned");
    const int64_t F = c->frames[first_layer];
    for (int32_t l = first_layer + 1; l < first_layer + n_layers; ++l)
        if (c->frames[l] != F)
            return fail(WMK_ERR_RANGE, "layer %d holds %lld frames, layer %d holds %lld: one call appends to layers "
                        "in step only", l, (long long)c->frames[l], first_layer, (long long)F);

    wmk::CopyRange r[wmk::kMaxCopy];
    const int nr = append_ranges(c, first_layer, F, k_new, v_new, n_frames, r);
    if (nr < 0) return fail(WMK_ERR_SHAPE, "append maps to more slot ranges than one launch copies");
    const int64_t src_stride = (int64_t)n_frames * (int64_t)c->frame_bytes;  // one layer's k_new block
    if (fault_injected()) return fail(WMK_ERR_HIP, "launch refused (WMK_FAULT_INJECT)");
    if (dry_run_path() != nullptr) {
        dry_log("append_layers first=%d layers=%d F=%lld n=%d ranges=%d src_stride=%lld dst_stride=%lld", first_layer,
                n_layers, (long long)F, n_frames, nr / 2, (long long)src_stride, (long long)c->layer_bytes);
        dry_log_ranges(c, k_new, r, nr);
        for (int32_t l = first_layer; l < first_layer + n_layers; ++l) c->frames[l] = F + n_frames;
        return ok();
    }
    const hipError_t e = wmk::launch_copy_layers(r, nr, n_layers, src_stride, (int64_t)c->layer_bytes, stream);
    if (e != hipSuccess) return fail(WMK_ERR_HIP, "append launch failed: %s", hipGetErrorString(e));
    for (int32_t l = first_layer; l < first_layer + n_layers; ++l) c->frames[l] = F + n_frames;
    return ok();
}

wmk_status wmk_cache_slots(const wmk_cache* c, int32_t layer, int64_t* frame_of_slot, int64_t* frames_appended) {
    if (c == nullptr) return fail(WMK_ERR_NULL, "cache is NULL");
    const wmk_cache_desc& d = c->d;
    if (layer < 0 || layer >= d.num_layers)
        return fail(WMK_ERR_RANGE, "layer %d outside [0, %d)", layer, d.num_layers);
    const int64_t F = c->frames[layer];
    if (frames_appended) *frames_appended = F;
    if (frame_of_slot) {
        const int n = d.sink_frames + d.window_frames;
        for (int i = 0; i < n; ++i) frame_of_slot[i] = -1;
        for (int64_t f = 0; f < std::min<int64_t>(F, d.sink_frames); ++f) frame_of_slot[f] = f;
        for (int64_t f = std::max<int64_t>(d.sink_frames, F - d.window_frames); f < F; ++f)
            frame_of_slot[slot_of(d, f)] = f;
    }
    return ok();
}

size_t wmk_attention_workspace_bytes(const wmk_head_desc* hd, int32_t q_tokens) {
    if (check_head(hd) != WMK_OK || q_tokens <= 0 || hd->dtype != WMK_BF16) return 0;
    const DeviceInfo di = device_info();
    // the larger need of the two kernel shapes a call may get (pieces never
    // exceed the number of resident workgroups)
    size_t need = 0;
    for (const int waves : {wmk::kWavesLong, wmk::kWavesShort}) {
        if (waves == wmk::kWavesShort && hd->head_dim != 128) continue;
        const int slots = di.slots(hd->head_dim, waves);
        const int32_t bq = wmk::attn_bf16_block_q(waves);
        const int64_t units = (int64_t)((q_tokens + bq - 1) / bq) * hd->num_heads;
        const int32_t tail = (int32_t)std::min<int64_t>(units, slots);
        need = std::max(need, wmk::attn_bf16_split_ws_bytes(hd->head_dim, waves, tail,
                                                            std::max(1, slots / std::max(1, tail))));
    }
    return need;
}

wmk_status wmk_chunk_attention(const wmk_cache* c, int32_t layer, const wmk_head_desc* hd, const void* q,
                               int32_t q_tokens, const wmk_kv_segment* seg, int32_t n_seg, void* out, float scale,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return chunk_attention_impl(c, layer, nullptr, 0, hd, q, q_tokens, seg, n_seg, out, scale, workspace,
                                workspace_bytes, stream);
}

wmk_status wmk_chunk_attention_noalloc(const wmk_cache* c, int32_t layer, const wmk_head_desc* hd, const void* q,
                                       int32_t q_tokens, const wmk_kv_segment* seg, int32_t n_seg, void* out,
                                       float scale, hipStream_t stream) {
    void* ws = nullptr;
    if (dry_run_path() != nullptr) {
        ws = (void*)(uintptr_t)0x7000000000ull;  // no device: a stand-in address, only planned with
    } else {
        const hipError_t e = wmk::noalloc_scratch(&ws);
        if (e != hipSuccess) return fail(WMK_ERR_HIP, "library scratch not available: %s", hipGetErrorString(e));
    }
    return chunk_attention_impl(c, layer, nullptr, 0, hd, q, q_tokens, seg, n_seg, out, scale, ws,
                                wmk::noalloc_scratch_bytes(), stream, false, true);
}

size_t wmk_attention_qk8_workspace_bytes(const wmk_head_desc* hd, int32_t q_tokens, int64_t kv_tokens) {
    if (check_head(hd) != WMK_OK || hd->dtype != WMK_BF16 || hd->head_dim != 128 || q_tokens <= 0 || kv_tokens < 0 ||
        kv_tokens > INT32_MAX)
        return 0;
    return qk8_bytes(hd->num_heads, q_tokens, kv_tokens, nullptr, nullptr) +
           wmk_attention_workspace_bytes(hd, q_tokens);
}

wmk_status wmk_chunk_attention_qk8(const wmk_cache* c, int32_t layer, const wmk_head_desc* hd, const void* q,
                                   int32_t q_tokens, const wmk_kv_segment* seg, int32_t n_seg, void* out, float scale,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return chunk_attention_impl(c, layer, nullptr, 0, hd, q, q_tokens, seg, n_seg, out, scale, workspace,
                                workspace_bytes, stream, true);
}

wmk_status wmk_chunk_attention_retained(const wmk_cache* c, int32_t layer, const int64_t* keep_frames,
                                        int32_t n_keep, const wmk_head_desc* hd, const void* q, int32_t q_tokens,
                                        const wmk_kv_segment* seg, int32_t n_seg, void* out, float scale,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (c == nullptr) return fail(WMK_ERR_NULL, "retained attention needs a cache");
    if (n_keep < 0) return fail(WMK_ERR_SHAPE, "n_keep %d < 0", n_keep);
    if (n_keep > 0 && keep_frames == nullptr) return fail(WMK_ERR_NULL, "keep_frames is NULL with n_keep %d", n_keep);
    return chunk_attention_impl(c, layer, keep_frames == nullptr ? &kNoFrame : keep_frames, n_keep, hd, q, q_tokens,
                                seg, n_seg, out, scale, workspace, workspace_bytes, stream);
}

wmk_status wmk_moba_attention(const wmk_moba_desc* m, const wmk_head_desc* hd, const void* q, const void* k,
                              const void* v, void* out, float scale, hipStream_t stream) {
    wmk::AttnCall call;
    const wmk_status s = moba_call(m, hd, q, k, v, out, scale, call);
    if (s != WMK_OK) return s;
    // MoBA q-tiles differ in cost: they run longest first and need no split tail
    return run_attention(call, hd->dtype, nullptr, 0, stream);
}

wmk_status wmk_moba_attention_train(const wmk_moba_desc* m, const wmk_head_desc* hd, const void* q, const void* k,
                                    const void* v, void* out, float* lse, float scale, hipStream_t stream) {
    wmk::AttnCall call;
    wmk_status s = moba_call(m, hd, q, k, v, out, scale, call);
    if (s != WMK_OK) return s;
    if (lse == nullptr) return fail(WMK_ERR_NULL, "lse must not be NULL");
    if (!aligned16(lse)) return fail(WMK_ERR_ALIGN, "lse must be 16-byte aligned");
    if (hd->dtype != WMK_BF16) return fail(WMK_ERR_DTYPE, "the training forward takes bf16 inputs");
    call.lse = lse;
    return run_attention(call, hd->dtype, nullptr, 0, stream);
}

size_t wmk_moba_backward_workspace_bytes(const wmk_moba_desc* m, const wmk_head_desc* hd) {
    if (m == nullptr || check_head(hd) != WMK_OK || m->tokens_per_frame < 1 || m->frames < 1 ||
        (m->bidir_block != 0 && m->bidir_block != 1))
        return 0;
    const int64_t n = (int64_t)(2 + m->bidir_block) * m->frames * m->tokens_per_frame;
    if (n > INT32_MAX) return 0;
    return align256((size_t)n * hd->num_heads * sizeof(float));
}

wmk_status wmk_moba_attention_backward(const wmk_moba_desc* m, const wmk_head_desc* hd, const void* q, const void* k,
                                       const void* v, const void* out, const void* dout, const float* lse, void* dq,
                                       void* dk, void* dv, float scale, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
    wmk::AttnCall call;
    wmk_status s = moba_call(m, hd, q, k, v, const_cast<void*>(out), scale, call);
    if (s != WMK_OK) return s;
    if (dout == nullptr || lse == nullptr || dq == nullptr || dk == nullptr || dv == nullptr)
        return fail(WMK_ERR_NULL, "dout, lse, dq, dk and dv must not be NULL");
    if (hd->dtype != WMK_BF16) return fail(WMK_ERR_DTYPE, "the backward takes bf16 inputs");
    if (hd->head_dim != 128) return fail(WMK_ERR_SHAPE, "the backward is built for head_dim 128");
    if (!aligned16(dout) || !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
        return fail(WMK_ERR_ALIGN, "dout/lse/dq/dk/dv must be 16-byte aligned");
    const size_t need = wmk_moba_backward_workspace_bytes(m, hd);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(WMK_ERR_CAPACITY, "the backward needs %zu bytes of workspace, got %zu", need, workspace_bytes);
    if (!aligned16(workspace)) return fail(WMK_ERR_ALIGN, "workspace must be 16-byte aligned");
    if (fault_injected()) return fail(WMK_ERR_HIP, "launch refused (WMK_FAULT_INJECT)");
    wmk::MobaBwd b;
    memset(&b, 0, sizeof b);
    // longest walk first for both kernels (workgroups of 256 rows or keys, 64-wide tiles)
    const int32_t n = call.q_tokens, br = wmk::moba_bwd_block(), nt = (n + br - 1) / br;
    std::vector<int32_t> cost_q(nt), cost_k(nt);
    for (int32_t t = 0; t < nt; ++t) {
        cost_q[t] = moba_rows_cost(call.mask, n, t * br, t * br + br);
        cost_k[t] = moba_ktile_cost(call.mask, n, t * br, t * br + br);
    }
    b.n_groups_q = plan_groups(cost_q, b.grp_q_start, b.grp_q_count);
    b.n_groups_k = plan_groups(cost_k, b.grp_k_start, b.grp_k_count);
    if (dry_run_path() != nullptr) {
        dry_log("moba_bwd n=%d heads=%d part=%d chunk=%d parts=%d groups_q=%d groups_k=%d\n", call.q_tokens,
                call.heads, call.mask.part_len, call.mask.chunk_len, call.mask.parts, b.n_groups_q, b.n_groups_k);
        for (int g = 0; g < b.n_groups_q; ++g) dry_log("bgroup q %d %d\n", b.grp_q_start[g], b.grp_q_count[g]);
        for (int g = 0; g < b.n_groups_k; ++g) dry_log("bgroup k %d %d\n", b.grp_k_start[g], b.grp_k_count[g]);
        // the query tiles each key block's dK/dV workgroup walks, from the kernel's own planner
        const int32_t br = wmk::moba_bwd_block();
        for (int32_t c0 = 0; c0 < call.q_tokens; c0 += br) {
            const wmk::tiles::TileRanges tr = wmk::tiles::col_tile_ranges(call.mask, call.q_tokens, c0, c0 + br);
            dry_log("ktiles %d %d %d %d %d %d %d %d %d %d %d\n", c0, std::min(c0 + br, call.q_tokens), tr.b0, tr.e0,
                    tr.b1, tr.e1, tr.b2, tr.e2, tr.b3, tr.e3, tr.total);
        }
        return ok();
    }
    b.q = q;
    b.k = k;
    b.v = v;
    b.out = out;
    b.dout = dout;
    b.lse = lse;
    b.dsum = (float*)workspace;
    b.dq = dq;
    b.dk = dk;
    b.dv = dv;
    b.n = call.q_tokens;
    b.heads = call.heads;
    b.scale = scale;
    b.mask = call.mask;
    const hipError_t e = wmk::launch_moba_backward(b, stream);
    if (e != hipSuccess) return fail(WMK_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

wmk_status wmk_cross_attention_train(const wmk_xattn_desc* x, const wmk_head_desc* hd, const void* q, const void* k,
                                     const void* v, void* out, float scale, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
    if (x == nullptr) return fail(WMK_ERR_NULL, "cross-attention descriptor is NULL");
    wmk_status s = check_head(hd);
    if (s != WMK_OK) return s;
    if (q == nullptr || k == nullptr || v == nullptr || out == nullptr)
        return fail(WMK_ERR_NULL, "q, k, v and out must not be NULL");
    if (x->chunk_q_tokens < 1 || x->chunks < 1 || x->env_tokens < 0 || x->local_tokens < 0 ||
        x->env_tokens + (int64_t)x->local_tokens < 1)
        return fail(WMK_ERR_SHAPE, "cross-attention descriptor: chunk_q_tokens %d chunks %d env %d local %d",
                    x->chunk_q_tokens, x->chunks, x->env_tokens, x->local_tokens);
    const int64_t nq = (int64_t)x->chunk_q_tokens * x->chunks;
    const int64_t nk = x->env_tokens + (int64_t)x->local_tokens * x->chunks;
    if (nq > INT32_MAX || nk > INT32_MAX) return fail(WMK_ERR_SHAPE, "more than 2^31 - 1 query or key tokens");
    if ((s = check_scale(scale)) != WMK_OK) return s;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(WMK_ERR_ALIGN, "q/k/v/out must be 16-byte aligned");
    wmk::AttnCall call;
    memset(&call, 0, sizeof call);
    call.kv.k[0] = k;
    call.kv.v[0] = v;
    call.kv.end[0] = (int32_t)nk;
    call.kv.n = 1;
    call.q = q;
    call.out = out;
    call.q_tokens = (int32_t)nq;
    call.heads = hd->num_heads;
    call.head_dim = hd->head_dim;
    call.kv_total = (int32_t)nk;
    call.scale = scale;
    call.mask.mode = wmk::kMaskCross;
    call.mask.part_len = x->chunk_q_tokens;
    call.mask.chunk_len = x->local_tokens;
    call.mask.parts = x->chunks;
    call.mask.env_len = x->env_tokens;
    wmk::set_mask_divisors(call.mask);
    return run_attention(call, hd->dtype, workspace, workspace_bytes, stream);
}

const char* wmk_last_error(void) { return g_err.c_str(); }

}  // extern "C"
#pragma GCC visibility pop
