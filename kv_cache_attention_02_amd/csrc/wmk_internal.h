// Internal interface between the C ABI (wmk_api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fastdiv.h"

namespace wmk {

constexpr int kMaxSeg = 16;       // spans of one call: cache runs + caller segments
constexpr int kMaxCallerSeg = 4;  // caller segments of one call
constexpr int kFewSeg = 5;        // span count of the common kernel (one cache run + 4 segments)
constexpr int kMaxGroups = 64;    // q-tile groups of a longest-first launch order
constexpr int kNumXcd = 8;        // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kMaxHeads = 4096;   // a 64-key tile of all heads stays below 2^31 bytes (32-bit buffer offsets)

// Keys/values seen by one attention call: the virtual concatenation of up to
// N spans, each [tokens][heads][head_dim].  end is the exclusive prefix sum of
// the span lengths.
template <int N>
struct KvSpansN {
    const void* k[N];
    const void* v[N];
    int32_t end[N];
    int32_t n;
};
using KvSpans = KvSpansN<kMaxSeg>;

// Per-row key mask of an attention call (every row allows at most two
// half-open key ranges):
//   kMaskNone:  every key (chunk attention at a denoising step);
//   kMaskMoba:  the MoBA training sequence [clean | noisy | block]: part_len =
//               frames * tokens_per_frame, chunk_len = chunk_frames *
//               tokens_per_frame, parts = 2 or 3;
//   kMaskCross: chunk-causal cross-attention over a multi-chunk sequence: query
//               chunk i (part_len rows each, parts chunks) reads the env_len
//               environment-prompt keys and local prompt i (chunk_len keys at
//               env_len + i * chunk_len) only.
constexpr int32_t kMaskNone = 0;
constexpr int32_t kMaskMoba = 1;
constexpr int32_t kMaskCross = 2;
struct MaskShape {
    int32_t mode;
    int32_t part_len;
    int32_t chunk_len;
    int32_t parts;
    int32_t env_len;
    FastDiv part_div;   // division by part_len (set with set_mask_divisors)
    FastDiv chunk_div;  // division by chunk_len
};

// Fill in the divisors of a mask (a length of 0, which no kernel divides by,
// gets the divisor 1).
inline void set_mask_divisors(MaskShape& m) {
    m.part_div = make_fastdiv(m.part_len > 1 ? (uint32_t)m.part_len : 1u);
    m.chunk_div = make_fastdiv(m.chunk_len > 1 ? (uint32_t)m.chunk_len : 1u);
}

template <int N>
struct AttnCallN {
    const void* q;
    void* out;
    int32_t q_tokens;
    int32_t heads;
    int32_t head_dim;
    int32_t kv_total;
    float scale;
    KvSpansN<N> kv;
    MaskShape mask;
    float* lse;  // optional [heads][q_tokens] natural-log sum of exp of the scaled scores (NULL: not written)
};
using AttnCall = AttnCallN<kMaxSeg>;

// Work plan for the bf16 MFMA kernel: which (head, q-tile) units run in which
// launch order, and how the last partial round is split over the key range.
// Waves per workgroup of the bf16 kernel: 8 (one workgroup per CU) for the
// long key walks; 4 (two workgroups per CU, so that one's unit fill runs beside
// the other's steps) for calls whose units walk at most kShortUnitTiles key
// tiles -- bf16, head_dim 128.
constexpr int kWavesLong = 8;
constexpr int kWavesShort = 4;
constexpr int kShortUnitTiles = 32;

struct AttnPlan {
    int32_t waves;          // kWavesLong or kWavesShort
    int32_t n_qtiles;       // ceil(q_tokens / attn_bf16_block_q(waves))
    int32_t n_units;        // n_qtiles * heads
    int32_t n_groups;       // > 0: q-tiles visited in this group order (longest first, grp_* below)
    int32_t xcd_remap;      // 1: keep consecutive units of one head on one XCD
    // split tail: the last `split_units` units (in launch order) run as
    // `splits` pieces each over disjoint key-tile ranges, merged in-kernel.
    int32_t split_units;
    int32_t splits;
    // the same counts as multiply-shift divisors: heads (c.heads), n_qtiles, splits
    FastDiv heads_div;
    FastDiv qtiles_div;
    FastDiv splits_div;
    void* ws;               // workspace for the split tail (may be NULL when split_units == 0)
    // FP8 QK^T (all NULL for the bf16 product): e4m3 codes of Q in blocks of 32
    // rows and of K in blocks of 64 keys (one tile, stored in the kernel's LDS
    // layout), each block [rows][head_dim] per (block, head), and the fp32 scale
    // of each block at [block * heads + head]
    const uint8_t* q8;
    const float* q8_scale;
    const uint8_t* k8;
    const float* k8_scale;
    // the group order (last: the kernel reads the fields above at its start)
    int32_t grp_start[kMaxGroups];
    int32_t grp_count[kMaxGroups];
};

// bf16 MFMA attention.  Returns the launch status.
hipError_t launch_attn_bf16(const AttnCall& c, const AttnPlan& plan, hipStream_t s);

// Query rows per workgroup (q-tile) of the bf16 kernel with `waves` waves.
int attn_bf16_block_q(int waves);

// Number of resident workgroups of the bf16 kernel per CU (occupancy) for head_dim and waves.
int attn_bf16_blocks_per_cu(int head_dim, int waves);

// Workspace bytes the bf16 kernel's split tail needs for split_units x splits pieces.
size_t attn_bf16_split_ws_bytes(int head_dim, int waves, int32_t split_units, int32_t splits);

// FP8 e4m3 block quantization of a bf16 [tokens][heads][head_dim] sequence
// given as n_spans spans (end: exclusive prefix sums of their lengths) into
// blocks of `rows` rows per head (rows = 64: key tiles in the attention
// kernel's LDS layout; rows = 32: plain row-major query blocks).  head_dim 128.
hipError_t launch_quant_e4m3(const void* const* src, const int32_t* end, int n_spans, int32_t tokens, int32_t heads,
                             int head_dim, int rows, uint8_t* codes, float* scales, hipStream_t s);

// Backward of the MoBA-masked attention (bf16, head_dim 128): all tensors
// [n][heads][128] bf16 except lse ([heads][n] natural log, from the forward)
// and dsum ([heads][n] fp32 scratch for D = dO . O).
struct MobaBwd {
    const void* q;
    const void* k;
    const void* v;
    const void* out;
    const void* dout;
    const float* lse;
    float* dsum;
    void* dq;
    void* dk;
    void* dv;
    int32_t n;
    int32_t heads;
    float scale;
    MaskShape mask;
    // launch order, longest walk first, of the 256-row tiles (dQ kernel) and of
    // the 256-key tiles (dK/dV kernel): runs of consecutive tiles, all heads of
    // a tile together (0 groups: the natural order)
    int32_t n_groups_q, n_groups_k;
    int32_t grp_q_start[kMaxGroups], grp_q_count[kMaxGroups];
    int32_t grp_k_start[kMaxGroups], grp_k_count[kMaxGroups];
};
hipError_t launch_moba_backward(const MobaBwd& b, hipStream_t s);

// Rows (dQ kernel) or keys (dK/dV kernel) a workgroup of the backward owns.
int moba_bwd_block();

// Library-held split-tail scratch of wmk_chunk_attention_noalloc: its size,
// and the device address of the current device's copy (looked up on the
// first call on each device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** out);

// fp32 attention (plain SIMT; correctness path for fp32 inputs).
hipError_t launch_attn_f32(const AttnCall& c, hipStream_t s);

// Copy of up to 8 byte ranges (all multiples of 16 bytes, 16-byte aligned) in one launch.
struct CopyRange {
    const void* src;
    void* dst;
    int64_t bytes;
};
constexpr int kMaxCopy = 8;
hipError_t launch_copy_ranges(const CopyRange* r, int n, hipStream_t s);
// the ranges of one layer's append, repeated for `layers` consecutive layers
// (sources and destinations advanced by the given byte strides per layer)
hipError_t launch_copy_layers(const CopyRange* r, int n, int32_t layers, int64_t src_stride_bytes,
                              int64_t dst_stride_bytes, hipStream_t s);

}  // namespace wmk
