// Cache append/evict data movement: an exact copy of the finalized chunk's K
// and V rows into their ring slots.  Eviction is the overwrite itself and moves
// no bytes.  A chunk lands in at most three contiguous slot ranges (sink part,
// window part up to the ring end, wrapped window part) per tensor, so one
// launch copies a short list of (src, dst, bytes) ranges with 16-byte vector
// loads and stores.  ("How the cache keeps the world alive": the sliding
// cache keeps its sink frames and discards the oldest window frame; the
// frames appended are the recently finalized ones, "World in World", second
// paragraph.)
// HBM-bound: bytes read = bytes written = the chunk's K + V.
#include <algorithm>

#include "wmk_internal.h"

namespace wmk {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct CopyArgs {
    const u32x4* src[kMaxCopy];
    u32x4* dst[kMaxCopy];
    int64_t end[kMaxCopy];  // exclusive prefix sum of range lengths, in 16-byte units
    int32_t n;
};

constexpr int kThreads = 256;
constexpr int kMaxBlocks = 1024;  // grid-stride beyond this (4 workgroups per CU)

// One 16-byte load and one 16-byte store per lane and pass, both nontemporal:
// the finalized chunk is read once, and the slots written are read again only
// by a later chunk's attention, after every other layer's traffic has passed
// through the caches.  Consecutive workgroups take consecutive 4 KB pieces, so
// the whole grid sweeps each range front to back.  Measured on MI355X with a
// working set beyond the Infinity Cache (30 layers, distinct sources), this
// form moved 74 MB in 13.3-13.4 us; plain accesses with two or more units per
// lane took 14.7-15.8 us, and block-contiguous slices 14.8 us or more.
__global__ __launch_bounds__(kThreads) void copy_ranges_kernel(CopyArgs a) {
    // The grid strides over the concatenation of the ranges, so every thread
    // moves the same number of units (+-1) however the ranges are cut; each
    // range gets its own loop (uniform: its pointers stay in scalar registers),
    // entered at the thread's position in the concatenated index space.
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const int64_t first = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    int64_t start = 0;  // first unit of range r in the concatenation
    for (int r = 0; r < a.n; ++r) {
        const int64_t len = a.end[r] - start;
        const u32x4* src = a.src[r];
        u32x4* dst = a.dst[r];
        for (int64_t j = (first - start % stride + stride) % stride; j < len; j += stride)
            __builtin_nontemporal_store(__builtin_nontemporal_load(src + j), dst + j);
        start = a.end[r];
    }
}

// The same copy for a run of layers in one launch: the ranges of the first
// layer, repeated for each next layer at fixed strides (its source is the next
// [n_frames * tpf][H][D] block, its slots the same slots of the next layer).
// One launch then moves the whole run's bytes: at the rolling session's 30
// layers, 2.2 GB instead of 30 launches of 74 MB, each of which loses its ramp
// and tail.  The grid strides over the concatenation of all layers' ranges as
// above; len_mod[r] = (length of range r) mod (grid stride), from the host,
// carries each thread's entry offset from range to range without a 64-bit
// modulo per range.
struct LayerCopyArgs {
    CopyArgs r;                // ranges of the first layer
    int64_t len_mod[kMaxCopy];
    int64_t src_stride;        // 16-byte units from one layer's source to the next
    int64_t dst_stride;        // 16-byte units from one layer's slots to the next
    int32_t layers;
};

__global__ __launch_bounds__(kThreads) void copy_layers_kernel(LayerCopyArgs a) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t j0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;  // entry offset into the current range
    for (int l = 0; l < a.layers; ++l) {
        for (int r = 0; r < a.r.n; ++r) {
            const int64_t len = a.r.end[r] - (r == 0 ? 0 : a.r.end[r - 1]);
            const u32x4* src = a.r.src[r] + l * a.src_stride;
            u32x4* dst = a.r.dst[r] + l * a.dst_stride;
            for (int64_t j = j0; j < len; j += stride)
                __builtin_nontemporal_store(__builtin_nontemporal_load(src + j), dst + j);
            j0 -= a.len_mod[r];
            if (j0 < 0) j0 += stride;
        }
    }
}

}  // namespace

hipError_t launch_copy_ranges(const CopyRange* r, int n, hipStream_t s) {
    CopyArgs a = {};
    int m = 0;
    int64_t acc = 0;
    for (int i = 0; i < n && i < kMaxCopy; ++i) {
        if (r[i].bytes <= 0) continue;
        a.src[m] = (const u32x4*)r[i].src;
        a.dst[m] = (u32x4*)r[i].dst;
        acc += r[i].bytes / 16;
        a.end[m] = acc;
        ++m;
    }
    if (m == 0) return hipSuccess;
    a.n = m;
    const int64_t blocks = std::min<int64_t>((acc + kThreads - 1) / kThreads, kMaxBlocks);
    hipLaunchKernelGGL(copy_ranges_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_copy_layers(const CopyRange* r, int n, int32_t layers, int64_t src_stride_bytes,
                              int64_t dst_stride_bytes, hipStream_t s) {
    LayerCopyArgs a = {};
    int m = 0;
    int64_t acc = 0;
    for (int i = 0; i < n && i < kMaxCopy; ++i) {
        if (r[i].bytes <= 0) continue;
        a.r.src[m] = (const u32x4*)r[i].src;
        a.r.dst[m] = (u32x4*)r[i].dst;
        acc += r[i].bytes / 16;
        a.r.end[m] = acc;
        ++m;
    }
    if (m == 0 || layers <= 0) return hipSuccess;
    a.r.n = m;
    a.layers = layers;
    a.src_stride = src_stride_bytes / 16;
    a.dst_stride = dst_stride_bytes / 16;
    const int64_t total = acc * layers;
    const int64_t blocks = std::min<int64_t>((total + kThreads - 1) / kThreads, kMaxBlocks);
    const int64_t stride = blocks * kThreads;
    for (int i = 0; i < m; ++i) a.len_mod[i] = (a.r.end[i] - (i == 0 ? 0 : a.r.end[i - 1])) % stride;
    hipLaunchKernelGGL(copy_layers_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace wmk
