// Cache append/evict data movement: an exact copy of the finalized chunk's K
// and V rows into their ring slots.  Eviction is the overwrite itself and moves
// no bytes.  A chunk lands in at most three contiguous slot ranges (sink part,
// window part up to the ring end, wrapped window part) per tensor, so one
// launch copies a short list of (src, dst, bytes) ranges with 16-byte vector
// loads and stores.
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
constexpr int kUnroll = 2;      // 16-byte transfers in flight per lane and pass
constexpr int kMaxBlocks = 4096;  // grid-stride beyond this (16 workgroups per CU)

// Plain (cached) loads and stores: on MI355X they sustain a higher copy rate
// than nontemporal ones for these sizes.  Each pass of a workgroup moves
// kThreads * kUnroll 16-byte units: all loads, then all stores.
__global__ __launch_bounds__(kThreads) void copy_ranges_kernel(CopyArgs a) {
    const int64_t total = a.end[a.n - 1];
    const int64_t stride = (int64_t)gridDim.x * (kThreads * kUnroll);
    for (int64_t base = (int64_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x; base < total; base += stride) {
        u32x4 buf[kUnroll];
        const u32x4* src[kUnroll];
        u32x4* dst[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + (int64_t)u * kThreads;
            int r = 0;
#pragma unroll
            for (int t = 0; t < kMaxCopy - 1; ++t)
                if (t < a.n - 1 && i >= a.end[t]) r = t + 1;
            const int64_t off = i - (r ? a.end[r - 1] : 0);
            src[u] = a.src[r] + off;
            dst[u] = a.dst[r] + off;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if (base + (int64_t)u * kThreads < total) buf[u] = *src[u];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if (base + (int64_t)u * kThreads < total) *dst[u] = buf[u];
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
    const int64_t per_block = (int64_t)kThreads * kUnroll;
    const int64_t blocks = std::min<int64_t>((acc + per_block - 1) / per_block, kMaxBlocks);
    hipLaunchKernelGGL(copy_ranges_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace wmk
