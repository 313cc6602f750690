// fp32 attention: the plain SIMT path for fp32 inputs (no matrix cores).
//
// Four lanes share one (query row, head); each owns head_dim/4 dimensions of
// q and of the output accumulator.  Keys are visited one at a time inside the
// row's allowed key intervals with an online (running max) softmax in fp32:
// the same computation as the MFMA path, without tiling, for small fp32
// workloads such as the tiny rollout.
#include <math.h>

#include "wmk_internal.h"

namespace wmk {
namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerRow = 4;

__device__ __forceinline__ void row_intervals(const AttnCall& c, int64_t i, int32_t* lo, int32_t* hi) {
    lo[1] = 0; hi[1] = 0;
    if (c.mask.mode == kMaskNone) {
        lo[0] = 0; hi[0] = c.kv_total;
        return;
    }
    if (c.mask.mode == kMaskCross) {  // environment prompt + this chunk's local prompt
        const int32_t ch = (int32_t)(i / c.mask.part_len);
        lo[0] = 0; hi[0] = c.mask.env_len;
        lo[1] = c.mask.env_len + ch * c.mask.chunk_len; hi[1] = lo[1] + c.mask.chunk_len;
        return;
    }
    const int32_t L = c.mask.part_len, cl = c.mask.chunk_len;
    const int32_t part = (int32_t)(i / L), r = (int32_t)(i % L), k = r / cl;
    const int32_t e = min((k + 1) * cl, L);
    if (part == 0) {              // clean: block-causal over clean chunks
        lo[0] = 0; hi[0] = e;
    } else if (part == 1) {       // noisy: earlier clean chunks + its own noisy chunk
        lo[0] = 0; hi[0] = k * cl; lo[1] = L + k * cl; hi[1] = L + e;
    } else {                      // appended bidirectional block: itself only
        lo[0] = 2 * L; hi[0] = 3 * L;
    }
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_f32_kernel(AttnCall c) {
    constexpr int DL = D / kLanesPerRow;
    const int64_t pair = ((int64_t)blockIdx.x * kThreads + threadIdx.x) / kLanesPerRow;
    const int sub = threadIdx.x % kLanesPerRow;
    const int64_t n_pairs = (int64_t)c.q_tokens * c.heads;
    const bool active = pair < n_pairs;
    const int64_t row = active ? pair / c.heads : 0;
    const int32_t head = active ? (int32_t)(pair % c.heads) : 0;
    const int64_t stride = (int64_t)c.heads * D;
    const float cs = c.scale * 1.4426950408889634f;  // scale * log2(e): softmax via exp2

    float q[DL], acc[DL];
    const float* qp = (const float*)c.q + row * stride + (int64_t)head * D + sub * DL;
#pragma unroll
    for (int d = 0; d < DL; ++d) { q[d] = active ? qp[d] : 0.0f; acc[d] = 0.0f; }
    float m = -INFINITY, l = 0.0f;

    int32_t lo[2], hi[2];
    row_intervals(c, row, lo, hi);
    for (int t = 0; t < 2; ++t) {
        int32_t start = 0;
        for (int s = 0; s < c.kv.n; ++s) {
            const int32_t end = c.kv.end[s];
            const int32_t a = max(lo[t], start), b = min(hi[t], end);
            const float* kb = (const float*)c.kv.k[s] + (int64_t)head * D + sub * DL;
            const float* vb = (const float*)c.kv.v[s] + (int64_t)head * D + sub * DL;
            for (int32_t j = a; j < b; ++j) {
                const float* kp = kb + (int64_t)(j - start) * stride;
                float dot = 0.0f;
#pragma unroll
                for (int d = 0; d < DL; ++d) dot = fmaf(q[d], kp[d], dot);
                dot += __shfl_xor(dot, 1, kLanesPerRow);
                dot += __shfl_xor(dot, 2, kLanesPerRow);
                const float sc = dot * cs;
                const float m_new = fmaxf(m, sc);
                const float alpha = exp2f(m - m_new);
                const float p = exp2f(sc - m_new);
                l = l * alpha + p;
                const float* vp = vb + (int64_t)(j - start) * stride;
#pragma unroll
                for (int d = 0; d < DL; ++d) acc[d] = fmaf(acc[d], alpha, p * vp[d]);
                m = m_new;
            }
            start = end;
        }
    }
    if (!active) return;
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    float* op = (float*)c.out + row * stride + (int64_t)head * D + sub * DL;
#pragma unroll
    for (int d = 0; d < DL; ++d) op[d] = acc[d] * inv;
}

}  // namespace

hipError_t launch_attn_f32(const AttnCall& c, hipStream_t s) {
    const int64_t threads = (int64_t)c.q_tokens * c.heads * kLanesPerRow;
    const unsigned blocks = (unsigned)((threads + kThreads - 1) / kThreads);
    if (c.head_dim == 64)
        hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(blocks), dim3(kThreads), 0, s, c);
    else if (c.head_dim == 128)
        hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(blocks), dim3(kThreads), 0, s, c);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace wmk
