// Reference rates for the benchmark (measurement code, not part of the C ABI
// of include/wmk.h): the bf16 matrix-core rate that a long stream of
// independent v_mfma_f32_32x32x16_bf16 instructions reaches on this device
// (the attention kernels' fraction of peak is also reported against this
// measured rate, which includes the shader clock the chip holds under a
// sustained matrix-core load), and the rate of fp32 atomic adds in the
// pattern of a dQ accumulation (the cost a fused attention backward would pay).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;  // 4 waves: one per SIMD
constexpr int kChains = 4;     // independent accumulators per wave

// Each wave issues iters * kChains MFMAs of 32x32x16 (32768 flops each) on
// operands held in registers; the sums are written so nothing is dropped.
// The operands are four register sets of pseudo-random bf16 values in
// [1/16, 2) with random signs, rotated from one MFMA to the next, so the
// multipliers switch as they do on real data (identical operands every time
// would draw less power and let the clock run higher than any kernel's).
__device__ __forceinline__ uint32_t mix(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    return x ^ (x >> 16);
}

__global__ __launch_bounds__(kThreads) void mfma_bf16_rate_kernel(int iters, float* sink) {
    const int lane = threadIdx.x;
    bf16x8 a[4], b[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t ha = mix((uint32_t)(blockIdx.x * kThreads + lane) * 64u + r * 8 + i);
            const uint32_t hb = mix(ha ^ 0x9e3779b9u);
            // sign, exponent 123..127 (values 2^-4 .. 2^0 scaled by 1.m), 7 random mantissa bits
            const uint16_t ba = (uint16_t)(((ha >> 31) << 15) | ((123u + (ha >> 8) % 5u) << 7) | (ha & 0x7fu));
            const uint16_t bb = (uint16_t)(((hb >> 31) << 15) | ((123u + (hb >> 8) % 5u) << 7) | (hb & 0x7fu));
            a[r][i] = __builtin_bit_cast(__bf16, ba);
            b[r][i] = __builtin_bit_cast(__bf16, bb);
        }
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
    for (int it = 0; it < iters; it += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int c = 0; c < kChains; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(c + u) & 3], b[(c + 2 * u + 1) & 3], acc[c], 0, 0,
                                                                 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    sink[(size_t)blockIdx.x * kThreads + lane] = s;
}

// fp32 atomic adds without return in the pattern a fused attention backward
// would accumulate dQ with: each workgroup adds a 64-row x 128-dim fp32 block
// (row stride heads x 128) at a pseudo-random 64-row tile of one head.
__global__ __launch_bounds__(512) void atomic_add_rate_kernel(float* acc, int n_tiles, int heads, int rounds) {
    const int t = threadIdx.x;
    const int head = blockIdx.x % heads;
    for (int r = 0; r < rounds; ++r) {
        const int tile = (int)(mix((uint32_t)blockIdx.x * 977u + (uint32_t)r) % (uint32_t)n_tiles);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int e = i * 512 + t;  // element of the 64 x 128 block
            float* p = acc + ((size_t)(tile * 64 + (e >> 7)) * heads + head) * 128 + (e & 127);
            __hip_atomic_fetch_add(p, 1.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace

extern "C" {

// Enqueue `blocks` workgroups of atomic_add_rate_kernel over acc, a [n_tiles * 64]
// [heads][128] fp32 buffer; each workgroup adds `rounds` blocks of 32 KiB.
// Returns the launch status (hipError_t as int).
__attribute__((visibility("default"))) int wmk_rate_atomic_add_f32(float* acc, int n_tiles, int heads, int blocks,
                                                                   int rounds, hipStream_t s) {
    if (acc == nullptr || n_tiles <= 0 || heads <= 0 || blocks <= 0 || rounds <= 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(atomic_add_rate_kernel, dim3(blocks), dim3(512), 0, s, acc, n_tiles, heads, rounds);
    return (int)hipGetLastError();
}

// Enqueue `blocks` workgroups of 4 waves, each wave running iters * 4 bf16
// 32x32x16 MFMAs (iters a positive multiple of 4); sink receives blocks * 256
// floats.  Returns the launch status (hipError_t as int); flops = blocks * 4 *
// iters * 4 * 32768.
__attribute__((visibility("default"))) int wmk_rate_mfma_bf16(int blocks, int iters, float* sink, hipStream_t s) {
    if (blocks <= 0 || iters <= 0 || iters % 4 != 0 || sink == nullptr) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_bf16_rate_kernel, dim3(blocks), dim3(kThreads), 0, s, iters, sink);
    return (int)hipGetLastError();
}

__attribute__((visibility("default"))) double wmk_rate_mfma_bf16_flops(int blocks, int iters) {
    return (double)blocks * (kThreads / 64) * iters * kChains * 32768.0;
}

}  // extern "C"
