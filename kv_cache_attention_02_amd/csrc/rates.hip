// Reference rates for the benchmark (measurement code, not part of the C ABI
// of include/wmk.h): the bf16 matrix-core rate that a long stream of
// independent v_mfma_f32_32x32x16_bf16 instructions reaches on this device.
// The attention kernels' fraction of peak is also reported against this
// measured rate, which includes the shader clock the chip holds under a
// sustained matrix-core load.
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

}  // namespace

extern "C" {

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
