/*
 * Seeded synthetic inputs for tests and benchmarks (GPU side).
 *
 * The same Philox4x32-10 (Salmon et al., SC'11) counter/key assignment and
 * Irwin-Hall-12 byte sum as philox.c, so that a tensor drawn here has the same
 * bits as one drawn on the host.  Used to fill large device tensors without a
 * host round trip; it draws numbers and holds no attention arithmetic.
 */
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ void philox10(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3,
                                         uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
        uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
        k0 += 0x9E3779B9u; k1 += 0xBB67AE85u;
    }
}

__device__ __forceinline__ int bytesum(uint32_t x) {
    return (int)(x & 0xffu) + (int)((x >> 8) & 0xffu) + (int)((x >> 16) & 0xffu) + (int)(x >> 24);
}

__device__ __forceinline__ float draw(uint64_t idx, uint32_t chunk, uint32_t tag, uint32_t k0, uint32_t k1) {
    uint32_t c0 = (uint32_t)idx, c1 = (uint32_t)(idx >> 32), c2 = chunk, c3 = tag;
    philox10(c0, c1, c2, c3, k0, k1);
    return (float)(bytesum(c0) + bytesum(c1) + bytesum(c2) - 1530) / 256.0f;
}

__global__ void fill_f32(float* __restrict__ dst, uint64_t start, uint64_t n, uint32_t chunk, uint32_t tag,
                         uint32_t k0, uint32_t k1) {
    uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = draw(start + i, chunk, tag, k0, k1);
}

__global__ void fill_bf16(uint16_t* __restrict__ dst, uint64_t start, uint64_t n, uint32_t chunk, uint32_t tag,
                          uint32_t k0, uint32_t k1) {
    uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        uint32_t u = __float_as_uint(draw(start + i, chunk, tag, k0, k1));
        dst[i] = (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
    }
}

}  // namespace

/* dtype: 0 = fp32, 1 = bf16.  Returns a hipError_t value (0 on success). */
extern "C" int synth_gpu_fill(void* dst, uint64_t start, uint64_t n, int dtype, uint64_t seed, uint32_t chunk,
                              uint32_t layer, uint32_t step, uint32_t kind, hipStream_t stream) {
    if (n == 0) return 0;
    if (dst == nullptr || (dtype != 0 && dtype != 1)) return (int)hipErrorInvalidValue;
    uint32_t tag = (kind & 0xffu) | ((step & 0xffu) << 8) | (layer << 16);
    uint64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (dtype == 0)
        fill_f32<<<(unsigned)blocks, 256, 0, stream>>>((float*)dst, start, n, chunk, tag, (uint32_t)seed,
                                                       (uint32_t)(seed >> 32));
    else
        fill_bf16<<<(unsigned)blocks, 256, 0, stream>>>((uint16_t*)dst, start, n, chunk, tag, (uint32_t)seed,
                                                        (uint32_t)(seed >> 32));
    return (int)hipGetLastError();
}
