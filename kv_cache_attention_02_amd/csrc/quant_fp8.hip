// FP8 (OCP e4m3) block quantization of the QK^T operands: the precision
// variant of the attention step ("LingBot-World-Infinity" acceleration table:
// a quantized-QK^T attention kernel replaces FlashAttention-2).
//
// A [tokens][heads][head_dim] bf16 sequence -- the queries, or the keys as the
// attention kernel reads them (the virtual concatenation of its spans) -- is
// cut into blocks of ROWS consecutive rows per head.  Per block, in fp32:
//   amax = max |x|,  scale = amax / 448,  inv = 448 / amax  (0 and 0 if amax = 0),
//   code = e4m3(clamp(x * inv, -448, 448))  rounded to nearest even,
// so the block's largest entry maps to +-448.  Rows past the end quantize as
// zeros.  Output: per (block, head) the ROWS x head_dim codes as one
// contiguous block, row-major, and one fp32 scale at [block * heads + head].
// Key blocks (64 rows, one attention tile) are stored in the attention
// kernel's LDS layout: the 16-byte chunks of row r are XOR-permuted by
// (r / rows-per-256-bytes) % chunks-per-row, so that a straight copy of the
// block into LDS gives bank-conflict-free fragment reads.
//
// HBM-bound: reads 2 bytes and writes 1 byte per element, plus one scale per
// block and head.
#include "wmk_internal.h"

namespace wmk {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kQThreads = 256;
constexpr float kE4m3Max = 448.0f;

struct QuantArgs {
    const void* src[kMaxSeg];  // spans of the sequence, each [tokens][heads][head_dim] bf16
    int32_t end[kMaxSeg];      // exclusive prefix sums of the span lengths
    int32_t n_spans;
    int32_t tokens;            // rows of the sequence (= end of the last span)
    int32_t heads;
    uint8_t* codes;            // [blocks][heads][ROWS][head_dim]
    float* scales;             // [blocks][heads]
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Four fp32 values -> four e4m3 codes (byte i = value i), nearest even.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    const uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

__device__ __forceinline__ float clamp448(float x) { return fminf(fmaxf(x, -kE4m3Max), kE4m3Max); }

// One workgroup per (block, head).  Thread t handles row t / TPR of the block
// and the DPT dims (t % TPR) * DPT .. + DPT - 1.
template <int D, int ROWS, bool SWZ>
__global__ __launch_bounds__(kQThreads) void quant_e4m3_kernel(QuantArgs a) {
    constexpr int TPR = kQThreads / ROWS;  // threads per row
    constexpr int DPT = D / TPR;           // dims per thread
    static_assert(DPT % 8 == 0, "whole 16-byte loads per thread");
    constexpr int CPR = D / 16;            // 16-byte code chunks per row
    constexpr int RPB = 256 / D;           // rows per 256 bytes of codes (one LDS bank row)
    const int32_t blk = blockIdx.x / a.heads, head = blockIdx.x % a.heads;
    const int t = threadIdx.x;
    const int r = t / TPR, part = t % TPR;
    const int32_t j = blk * ROWS + r;

    // load DPT bf16 values of row j (zeros past the end)
    u32x4 raw[DPT / 8];
#pragma unroll
    for (int i = 0; i < DPT / 8; ++i) raw[i] = u32x4{0u, 0u, 0u, 0u};
    if (j < a.tokens) {
        int x = 0;
        while (x + 1 < a.n_spans && j >= a.end[x]) ++x;
        const int32_t start = x == 0 ? 0 : a.end[x - 1];
        const u32x4* p = (const u32x4*)((const char*)a.src[x] +
                                        (((int64_t)(j - start) * a.heads + head) * D + part * DPT) * 2);
#pragma unroll
        for (int i = 0; i < DPT / 8; ++i) raw[i] = p[i];
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < DPT / 8; ++i)
#pragma unroll
        for (int w = 0; w < 4; ++w)
            amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(raw[i][w])), fabsf(bf16_hi(raw[i][w]))));
    // workgroup max: butterfly in the wave, then across the 4 waves through LDS
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    __shared__ float s_max[kQThreads / 64];
    if ((t & 63) == 0) s_max[t >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    const float inv = amax > 0.0f ? kE4m3Max / amax : 0.0f;
    const float scale = amax / kE4m3Max;

    // DPT codes -> DPT / 4 words, stored as 16-byte chunks (or one 8-byte half chunk)
    uint32_t w[DPT / 4];
#pragma unroll
    for (int i = 0; i < DPT / 8; ++i)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const uint32_t x0 = raw[i][2 * h2], x1 = raw[i][2 * h2 + 1];
            w[2 * i + h2] = e4m3x4(clamp448(bf16_lo(x0) * inv), clamp448(bf16_hi(x0) * inv),
                                   clamp448(bf16_lo(x1) * inv), clamp448(bf16_hi(x1) * inv));
        }
    uint8_t* out = a.codes + ((size_t)blk * a.heads + head) * ROWS * D + (size_t)r * D;
    if constexpr (DPT >= 16) {
#pragma unroll
        for (int c = 0; c < DPT / 16; ++c) {
            const int chunk = part * (DPT / 16) + c;
            const int phys = SWZ ? (chunk ^ ((r / RPB) % CPR)) : chunk;
            *(u32x4*)(out + phys * 16) = u32x4{w[4 * c], w[4 * c + 1], w[4 * c + 2], w[4 * c + 3]};
        }
    } else {
        static_assert(!SWZ || DPT >= 16, "swizzled blocks store whole chunks");
        *(u32x2*)(out + part * 8) = u32x2{w[0], w[1]};
    }
    if (t == 0) a.scales[(size_t)blk * a.heads + head] = scale;
}

}  // namespace

hipError_t launch_quant_e4m3(const void* const* src, const int32_t* end, int n_spans, int32_t tokens, int32_t heads,
                             int head_dim, int rows, uint8_t* codes, float* scales, hipStream_t s) {
    if (n_spans < 1 || n_spans > kMaxSeg || tokens <= 0 || heads <= 0) return hipErrorInvalidValue;
    QuantArgs a;
    for (int x = 0; x < kMaxSeg; ++x) {
        a.src[x] = x < n_spans ? src[x] : nullptr;
        a.end[x] = x < n_spans ? end[x] : tokens;
    }
    a.n_spans = n_spans;
    a.tokens = tokens;
    a.heads = heads;
    a.codes = codes;
    a.scales = scales;
    const int64_t blocks = (int64_t)(tokens + rows - 1) / rows * heads;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    if (head_dim == 128 && rows == 64)
        hipLaunchKernelGGL((quant_e4m3_kernel<128, 64, true>), dim3((uint32_t)blocks), dim3(kQThreads), 0, s, a);
    else if (head_dim == 128 && rows == 32)
        hipLaunchKernelGGL((quant_e4m3_kernel<128, 32, false>), dim3((uint32_t)blocks), dim3(kQThreads), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace wmk
