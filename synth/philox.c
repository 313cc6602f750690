/*
 * Seeded synthetic inputs for tests and benchmarks (CPU side).
 *
 * Philox4x32-10 from Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers:
 * As Easy as 1, 2, 3" (SC'11): a 4x32-bit counter is run through ten rounds
 * of two 32x32->64 multiplies with xor mixing, the 2x32-bit key being bumped
 * by the Weyl constants between rounds.
 *
 * An element with flat index idx of tensor kind `kind` under the stream key
 * (seed, chunk, layer, step) takes counter
 *     (idx & 0xffffffff, idx >> 32, chunk, kind | step << 8 | layer << 16)
 * and key (seed & 0xffffffff, seed >> 32).  Twelve bytes of the first three
 * output words are summed (Irwin-Hall with twelve uniform bytes); the value
 * is (sum - 1530) / 256, exact in fp32 (mean 0, variance 65535/65536, range
 * +-5.977).  bf16 outputs are that fp32 value rounded to nearest-even.
 *
 * This file holds no attention arithmetic; it only draws numbers.  Its GPU
 * twin (gen.hip) must produce identical bits.
 */
#include <stdint.h>
#include <stddef.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void synth_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
        k0 += PHILOX_W0; k1 += PHILOX_W1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static inline int32_t byte_sum3(uint32_t a, uint32_t b, uint32_t c) {
    int32_t s = 0;
    for (int i = 0; i < 4; ++i) {
        s += (int32_t)((a >> (8 * i)) & 0xffu);
        s += (int32_t)((b >> (8 * i)) & 0xffu);
        s += (int32_t)((c >> (8 * i)) & 0xffu);
    }
    return s;
}

static inline float value_at(uint64_t seed, uint32_t chunk, uint32_t tag, uint64_t idx) {
    uint32_t ctr[4] = {(uint32_t)idx, (uint32_t)(idx >> 32), chunk, tag};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t o[4];
    synth_philox4x32_10(ctr, key, o);
    return (float)(byte_sum3(o[0], o[1], o[2]) - 1530) / 256.0f;
}

static inline uint16_t f32_to_bf16_rne(float x) {
    union { float f; uint32_t u; } v;
    v.f = x;
    uint32_t bias = 0x7fffu + ((v.u >> 16) & 1u);
    return (uint16_t)((v.u + bias) >> 16);
}

static uint32_t make_tag(uint32_t kind, uint32_t step, uint32_t layer) {
    return (kind & 0xffu) | ((step & 0xffu) << 8) | (layer << 16);
}

void synth_fill_f32(float* dst, uint64_t start, uint64_t n, uint64_t seed, uint32_t chunk,
                    uint32_t layer, uint32_t step, uint32_t kind) {
    uint32_t tag = make_tag(kind, step, layer);
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) dst[i] = value_at(seed, chunk, tag, start + (uint64_t)i);
}

void synth_fill_bf16(uint16_t* dst, uint64_t start, uint64_t n, uint64_t seed, uint32_t chunk,
                     uint32_t layer, uint32_t step, uint32_t kind) {
    uint32_t tag = make_tag(kind, step, layer);
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i)
        dst[i] = f32_to_bf16_rne(value_at(seed, chunk, tag, start + (uint64_t)i));
}
