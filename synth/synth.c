/*
 * Seeded synthetic inputs, shared as data by the CPU oracle and the HIP path.
 *
 * This file holds no arithmetic of the denoising method: it only turns a
 * 64-bit tensor key and an element index into a reproducible number.
 *
 * Generator: Philox4x32-10, the counter-based generator published by Salmon,
 * Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3"
 * (SC'11): ten rounds of two 32x32->64 multiplies with the constants
 * 0xD2511F53 / 0xCD9E8D57 and a Weyl key schedule 0x9E3779B9 / 0xBB67AE85.
 * Element i uses the counter (lo32(i), hi32(i), stream, 0) under the key.
 *
 * Distributions (all integer-exact up to one correctly rounded fp32 multiply,
 * so any IEEE implementation reproduces them bit for bit):
 *   normal:  the 128 output bits are read as eight uint16 u_j; the centred
 *            sum z = 2*sum(u_j) - 8*65535 (an even integer, |z| < 2^20) is an
 *            Irwin-Hall(8) variate; value = float(z) * c with
 *            c = sigma / (2*sqrt(8*(65536^2-1)/12)) rounded to fp32, so the
 *            value has mean 0 and standard deviation sigma (tails bounded at
 *            +-4.9 sigma).
 *   uniform: value = (w0 >> 8) * 2^-23 - 1, exactly representable, in [-1, 1).
 * Every value is then rounded to bfloat16 (round to nearest, ties to even),
 * so the same numbers can be handed to a bf16 kernel, an fp32 kernel and an
 * fp32/fp64 oracle without any of them seeing a different input.
 */
#include <stdint.h>
#include <stddef.h>

static inline void mulhilo32(uint32_t a, uint32_t b, uint32_t *hi, uint32_t *lo) {
    uint64_t p = (uint64_t)a * (uint64_t)b;
    *hi = (uint32_t)(p >> 32);
    *lo = (uint32_t)p;
}

static inline void philox4x32_10(const uint32_t in[4], uint32_t k0, uint32_t k1, uint32_t out[4]) {
    uint32_t c0 = in[0], c1 = in[1], c2 = in[2], c3 = in[3];
    for (int r = 0; r < 10; ++r) {
        uint32_t hi0, lo0, hi1, lo1;
        mulhilo32(0xD2511F53u, c0, &hi0, &lo0);
        mulhilo32(0xCD9E8D57u, c2, &hi1, &lo1);
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static inline uint16_t f32_to_bf16_rne(float f) {
    union { float f; uint32_t u; } v;
    v.f = f;
    uint32_t u = v.u;
    if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

static inline float bf16_to_f32(uint16_t b) {
    union { uint32_t u; float f; } v;
    v.u = ((uint32_t)b) << 16;
    return v.f;
}

static inline float normal_value(uint32_t k0, uint32_t k1, uint32_t stream, uint64_t i, float c) {
    uint32_t ctr[4] = {(uint32_t)i, (uint32_t)(i >> 32), stream, 0u}, w[4];
    philox4x32_10(ctr, k0, k1, w);
    int32_t s = 0;
    for (int j = 0; j < 4; ++j) s += (int32_t)(w[j] & 0xFFFFu) + (int32_t)(w[j] >> 16);
    int32_t z = 2 * s - 8 * 65535;
    return (float)z * c; /* (float)z is exact: |z| < 2^24 */
}

static inline float uniform_pm1_value(uint32_t k0, uint32_t k1, uint32_t stream, uint64_t i) {
    uint32_t ctr[4] = {(uint32_t)i, (uint32_t)(i >> 32), stream, 0u}, w[4];
    philox4x32_10(ctr, k0, k1, w);
    return (float)(w[0] >> 8) * (1.0f / 8388608.0f) - 1.0f;
}

/* kind: 0 = normal(sigma via c), 1 = uniform[-1,1). out_bf16 and/or out_f32 may be NULL. */
void synth_fill(uint64_t key, uint32_t stream, int kind, float c, uint64_t n,
                uint16_t *out_bf16, float *out_f32) {
    uint32_t k0 = (uint32_t)key, k1 = (uint32_t)(key >> 32);
    long long nn = (long long)n;
#pragma omp parallel for schedule(static)
    for (long long i = 0; i < nn; ++i) {
        float v = (kind == 0) ? normal_value(k0, k1, stream, (uint64_t)i, c)
                              : uniform_pm1_value(k0, k1, stream, (uint64_t)i);
        uint16_t b = f32_to_bf16_rne(v);
        if (out_bf16) out_bf16[i] = b;
        if (out_f32) out_f32[i] = bf16_to_f32(b);
    }
}

/* Raw Philox words for the known-answer test of the generator itself. */
void synth_philox(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    philox4x32_10(ctr, key[0], key[1], out);
}

/* bf16 <-> fp32 helpers for callers that hold data in one form. */
void synth_bf16_to_f32(const uint16_t *in, float *out, uint64_t n) {
    long long nn = (long long)n;
#pragma omp parallel for schedule(static)
    for (long long i = 0; i < nn; ++i) out[i] = bf16_to_f32(in[i]);
}

void synth_f32_to_bf16(const float *in, uint16_t *out, uint64_t n) {
    long long nn = (long long)n;
#pragma omp parallel for schedule(static)
    for (long long i = 0; i < nn; ++i) out[i] = f32_to_bf16_rne(in[i]);
}

/* n doubles in [0, 1) with 53 random bits each (host-side scalars such as timesteps). */
void synth_uniform01_f64(uint64_t key, uint32_t stream, uint64_t n, double *out) {
    uint32_t k0 = (uint32_t)key, k1 = (uint32_t)(key >> 32);
    for (uint64_t i = 0; i < n; ++i) {
        uint32_t ctr[4] = {(uint32_t)i, (uint32_t)(i >> 32), stream, 0x5EEDu}, w[4];
        philox4x32_10(ctr, k0, k1, w);
        uint64_t x = (((uint64_t)w[0]) << 32 | w[1]) >> 11;
        out[i] = (double)x * (1.0 / 9007199254740992.0);
    }
}
