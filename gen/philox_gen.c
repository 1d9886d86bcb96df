/*
 * Seeded synthetic input generator shared by the tests, the benchmark and the
 * smoke check.  It holds none of the MoE layer's arithmetic: it only turns
 * (seed, tensor id, flat element index) into normally distributed numbers and
 * stores them as fp32 or bf16.
 *
 * Generator: Philox-4x32-10, the counter-based generator of Salmon, Moraes,
 * Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11),
 * written from its published definition: 10 rounds of two 32x32->64-bit
 * multiplies with the multipliers 0xD2511F53 / 0xCD9E8D57 and a Weyl key
 * schedule with increments 0x9E3779B9 / 0xBB67AE85.
 *
 * Key   = (seed, tensor_id).
 * Counter = (j mod 2^32, j div 2^32, 0, 0) for the element pair j = i / 2.
 * The four 32-bit outputs form two 53-bit uniforms u1, u2 in (0, 1); the
 * Box-Muller transform gives z0 = r cos(2 pi u2) for element 2j and
 * z1 = r sin(2 pi u2) for element 2j + 1, with r = sqrt(-2 ln u1).
 * The value is z * stddev in fp64, rounded to nearest-even to fp32, and for
 * bf16 output rounded to nearest-even once more from that fp32 value.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static void philox_round(uint32_t c[4], const uint32_t k[2]) {
    uint64_t p0 = (uint64_t)PHILOX_M0 * c[0];
    uint64_t p1 = (uint64_t)PHILOX_M1 * c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k[0];
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c[3] ^ k[1];
    uint32_t n3 = lo0;
    c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
}

/* One Philox-4x32-10 block: out = philox(ctr, key). */
void gen_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k[2] = {key[0], key[1]};
    for (int r = 0; r < 10; ++r) {
        if (r) { k[0] += PHILOX_W0; k[1] += PHILOX_W1; }
        philox_round(c, k);
    }
    memcpy(out, c, sizeof(c));
}

static double u53(uint32_t hi, uint32_t lo) {
    /* 53 random bits mapped to the open interval (0, 1). */
    uint64_t bits = (((uint64_t)hi << 32) | lo) >> 11;
    return ((double)bits + 0.5) * (1.0 / 9007199254740992.0);
}

static void normal_pair(uint64_t j, uint32_t seed, uint32_t tensor_id, double *z0, double *z1) {
    uint32_t ctr[4] = {(uint32_t)j, (uint32_t)(j >> 32), 0u, 0u};
    uint32_t key[2] = {seed, tensor_id};
    uint32_t r[4];
    gen_philox4x32_10(ctr, key, r);
    double u1 = u53(r[0], r[1]);
    double u2 = u53(r[2], r[3]);
    double rad = sqrt(-2.0 * log(u1));
    double th = 6.283185307179586476925286766559 * u2;
    *z0 = rad * cos(th);
    *z1 = rad * sin(th);
}

static uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    /* inputs are finite: no NaN handling needed */
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* Elements [begin, begin + n) of the stream (seed, tensor_id), scaled by stddev.
 * dtype 0: fp32 into out (float*), dtype 1: bf16 bits into out (uint16_t*). */
void gen_normal(uint32_t seed, uint32_t tensor_id, uint64_t begin, uint64_t n,
                double stddev, int dtype, void *out) {
    if (n == 0) return;
    #pragma omp parallel for schedule(static)
    for (int64_t q = (int64_t)(begin / 2); q <= (int64_t)((begin + n - 1) / 2); ++q) {
        double z[2];
        normal_pair((uint64_t)q, seed, tensor_id, &z[0], &z[1]);
        for (int s = 0; s < 2; ++s) {
            uint64_t i = 2 * (uint64_t)q + (uint64_t)s;
            if (i < begin || i >= begin + n) continue;
            float f = (float)(z[s] * stddev);
            if (dtype == 0) ((float *)out)[i - begin] = f;
            else ((uint16_t *)out)[i - begin] = f32_to_bf16_rne(f);
        }
    }
}

/* fp32 -> bf16 (RNE) for host-side conversion of generated or hand-built data. */
void gen_f32_to_bf16(const float *in, uint16_t *out, uint64_t n) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = f32_to_bf16_rne(in[i]);
}
