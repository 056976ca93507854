/*
 * Seeded synthetic input streams shared by the test/bench inputs of both the
 * GPU library and the CPU oracle.  This file holds no arithmetic of the
 * compression method itself: it only draws numbers.
 *
 * Generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random
 * Numbers: As Easy as 1, 2, 3", SC'11), a counter-based generator: output
 * block i is a pure function of (counter = i, key), so any element of any
 * stream can be produced independently and in parallel.
 *
 * Normals: Box-Muller in double precision from two 53-bit uniforms taken from
 * one 128-bit Philox block (two normals per block).
 * Student-t(3): Z / sqrt((Z1^2 + Z2^2 + Z3^2) / 3) from four normals.
 * Outputs are float32; conversion to the storage type happens in Python.
 */
#include <stdint.h>
#include <math.h>
#include <stddef.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void philox_round(uint32_t c[4], const uint32_t k[2]) {
    uint64_t p0 = (uint64_t)PHILOX_M0 * c[0];
    uint64_t p1 = (uint64_t)PHILOX_M1 * c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k[0];
    uint32_t n2 = hi0 ^ c[3] ^ k[1];
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
}

/* Philox4x32 with 10 rounds; the key is bumped by the Weyl constants between rounds. */
void synth_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
    uint32_t k[2] = {key_in[0], key_in[1]};
    for (int r = 0; r < 10; ++r) {
        if (r) { k[0] += PHILOX_W0; k[1] += PHILOX_W1; }
        philox_round(c, k);
    }
    out[0] = c[0]; out[1] = c[1]; out[2] = c[2]; out[3] = c[3];
}

/* splitmix64 finaliser (Steele, Lea, Flood 2014), used to fold stream ids into a key. */
static inline uint64_t splitmix64(uint64_t x) {
    uint64_t z = x + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

uint64_t synth_stream_key(uint64_t seed, uint64_t cfg, uint64_t tensor, uint64_t layer, uint64_t step) {
    uint64_t s = splitmix64(seed);
    s = splitmix64(s ^ cfg);
    s = splitmix64(s ^ (tensor + 0x100));
    s = splitmix64(s ^ (layer + 0x10000));
    s = splitmix64(s ^ (step + 0x1000000));
    return s;
}

static inline void block(uint64_t key, uint64_t idx, uint32_t lane, uint32_t out[4]) {
    uint32_t c[4] = {(uint32_t)idx, (uint32_t)(idx >> 32), lane, 0x5eedu};
    uint32_t k[2] = {(uint32_t)key, (uint32_t)(key >> 32)};
    synth_philox4x32_10(c, k, out);
}

static inline double u53(uint32_t hi, uint32_t lo) {
    uint64_t v = (((uint64_t)hi << 32) | lo) >> 11;        /* 53 random bits */
    return ((double)v + 0.5) * (1.0 / 9007199254740992.0);  /* open interval (0, 1) */
}

/* Both normals of pair p of stream `key` (Box-Muller on one Philox block). */
static inline void normal_pair(uint64_t key, uint64_t p, double *z0, double *z1) {
    uint32_t r[4];
    block(key, p, 0u, r);
    double u1 = u53(r[0], r[1]);
    double u2 = u53(r[2], r[3]);
    double rad = sqrt(-2.0 * log(u1));
    double ang = 6.283185307179586476925286766559 * u2;
    *z0 = rad * cos(ang);
    *z1 = rad * sin(ang);
}

/* out[i] = (float)(sigma * Z_{first+i}), i in [0, n): element e of the stream is
 * the cosine (e even) or sine (e odd) branch of pair e/2. */
void synth_normal_f32(uint64_t key, uint64_t first, int64_t n, double sigma, float *out) {
    if (n <= 0) return;
    int64_t p0 = (int64_t)(first >> 1), p1 = (int64_t)((first + (uint64_t)n + 1) >> 1);
    #pragma omp parallel for schedule(static)
    for (int64_t p = p0; p < p1; ++p) {
        double z[2];
        normal_pair(key, (uint64_t)p, &z[0], &z[1]);
        for (int j = 0; j < 2; ++j) {
            int64_t e = 2 * p + j - (int64_t)first;
            if (e >= 0 && e < n) out[e] = (float)(sigma * z[j]);
        }
    }
}

/* Student-t with 3 degrees of freedom, element e from normals 4e..4e+3:
 * Z / sqrt((Z1^2 + Z2^2 + Z3^2) / 3). */
void synth_student_t3_f32(uint64_t key, uint64_t first, int64_t n, double sigma, float *out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint64_t e = first + (uint64_t)i;
        double z, z1, z2, z3;
        normal_pair(key, 2 * e, &z, &z1);
        normal_pair(key, 2 * e + 1, &z2, &z3);
        out[i] = (float)(sigma * z / sqrt((z1 * z1 + z2 * z2 + z3 * z3) / 3.0));
    }
}

/* Uniform doubles in (0, 1) from counter lane 1 (independent of the normal lane). */
void synth_uniform_f64(uint64_t key, uint64_t first, int64_t n, double *out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint32_t r[4];
        block(key, first + (uint64_t)i, 1u, r);
        out[i] = u53(r[0], r[1]);
    }
}
