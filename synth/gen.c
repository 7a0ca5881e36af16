/*
 * Seeded synthetic inputs for the MoE layer: counter-based, so any slice of
 * any tensor (one expert's weights, one token's row) can be regenerated on
 * its own without producing the rest.
 *
 * This file holds no step of the layer's arithmetic.  It only draws numbers:
 *   - SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 *     generators", OOPSLA 2014) used as a counter hash: the n-th 64-bit word
 *     of stream (seed, stream) is mix64(key + (n + 1) * GAMMA), where
 *     key = mix64(seed * GAMMA + stream) and mix64 is SplitMix64's finaliser.
 *   - Box and Muller (1958): two uniforms u1 in (0,1], u2 in [0,1) give
 *     z0 = r cos(2 pi u2), z1 = r sin(2 pi u2), r = sqrt(-2 ln u1).
 *     Element 2p of a stream takes z0 of pair p, element 2p+1 takes z1.
 *   - Each N(0,1) draw is scaled by sigma in double and rounded once to
 *     bfloat16, round-to-nearest-even (via a round-to-odd float step, which
 *     makes the two-step rounding exact).
 *   - A seeded permutation (Fisher-Yates driven by the same counter hash)
 *     for the per-expert Zipf ranks.
 *   - Synthetic 8-bit weight codes in the OCP FP8 E4M3 layout (sign, 4-bit
 *     exponent field, 3-bit mantissa field) drawn directly as bit fields, and
 *     uniform floats for their per-row scales.  Nothing is rounded or
 *     encoded: the codes are drawn, not produced from real values.
 *
 * Built with gcc; OpenMP splits the element range across host threads.  The
 * result does not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
    return mix64(seed * GAMMA + stream);
}

/* n-th 64-bit word of a stream (n counts from 0). */
static inline uint64_t word_at(uint64_t key, uint64_t n) {
    return mix64(key + (n + 1) * GAMMA);
}

uint64_t synth_word(uint64_t seed, uint64_t stream, uint64_t n) {
    return word_at(stream_key(seed, stream), n);
}

/* Round a double to bfloat16, nearest-even.  First to float with
 * round-to-odd (truncate toward zero, then force the last bit to 1 when
 * anything was dropped), then float -> bf16 nearest-even; with 16 spare
 * bits the second rounding sees an exact sticky bit, so the pair equals a
 * single correct rounding.  Infinities and NaN are not produced here. */
uint16_t synth_bf16_from_double(double v) {
    float f = (float)v;                       /* nearest-even */
    if ((double)f != v) {
        /* step back toward zero if the nearest float overshot |v| */
        if (fabs((double)f) > fabs(v)) f = nextafterf(f, 0.0f);
        uint32_t b;
        memcpy(&b, &f, 4);
        b |= 1u;                              /* sticky: round to odd */
        memcpy(&f, &b, 4);
    }
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

static inline void normal_pair(uint64_t key, uint64_t p, double* z0, double* z1) {
    uint64_t a = word_at(key, 2 * p);
    uint64_t b = word_at(key, 2 * p + 1);
    double u1 = ((double)(a >> 11) + 1.0) * 0x1.0p-53;   /* (0, 1] */
    double u2 = (double)(b >> 11) * 0x1.0p-53;           /* [0, 1) */
    double r = sqrt(-2.0 * log(u1));
    double th = 6.283185307179586476925286766559 * u2;
    *z0 = r * cos(th);
    *z1 = r * sin(th);
}

/* out[i] = bf16(sigma * N_{offset+i}) for i in [0, n), N_j the j-th normal
 * draw of stream (seed, stream). */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t offset,
                       uint64_t n, double sigma, uint16_t* out) {
    const uint64_t key = stream_key(seed, stream);
    const uint64_t p0 = offset >> 1;
    const uint64_t p1 = (offset + n + 1) >> 1;            /* exclusive */
#pragma omp parallel for schedule(static)
    for (int64_t pp = (int64_t)p0; pp < (int64_t)p1; ++pp) {
        double z0, z1;
        normal_pair(key, (uint64_t)pp, &z0, &z1);
        uint64_t e0 = 2 * (uint64_t)pp, e1 = e0 + 1;
        if (e0 >= offset && e0 < offset + n) out[e0 - offset] = synth_bf16_from_double(sigma * z0);
        if (e1 >= offset && e1 < offset + n) out[e1 - offset] = synth_bf16_from_double(sigma * z1);
    }
}

/* Same draws in double, unrounded (for tests of the draw itself). */
void synth_normal_f64(uint64_t seed, uint64_t stream, uint64_t offset,
                      uint64_t n, double* out) {
    const uint64_t key = stream_key(seed, stream);
    for (uint64_t i = 0; i < n; ++i) {
        uint64_t e = offset + i;
        double z0, z1;
        normal_pair(key, e >> 1, &z0, &z1);
        out[i] = (e & 1) ? z1 : z0;
    }
}

/* perm[0..n) = a seeded permutation of 1..n (Fisher-Yates, the j-th swap
 * index drawn from word j of the stream by a 128-bit multiply-high). */
void synth_permutation(uint64_t seed, uint64_t stream, int32_t n, int32_t* perm) {
    const uint64_t key = stream_key(seed, stream);
    for (int32_t i = 0; i < n; ++i) perm[i] = i + 1;
    for (int32_t i = n - 1; i > 0; --i) {
        uint64_t w = word_at(key, (uint64_t)(n - 1 - i));
        uint32_t j = (uint32_t)(((unsigned __int128)w * (uint64_t)(i + 1)) >> 64);
        int32_t t = perm[i];
        perm[i] = perm[j];
        perm[j] = t;
    }
}

/* Code n of an 8-bit weight stream, from word n: sign = bit 0; exponent field
 * 14 - g, g = the number of leading zeros of the 14-bit field (bits 8..21)
 * (so field 14 has probability 1/2, 13 probability 1/4, ... like values
 * scaled so that the largest sit near the top of the range); mantissa field
 * = bits 1..3.  The largest exponent field (15) is never drawn, so no code is
 * NaN. */
void synth_fp8_codes(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n, uint8_t* out) {
    const uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) {
        const uint64_t w = word_at(key, offset + (uint64_t)i);
        const uint32_t field = (uint32_t)((w >> 8) & 0x3FFFu);        /* 14 bits */
        int g = 0;
        while (g < 14 && !(field & (0x2000u >> g))) ++g;
        const uint32_t e = 14u - (uint32_t)g;
        const uint32_t m = (uint32_t)((w >> 1) & 7u);
        out[i] = (uint8_t)(((w & 1u) << 7) | (e << 3) | m);
    }
}

/* Uniform floats in [lo, hi): the top 24 bits of word n as a fraction u,
 * then lo + (hi - lo) * u in float. */
void synth_uniform_f32(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n, float lo,
                       float hi, float* out) {
    const uint64_t key = stream_key(seed, stream);
    for (uint64_t i = 0; i < n; ++i) {
        const float u = (float)(word_at(key, offset + i) >> 40) * (1.0f / 16777216.0f);
        out[i] = lo + (hi - lo) * u;
    }
}
