/*
 * synth.c - seeded synthetic inputs for the batch-1 decode step.
 *
 * This file holds no arithmetic of the decoder itself.  It only draws random
 * numbers and rounds them into the storage formats the decoder consumes
 * (bf16 weights, packed 4-bit codes, fp16 group scales, token ids).  Both the
 * CPU oracle and the GPU library receive the same bytes from here.
 *
 * Generator: SplitMix64 used as a counter-based stream.  Element i of a stream
 * keyed by `key` is mix(key + (i + 1) * 0x9E3779B97F4A7C15), which is exactly
 * the i-th output of SplitMix64 started from state `key` (Steele, Lea and
 * Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014).
 * Being counter-based, every element can be produced independently, so the
 * fills below are parallel and still deterministic.
 *
 * Normals: Box-Muller in double, one normal per pair of uniforms
 * (z = sqrt(-2 ln u1) cos(2 pi u2)), then scaled, rounded to fp32 and from
 * there to the storage format with round-to-nearest-even.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* i-th output of SplitMix64 seeded with `key` (i counts from 0). */
static inline uint64_t stream_at(uint64_t key, uint64_t i) {
    return mix64(key + (i + 1) * GOLDEN);
}

/* Uniform double in [0, 1) from the top 53 bits. */
static inline double u01(uint64_t r) { return (double)(r >> 11) * (1.0 / 9007199254740992.0); }

static inline uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* fp32 -> bf16, round to nearest even.  NaN stays NaN (quiet). */
static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = f32_bits(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

/* fp32 -> IEEE binary16, round to nearest even, with subnormals and overflow to inf. */
static inline uint16_t f32_to_f16_rne(float f) {
    uint32_t u = f32_bits(f);
    uint32_t sign = (u >> 16) & 0x8000u;
    uint32_t exp = (u >> 23) & 0xffu;
    uint32_t man = u & 0x7fffffu;
    if (exp == 0xffu) return (uint16_t)(sign | 0x7c00u | (man ? 0x200u : 0u));
    int e = (int)exp - 127 + 15;
    if (e >= 31) return (uint16_t)(sign | 0x7c00u);
    if (e <= 0) {
        /* subnormal (or zero) in fp16: value = man_full * 2^(exp-150); unit = 2^-24 */
        if (e < -10) return (uint16_t)sign;
        uint32_t full = man | 0x800000u;
        int shift = 14 - e; /* 2^(exp-127-23) / 2^-24 = 2^(e - 15 + 24 - 23 ... ) */
        uint32_t q = full >> shift;
        uint32_t rem = full & ((1u << shift) - 1u);
        uint32_t half = 1u << (shift - 1);
        if (rem > half || (rem == half && (q & 1u))) q++;
        return (uint16_t)(sign | q);
    }
    uint32_t q = ((uint32_t)e << 10) | (man >> 13);
    uint32_t rem = man & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (q & 1u))) q++; /* carry may bump exponent: correct */
    return (uint16_t)(sign | q);
}

static inline double normal_at(uint64_t key, uint64_t i) {
    double a = u01(stream_at(key, 2 * i));
    double b = u01(stream_at(key, 2 * i + 1));
    double u1 = 1.0 - a; /* (0, 1] so log is finite */
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * b);
}

/* FNV-1a over the name, folded with the layer index and the seed, then mixed. */
uint64_t synth_key(uint64_t seed, int32_t layer, const char* name) {
    uint64_t h = 0xcbf29ce484222325ULL;
    for (const unsigned char* p = (const unsigned char*)name; *p; ++p) {
        h ^= *p;
        h *= 0x100000001b3ULL;
    }
    h ^= (uint64_t)(uint32_t)layer * 0xD6E8FEB86659FD93ULL;
    return mix64(seed ^ mix64(h));
}

/* bf16 values drawn from N(mean, std). */
void synth_fill_bf16_normal(uint16_t* out, int64_t n, uint64_t key, double mean, double std) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = f32_to_bf16_rne((float)(mean + std * normal_at(key, (uint64_t)i)));
}

/* bf16 constant (e.g. norm gains of 1.0). */
void synth_fill_bf16_const(uint16_t* out, int64_t n, float v) {
    uint16_t b = f32_to_bf16_rne(v);
    for (int64_t i = 0; i < n; ++i) out[i] = b;
}

/* fp16 values |N(0, std)|, rounded to nearest even (subnormals kept). */
void synth_fill_f16_absnormal(uint16_t* out, int64_t n, uint64_t key, double std) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = f32_to_f16_rne((float)fabs(std * normal_at(key, (uint64_t)i)));
}

/* Bytes whose two 4-bit halves are independent and uniform over 0..15. */
void synth_fill_u8_uniform(uint8_t* out, int64_t n, uint64_t key) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)(stream_at(key, (uint64_t)i) >> 56);
}

/* Integers uniform in [0, hi) by the multiply-high reduction of 32 random bits. */
void synth_fill_i32_uniform(int32_t* out, int64_t n, uint64_t key, int32_t hi) {
    for (int64_t i = 0; i < n; ++i) {
        uint64_t r = stream_at(key, (uint64_t)i) >> 32;
        out[i] = (int32_t)((r * (uint64_t)(uint32_t)hi) >> 32);
    }
}

/* Exposed for the generator's own tests. */
uint64_t synth_stream_at(uint64_t key, uint64_t i) { return stream_at(key, i); }
uint16_t synth_f32_to_bf16(float f) { return f32_to_bf16_rne(f); }
uint16_t synth_f32_to_f16(float f) { return f32_to_f16_rne(f); }
