/*
 * Seeded synthetic inputs for the quantized MoE layer.
 *
 * This module draws random numbers and nothing else: it holds none of the
 * layer's arithmetic (no quantisation, no dot products, no routing).  Both the
 * CPU oracle's tests and the GPU path take their inputs from here.
 *
 * Generator: splitmix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014).  Its i-th output for a starting state s is
 * mix(s + (i + 1) * 0x9E3779B97F4A7C15), so any element of any tensor can be
 * drawn independently of every other one (counter-based).  Each tensor gets
 * its own starting state key(seed, stream).
 *
 * Normals: Box-Muller in double precision from two 53-bit uniforms.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

static inline uint64_t sm_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static inline uint64_t sm_key(uint64_t seed, uint64_t stream) {
    return sm_mix(sm_mix(seed) ^ (stream * 0xD1B54A32D192ED03ull));
}

static inline uint64_t sm_draw(uint64_t key, uint64_t i) {
    return sm_mix(key + (i + 1) * 0x9E3779B97F4A7C15ull);
}

/* uniform double in (0, 1] from the top 53 bits */
static inline double u53_open0(uint64_t r) {
    return ((double)(r >> 11) + 1.0) * (1.0 / 9007199254740992.0);
}
/* uniform double in [0, 1) */
static inline double u53(uint64_t r) {
    return (double)(r >> 11) * (1.0 / 9007199254740992.0);
}

static inline double normal_at(uint64_t key, uint64_t i) {
    const double two_pi = 6.283185307179586476925286766559;
    double u1 = u53_open0(sm_draw(key, 2 * i));
    double u2 = u53(sm_draw(key, 2 * i + 1));
    return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

/* out[i] = (float)(scale * N(0,1)_i), i in [first, first + n) of the stream */
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n,
                      double scale, float* out) {
    uint64_t key = sm_key(seed, stream);
    for (uint64_t i = 0; i < n; ++i) out[i] = (float)(scale * normal_at(key, first + i));
}

/* out[i] = scale * |N(0,1)_i| in double (the caller rounds to its storage type) */
void synth_absnormal_f64(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n,
                         double scale, double* out) {
    uint64_t key = sm_key(seed, stream);
    for (uint64_t i = 0; i < n; ++i) out[i] = scale * fabs(normal_at(key, first + i));
}

/*
 * Integers uniform in [-127, 127]: each 64-bit draw gives four 16-bit slices u,
 * each mapped to ((u * 255) >> 16) - 127 (multiply-shift range reduction).
 * Element i of the stream uses slice i % 4 of draw i / 4.
 */
void synth_int8_sym127(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n, int8_t* out) {
    uint64_t key = sm_key(seed, stream);
    uint64_t i = 0;
    while (i < n) {
        uint64_t g = first + i;
        uint64_t r = sm_draw(key, g >> 2);
        for (unsigned s = (unsigned)(g & 3); s < 4 && i < n; ++s, ++i) {
            uint32_t u = (uint32_t)((r >> (16 * s)) & 0xFFFFu);
            out[i] = (int8_t)((int)((u * 255u) >> 16) - 127);
        }
    }
}

/*
 * Bytes whose two nibbles are independent and uniform in [0, 15]: byte i of the
 * stream is byte i % 8 of draw i / 8.
 */
void synth_nibble_bytes(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n, uint8_t* out) {
    uint64_t key = sm_key(seed, stream);
    uint64_t i = 0;
    while (i < n) {
        uint64_t g = first + i;
        uint64_t r = sm_draw(key, g >> 3);
        for (unsigned s = (unsigned)(g & 7); s < 8 && i < n; ++s, ++i)
            out[i] = (uint8_t)((r >> (8 * s)) & 0xFFu);
    }
}

/*
 * Interleave nblk block scales (2 bytes each) and payloads (pay bytes each)
 * into blocks of 2 + pay bytes: scale first, little-endian, then the payload.
 */
void synth_interleave_blocks(uint64_t nblk, const uint16_t* scale, const uint8_t* payload,
                             uint64_t pay, uint8_t* out) {
    for (uint64_t b = 0; b < nblk; ++b) {
        uint8_t* o = out + b * (2 + pay);
        o[0] = (uint8_t)(scale[b] & 0xFFu);
        o[1] = (uint8_t)(scale[b] >> 8);
        const uint8_t* p = payload + b * pay;
        for (uint64_t j = 0; j < pay; ++j) o[2 + j] = p[j];
    }
}
