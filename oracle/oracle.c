/*
 * CPU oracle for the quantized mixture-of-experts expert FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file; only the tests, the smoke check and the CPU baseline of the
 * benchmark do.  It shares no code, header, table or helper with the HIP path.
 *
 * It is the plain definition of what the layer computes, written out in scalar
 * C with no blocking, fusion or reordering.  Sources (titles of the pages):
 *   [Q8] "Q8 0 support" (Strata pull request 255), section "GPU expert kernels":
 *        Q8_0 expert blocks of 32 ("qk 32"), the Q8_0 x Q8_1 block dot, the
 *        grouped gate/up/down expert path; section "Verified against an oracle":
 *        Strata's GPU experts quantise activations to Q8_1.
 *   [KQ] same page, the K-quant follow-up commit: the block sum uses the sum
 *        of the QUANTISED activations, not the float sum.
 *   [SY] "Sync upstream Strata v0.1.39 into Lanes" (pull request 24), the SYCL
 *        port commits: Q8_1 activation bytes match only with a correctly
 *        rounded fp32 divide; per-token top-k routing over the experts.
 *   [Q5] same page, the K-quant follow-up commit: Q5_1 experts (llama.cpp's
 *        Q5_1 blocks), whose min term multiplies the sum of the QUANTISED
 *        activations of the Q8_1 block (the ggml CPU convention), not the
 *        float sum of the activations.
 *   [QK] same commit: Q4_K and Q5_K experts, whose dots are llama.cpp's q4_K /
 *        q5_K x q8_1 (the min term on the sum of the quantised activations of
 *        each Q8_1 block).
 *   [Q3] edge0-strata README, section "Changes from upstream Strata": Q3_K
 *        latent experts.  The pages name the format only; its block is read as
 *        llama.cpp's Q3_K (the ggml that the same README builds against), and
 *        its dot against Q8_1 as the block's two 16-element halves, each with
 *        its signed sub-block scale, times d * d_a (no min term).
 *   [NV] edge0-strata README, section "Changes from upstream Strata": NVFP4
 *        latent experts.  The pages name the format only; it is read as its
 *        published definition (FP4 E2M1 elements, one FP8 E4M3 scale per 16
 *        consecutive elements, one fp32 scale per tensor), and its dot against
 *        Q8_1 as each 16-element half's integer sum of 2 * e2m1(code) * q_a
 *        times that half's scale / 2, times d_a, times the tensor scale.
 *   [E0] edge0-strata README, section "Changes from upstream Strata":
 *        latent-MoE with dense D/U projections in Q8 or Q4 into a 1280/1792-
 *        wide latent space, expert group labels, Q4_0 x Q8_1 rows (the Q4 of
 *        the D/U projections is read as Q4_0).
 * Where the pages leave a step open the reading taken is stated at that step.
 *
 * Precision: integer block sums are exact int32; per-block contributions
 * d_w * d_a * isum are exact in double; rows, router logits, softmax, SwiGLU
 * and the combine are evaluated in double and rounded to float where the layer
 * stores a float.  Build without fast-math and with -ffp-contract=off.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_Q8_0 8
#define ORC_Q4_0 2
#define ORC_Q5_1 7
#define ORC_Q4_K 12
#define ORC_Q5_K 13
#define ORC_Q3_K 11
#define ORC_NVFP4 40
#define ORC_QK 32
#define ORC_Q8_1_BYTES 36

typedef struct {
    int hidden, n_experts, top_k, n_ff, latent;
    int expert_fmt;           /* ORC_Q8_0, ORC_Q4_0, ORC_Q5_1, ORC_Q4_K, ORC_Q5_K, ORC_Q3_K or ORC_NVFP4 */
    int n_groups, topk_groups;/* 0 = no group limit */
    int dense_fmt;            /* D/U: ORC_Q8_0 or ORC_Q4_0 */
} orc_desc;

/* Optional per-step outputs, indexed by position i in the token list. */
typedef struct {
    double*  logits;   /* [n][E]                      */
    int32_t* ids;      /* [n][k]                      */
    float*   weights;  /* [n][k]                      */
    uint8_t* xq;       /* [n][H/32][36]   Q8_1(x)     */
    float*   z;        /* [n][L]          latent only */
    uint8_t* zq;       /* [n][L/32][36]   latent only */
    float*   h;        /* [n][k][F]                   */
    uint8_t* hq;       /* [n][k][F/32][36]            */
    float*   y;        /* [n][k][Kout]                */
    float*   ylat;     /* [n][L]          latent only */
    uint8_t* ylq;      /* [n][L/32][36]   latent only */
    int32_t* isum_gu;  /* [n][k][2F][Kin/32]  gate rows then up rows */
    int32_t* isum_dn;  /* [n][k][Kout][F/32]          */
    int32_t* isum_d;   /* [n][L][H/32]    latent only */
    int32_t* isum_u;   /* [n][H][L/32]    latent only */
} orc_taps;

/*
 * Optional given intermediates, indexed like the taps (NULL = the oracle's
 * own).  Where several results are correct (a routing near-tie, a Q8_1 code
 * that a float computed in another order rounds to the other side of a .5
 * boundary), a check evaluates the oracle downstream of the result actually
 * taken: the given experts replace the top-k selection (their weights are
 * still the softmax over their logits), and a given Q8_1 vector replaces the
 * quantisation of z, of h or of y_lat.  Everything else is computed as usual.
 */
typedef struct {
    const int32_t* ids;   /* [n][k]                                    */
    const uint8_t* zq;    /* [n][L/32][36]     expert input (latent)   */
    const uint8_t* hq;    /* [n][k][F/32][36]  down projection input   */
    const uint8_t* ylq;   /* [n][L/32][36]     U input (latent)        */
} orc_given;

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16                                                         */
/* ------------------------------------------------------------------------ */

/* Exact value of a binary16 bit pattern (subnormals included). */
double orc_f16_decode(uint16_t h) {
    int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(1024 + m), e - 25);
    return sign ? -v : v;
}

/*
 * Round a double to binary16, to nearest with ties to even, in one step.
 * The bit patterns of finite binary16 values are monotonic in magnitude, so a
 * magnitude a is written as n quanta of its binade (quantum 2^-24 below 2^-14,
 * 2^(E-10) in binade [2^E, 2^(E+1))), n is rounded with rint (ties to even in
 * the default rounding mode) and the pattern is rebuilt; a carry out of the
 * mantissa lands in the next exponent, and past 65504 on infinity.
 */
uint16_t orc_f16_encode(double v) {
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v)) return 0x7E00;
    if (a == 0.0) return sign;
    if (a >= 65520.0) return sign | 0x7C00;
    if (a < ldexp(1.0, -14)) {
        double n = rint(ldexp(a, 24));          /* exact scaling */
        return sign | (uint16_t)n;               /* n <= 1024; 1024 is 2^-14 */
    }
    int ex;
    frexp(a, &ex);                               /* a = f * 2^ex, f in [0.5, 1) */
    int E = ex - 1;                              /* a in [2^E, 2^(E+1)) */
    double n = rint(ldexp(a, 10 - E));           /* in [1024, 2048] */
    uint32_t bits = ((uint32_t)(E + 15) << 10) + (uint32_t)(n - 1024.0);
    return sign | (uint16_t)bits;
}

static inline uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static inline void wr16(uint8_t* p, uint16_t v) { p[0] = (uint8_t)(v & 0xFF); p[1] = (uint8_t)(v >> 8); }

/* ------------------------------------------------------------------------ */
/* Q8_1 activation blocks [Q8], [KQ], [SY]                                   */
/* ------------------------------------------------------------------------ */

/*
 * Quantise 32 floats to one Q8_1 block: bytes 0-1 binary16 d, bytes 2-3
 * binary16 s, bytes 4-35 int8 q.
 *   amax = max |v|, d = amax / 127 (fp32, correctly rounded divide [SY]),
 *   q_j  = round-half-away-from-zero(v_j / d) (fp32 divide), 0 when d == 0,
 *   s    = d * sum_j q_j (fp32 product; the quantised sum [KQ]).
 * Readings: ties round away from zero (C roundf); q is taken from the fp32 d,
 * only its binary16 rounding is stored; "d == 0" covers amax == 0 and an amax
 * so small that amax / 127 underflows.
 */
void orc_quantize_q8_1_block(const float* v, uint8_t* out) {
    float amax = 0.0f;
    for (int j = 0; j < ORC_QK; ++j) {
        float a = fabsf(v[j]);
        if (a > amax) amax = a;
    }
    float d = amax / 127.0f;
    int sum = 0;
    for (int j = 0; j < ORC_QK; ++j) {
        int q = 0;
        if (d != 0.0f) q = (int)roundf(v[j] / d);
        out[4 + j] = (uint8_t)(int8_t)q;
        sum += q;
    }
    wr16(out, orc_f16_encode((double)d));
    float s = d * (float)sum;
    wr16(out + 2, orc_f16_encode((double)s));
}

/* n floats (n a multiple of 32) to n/32 Q8_1 blocks */
void orc_quantize_q8_1(const float* v, int n, uint8_t* out) {
    for (int b = 0; b < n / ORC_QK; ++b) orc_quantize_q8_1_block(v + b * ORC_QK, out + b * ORC_Q8_1_BYTES);
}

/* ------------------------------------------------------------------------ */
/* Weight blocks and block dots                                              */
/* ------------------------------------------------------------------------ */

/* Q8_0: binary16 d then 32 int8 q; weight value d * q [Q8]. */
int32_t orc_isum_q8_0(const uint8_t* w, const uint8_t* a) {
    int32_t s = 0;
    for (int j = 0; j < ORC_QK; ++j) s += (int32_t)(int8_t)w[2 + j] * (int32_t)(int8_t)a[4 + j];
    return s;
}

/*
 * Q4_0: binary16 d then 16 bytes; byte j holds element j in its low nibble and
 * element j + 16 in its high nibble; weight value d * (c - 8) [E0].
 * Reading: the standard nibble order (the pages call the formats llama.cpp's).
 */
int32_t orc_isum_q4_0(const uint8_t* w, const uint8_t* a) {
    int32_t s = 0;
    for (int j = 0; j < 16; ++j) {
        int lo = (w[2 + j] & 0x0F) - 8;
        int hi = (w[2 + j] >> 4) - 8;
        s += lo * (int32_t)(int8_t)a[4 + j];
        s += hi * (int32_t)(int8_t)a[4 + j + 16];
    }
    return s;
}

/*
 * Q5_1: binary16 d, binary16 m, a 32-bit little-endian qh, then 16 bytes.
 * Element j < 16 takes the low nibble of byte j and bit j of qh as its fifth
 * bit; element j + 16 the high nibble of byte j and bit j + 16 of qh.  The
 * weight value is d * q + m with q in [0, 31] [Q5].
 */
static inline uint32_t rd32(const uint8_t* p) {
    return (uint32_t)p[0] | (uint32_t)p[1] << 8 | (uint32_t)p[2] << 16 | (uint32_t)p[3] << 24;
}

int orc_q5_1_code(const uint8_t* w, int j) {
    uint32_t qh = rd32(w + 4);
    int nib = j < 16 ? (w[8 + j] & 0x0F) : (w[8 + j - 16] >> 4);
    return nib | (int)((qh >> j) & 1u) << 4;
}

/* integer part of the Q5_1 x Q8_1 block dot: sum q_w * q_a */
int32_t orc_isum_q5_1(const uint8_t* w, const uint8_t* a) {
    int32_t s = 0;
    for (int j = 0; j < ORC_QK; ++j) s += orc_q5_1_code(w, j) * (int32_t)(int8_t)a[4 + j];
    return s;
}

/*
 * Q4_K: super-blocks of 256 elements (8 sub-blocks of 32) in 144 bytes:
 * binary16 d, binary16 dmin, 12 bytes of 6-bit sub-block scales and mins, 128
 * nibble bytes.  Sub-block b < 4: scale = s[b] & 63, min = s[b + 4] & 63; b >= 4:
 * scale = (s[b + 4] & 15) | (s[b - 4] >> 6) << 4, min = (s[b + 4] >> 4) |
 * (s[b] >> 6) << 4.  Element i of sub-block b is byte 32 * (b / 2) + i of the
 * nibble bytes, its low nibble for even b and its high nibble for odd b.  The
 * value is d * scale * q - dmin * min [QK] (llama.cpp's Q4_K).
 */
void orc_q4_k_scale_min(const uint8_t* sb, int b, int* sc, int* mn) {
    const uint8_t* s = sb + 4;
    if (b < 4) {
        *sc = s[b] & 63;
        *mn = s[b + 4] & 63;
    } else {
        *sc = (s[b + 4] & 15) | (s[b - 4] >> 6) << 4;
        *mn = (s[b + 4] >> 4) | (s[b] >> 6) << 4;
    }
}

int orc_q4_k_code(const uint8_t* sb, int e) {
    int b = e / 32, i = e % 32;
    uint8_t v = sb[16 + 32 * (b / 2) + i];
    return b % 2 ? v >> 4 : v & 0x0F;
}

/* integer part of sub-block b against one Q8_1 block: sum q * q_a */
int32_t orc_isum_q4_k(const uint8_t* sb, int b, const uint8_t* a) {
    int32_t s = 0;
    for (int i = 0; i < ORC_QK; ++i) s += orc_q4_k_code(sb, 32 * b + i) * (int32_t)(int8_t)a[4 + i];
    return s;
}

/*
 * Q5_K: 176-byte super-blocks: binary16 d, binary16 dmin, the 12 scale bytes of
 * Q4_K, 32 bytes qh, 128 nibble bytes.  Element i of sub-block b takes its
 * nibble as in Q4_K (nibble byte 32 * (b / 2) + i) and as its fifth bit bit b of
 * qh byte i; the value is d * scale * q - dmin * min, q in [0, 31] [QK].
 */
int orc_q5_k_code(const uint8_t* sb, int e) {
    int b = e / 32, i = e % 32;
    uint8_t v = sb[48 + 32 * (b / 2) + i];
    int nib = b % 2 ? v >> 4 : v & 0x0F;
    return nib | ((sb[16 + i] >> b) & 1) << 4;
}

int32_t orc_isum_q5_k(const uint8_t* sb, int b, const uint8_t* a) {
    int32_t s = 0;
    for (int i = 0; i < ORC_QK; ++i) s += orc_q5_k_code(sb, 32 * b + i) * (int32_t)(int8_t)a[4 + i];
    return s;
}

/*
 * Q3_K: super-blocks of 256 elements in 110 bytes: 32 bytes hmask, 64 bytes
 * qs, 12 bytes of 6-bit sub-block scales, binary16 d [Q3].  Element e, with
 * half = e / 128, j = (e % 128) / 32 and l = e % 32, has its low two bits at
 * bits 2j, 2j + 1 of qs byte 32 * half + l and its high bit at bit 4 * half + j
 * of hmask byte l; its code is low + 4 * high - 4, in [-4, 3].  Sixteen
 * sub-blocks of 16 elements; sub-block i's scale is the 6-bit value with low
 * nibble s[i] & 15 (i < 8) or s[i - 8] >> 4 (i >= 8) and top two bits
 * (s[8 + i % 4] >> 2 * (i / 4)) & 3, minus 32.  The value is d * scale * code.
 */
int orc_q3_k_code(const uint8_t* sb, int e) {
    int half = e / 128, j = (e % 128) / 32, l = e % 32;
    int low = (sb[32 + 32 * half + l] >> (2 * j)) & 3;
    int high = (sb[l] >> (4 * half + j)) & 1;
    return low + 4 * high - 4;
}

int orc_q3_k_scale(const uint8_t* sb, int i) {
    const uint8_t* s = sb + 96;
    int lo = i < 8 ? s[i] & 15 : s[i - 8] >> 4;
    int hi = (s[8 + i % 4] >> (2 * (i / 4))) & 3;
    return (lo | hi << 4) - 32;
}

/* integer part of block b (sub-blocks 2b, 2b + 1) against one Q8_1 block:
 * the sum over the two halves of scale * sum(code * q_a) */
int32_t orc_isum_q3_k(const uint8_t* sb, int b, const uint8_t* a) {
    int32_t s = 0;
    for (int h = 0; h < 2; ++h) {
        int32_t t = 0;
        for (int i = 0; i < 16; ++i)
            t += orc_q3_k_code(sb, 32 * b + 16 * h + i) * (int32_t)(int8_t)a[4 + 16 * h + i];
        s += orc_q3_k_scale(sb, 2 * b + h) * t;
    }
    return s;
}

/*
 * NVFP4 [NV].  A code c (4 bits) is FP4 E2M1: bit 3 the sign, bits 2..1 the
 * exponent e (bias 1), bit 0 the mantissa m; e = 0 is subnormal, m * 0.5, else
 * (1 + m / 2) * 2^(e - 1).  A scale s (8 bits) is FP8 E4M3: bit 7 the sign,
 * bits 6..3 the exponent e (bias 7), bits 2..0 the mantissa m; e = 0 is
 * subnormal, m / 8 * 2^-6, else (1 + m / 8) * 2^(e - 7); 0x7F and 0xFF are NaN.
 * Canonical block of 32 elements (18 bytes): byte 0 the scale of elements
 * 0..15, byte 1 that of 16..31, then 16 code bytes, element 2i in the low
 * nibble and 2i + 1 in the high nibble of byte 2 + i.
 */
double orc_e2m1_decode(int c) {
    int e = (c >> 1) & 3, m = c & 1;
    double v = e == 0 ? 0.5 * m : (1.0 + 0.5 * m) * ldexp(1.0, e - 1);
    return (c & 8) ? -v : v;
}

double orc_e4m3_decode(int s) {
    int e = (s >> 3) & 15, m = s & 7;
    if (e == 15 && m == 7) return NAN;
    double v = e == 0 ? (m / 8.0) * ldexp(1.0, -6) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
    return (s & 0x80) ? -v : v;
}

int orc_nvfp4_code(const uint8_t* w, int j) {
    uint8_t b = w[2 + j / 2];
    return (j & 1) ? b >> 4 : b & 0x0F;
}

/* half h (elements 16h .. 16h + 15) of a block against a Q8_1 block: the sum of
 * 2 * e2m1(code) * q_a, an integer (2 * e2m1 is one of 0, 1, 2, 3, 4, 6, 8, 12,
 * signed) */
int32_t orc_isum_nvfp4_half(const uint8_t* w, const uint8_t* a, int h) {
    int32_t s = 0;
    for (int i = 0; i < 16; ++i) {
        int j = 16 * h + i;
        int v2 = (int)(2.0 * orc_e2m1_decode(orc_nvfp4_code(w, j)));
        s += v2 * (int32_t)(int8_t)a[4 + j];
    }
    return s;
}

static inline int kq_bytes(int fmt) { return fmt == ORC_Q5_K ? 176 : fmt == ORC_Q3_K ? 110 : 144; }
static inline int is_kq(int fmt) { return fmt == ORC_Q4_K || fmt == ORC_Q5_K || fmt == ORC_Q3_K; }

static inline int fmt_bytes(int fmt) {   /* per 32; Q4_K: 144 per 256 */
    return fmt == ORC_Q4_0 || fmt == ORC_NVFP4 ? 18 : fmt == ORC_Q5_1 ? 24 : 34;
}

/* Dequantised value of element j of a weight block, for the cross-check tests. */
double orc_dequant_weight(int fmt, const uint8_t* w, int j) {
    if (fmt == ORC_NVFP4)                          /* without the tensor scale */
        return orc_e4m3_decode(w[j / 16]) * orc_e2m1_decode(orc_nvfp4_code(w, j));
    double d = orc_f16_decode(rd16(w));
    if (fmt == ORC_Q8_0) return d * (double)(int8_t)w[2 + j];
    if (fmt == ORC_Q5_1) return d * (double)orc_q5_1_code(w, j) + orc_f16_decode(rd16(w + 2));
    if (fmt == ORC_Q3_K)                           /* w: the super-block, j < 256 */
        return orc_f16_decode(rd16(w + 108)) * orc_q3_k_scale(w, j / 16) * (double)orc_q3_k_code(w, j);
    if (fmt == ORC_Q4_K || fmt == ORC_Q5_K) {      /* w: the super-block, j < 256 */
        int sc, mn;
        orc_q4_k_scale_min(w, j / 32, &sc, &mn);
        int q = fmt == ORC_Q4_K ? orc_q4_k_code(w, j) : orc_q5_k_code(w, j);
        return d * sc * (double)q - orc_f16_decode(rd16(w + 2)) * mn;
    }
    int c = j < 16 ? (w[2 + j] & 0x0F) : (w[2 + j - 16] >> 4);
    return d * (double)(c - 8);
}

/*
 * One output of a quantised matrix-vector product:
 *   y = sum_b f16(d_w,b) * f16(d_a,b) * isum_b  (+ f16(m_w,b) * f16(s_a,b) for Q5_1)
 * Each term is exact in double (22-bit scale product times a 20-bit integer;
 * two binary16 values); a block's terms and then the blocks are added in order
 * in double and the sum rounded to float.  The Q5_1 min term takes s, the
 * Q8_1 block's stored d * sum(q) [Q5], [KQ].
 */
static double row_dot_d(int fmt, const uint8_t* row, const uint8_t* act, int nblk, int32_t* isum_tap);

float orc_row_dot(int fmt, const uint8_t* row, const uint8_t* act, int nblk, int32_t* isum_tap) {
    return (float)row_dot_d(fmt, row, act, nblk, isum_tap);
}

/*
 * NVFP4 [NV]: tensor_scale * sum_b d_a,b * sum_h e4m3(s_b,h) / 2 * isum_b,h,
 * each term exact in double, the blocks added in order, rounded to float once.
 * The tap of block b holds its two half sums as 16-bit halves (half 0 low).
 */
float orc_row_dot_nvfp4(const uint8_t* row, const uint8_t* act, int nblk, double tensor_scale,
                        int32_t* isum_tap) {
    return (float)(row_dot_d(ORC_NVFP4, row, act, nblk, isum_tap) * tensor_scale);
}

static double row_dot_d(int fmt, const uint8_t* row, const uint8_t* act, int nblk, int32_t* isum_tap) {
    double acc = 0.0;
    if (fmt == ORC_NVFP4) {
        for (int b = 0; b < nblk; ++b) {
            const uint8_t* w = row + (size_t)b * 18;
            const uint8_t* a = act + (size_t)b * ORC_Q8_1_BYTES;
            int32_t i0 = orc_isum_nvfp4_half(w, a, 0), i1 = orc_isum_nvfp4_half(w, a, 1);
            if (isum_tap) isum_tap[b] = (int32_t)(((uint32_t)i0 & 0xFFFFu) | ((uint32_t)i1 << 16));
            double da = orc_f16_decode(rd16(a));
            acc += da * (orc_e4m3_decode(w[0]) * 0.5 * (double)i0 + orc_e4m3_decode(w[1]) * 0.5 * (double)i1);
        }
        return acc;
    }
    if (fmt == ORC_Q3_K) {
        /* block b against Q8_1 block b: d * d_a * isum_b, exact in double [Q3] */
        for (int b = 0; b < nblk; ++b) {
            const uint8_t* sb = row + (size_t)(b / 8) * 110;
            const uint8_t* a = act + (size_t)b * ORC_Q8_1_BYTES;
            int32_t is = orc_isum_q3_k(sb, b % 8, a);
            if (isum_tap) isum_tap[b] = is;
            acc += orc_f16_decode(rd16(sb + 108)) * orc_f16_decode(rd16(a)) * (double)is;
        }
        return acc;
    }
    if (fmt == ORC_Q4_K || fmt == ORC_Q5_K) {
        /*
         * Sub-block b against Q8_1 block b: d * scale_b * d_a * isum_b minus
         * dmin * min_b * d_a * sum(q_a), the activation sum taken from the
         * codes (llama.cpp's q4_K / q5_K x q8_1); each term exact in double.
         */
        for (int b = 0; b < nblk; ++b) {
            const uint8_t* sb = row + (size_t)(b / 8) * kq_bytes(fmt);
            const uint8_t* a = act + (size_t)b * ORC_Q8_1_BYTES;
            int sc, mn;
            orc_q4_k_scale_min(sb, b % 8, &sc, &mn);
            int32_t is = fmt == ORC_Q4_K ? orc_isum_q4_k(sb, b % 8, a) : orc_isum_q5_k(sb, b % 8, a);
            int32_t qs = 0;
            for (int i = 0; i < ORC_QK; ++i) qs += (int8_t)a[4 + i];
            if (isum_tap) isum_tap[b] = is;
            double da = orc_f16_decode(rd16(a));
            double c = orc_f16_decode(rd16(sb)) * sc * da * (double)is;
            c -= orc_f16_decode(rd16(sb + 2)) * mn * da * (double)qs;
            acc += c;
        }
        return acc;
    }
    int bb = fmt_bytes(fmt);
    for (int b = 0; b < nblk; ++b) {
        const uint8_t* w = row + (size_t)b * bb;
        const uint8_t* a = act + (size_t)b * ORC_Q8_1_BYTES;
        int32_t is = fmt == ORC_Q8_0 ? orc_isum_q8_0(w, a)
                   : fmt == ORC_Q5_1 ? orc_isum_q5_1(w, a) : orc_isum_q4_0(w, a);
        if (isum_tap) isum_tap[b] = is;
        double c = orc_f16_decode(rd16(w)) * orc_f16_decode(rd16(a)) * (double)is;
        if (fmt == ORC_Q5_1) c += orc_f16_decode(rd16(w + 2)) * orc_f16_decode(rd16(a + 2));
        acc += c;
    }
    return acc;
}

/* rows outputs of a [rows][nblk] block matrix times a Q8_1 vector */
static size_t row_bytes(int fmt, int nblk) {
    return is_kq(fmt) ? (size_t)(nblk / 8) * kq_bytes(fmt) : (size_t)nblk * fmt_bytes(fmt);
}

void orc_matvec(int fmt, int rows, int nblk, const uint8_t* W, const uint8_t* act, float* y,
                int32_t* isum_tap) {
    size_t rb = row_bytes(fmt, nblk);
    for (int r = 0; r < rows; ++r)
        y[r] = orc_row_dot(fmt, W + r * rb, act, nblk, isum_tap ? isum_tap + (size_t)r * nblk : NULL);
}

/* ------------------------------------------------------------------------ */
/* Router [SY], [E0]                                                         */
/* ------------------------------------------------------------------------ */

/*
 * For one token: logits l_e = sum_i x_i W_r[e,i] (+ b_e) in double; with group
 * labels, the groups ranked by their largest logit and the experts outside the
 * best topk_groups groups dropped; the top_k experts by logit (exact ties go to
 * the lower expert or group id); weights = softmax over the chosen logits,
 * w_j = exp(l_j - l_max) / sum_i exp(l_i - l_max), rounded to float.
 * Readings: group score = largest member logit; softmax after top-k equals
 * softmax over all experts renormalised over the chosen ones.
 */
static void route_token(const orc_desc* d, const float* x, const float* Wr, const float* br,
                        const int32_t* groups, const int32_t* given_ids, int32_t* ids, float* w,
                        double* logits_out) {
    int H = d->hidden, E = d->n_experts, k = d->top_k;
    double* l = (double*)malloc(sizeof(double) * E);
    char* allowed = (char*)malloc(E);
    for (int e = 0; e < E; ++e) {
        double acc = 0.0;
        for (int i = 0; i < H; ++i) acc += (double)x[i] * (double)Wr[(size_t)e * H + i];
        if (br) acc += (double)br[e];
        l[e] = acc;
        allowed[e] = 1;
        if (logits_out) logits_out[e] = acc;
    }
    if (given_ids) {
        memcpy(ids, given_ids, sizeof(int32_t) * k);
    } else {
        if (d->n_groups > 0 && groups) {
            int G = d->n_groups;
            double* gs = (double*)malloc(sizeof(double) * G);
            char* gsel = (char*)calloc(G, 1);
            for (int g = 0; g < G; ++g) gs[g] = -INFINITY;
            for (int e = 0; e < E; ++e)
                if (l[e] > gs[groups[e]]) gs[groups[e]] = l[e];
            for (int n = 0; n < d->topk_groups; ++n) {
                int best = -1;
                for (int g = 0; g < G; ++g)
                    if (!gsel[g] && (best < 0 || gs[g] > gs[best])) best = g;
                gsel[best] = 1;
            }
            for (int e = 0; e < E; ++e) allowed[e] = gsel[groups[e]];
            free(gs);
            free(gsel);
        }
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (allowed[e] && (best < 0 || l[e] > l[best])) best = e;
            ids[j] = best;
            allowed[best] = 0;
        }
    }
    /* the largest chosen logit: ids[0] for the oracle's own selection */
    double m = l[ids[0]], s = 0.0;
    for (int j = 1; j < k; ++j)
        if (l[ids[j]] > m) m = l[ids[j]];
    for (int j = 0; j < k; ++j) s += exp(l[ids[j]] - m);
    for (int j = 0; j < k; ++j) w[j] = (float)(exp(l[ids[j]] - m) / s);
    free(l);
    free(allowed);
}

void orc_route_token(const orc_desc* d, const float* x, const float* Wr, const float* br,
                     const int32_t* groups, int32_t* ids, float* w, double* logits_out) {
    route_token(d, x, Wr, br, groups, NULL, ids, w, logits_out);
}

/* ------------------------------------------------------------------------ */
/* Expert FFN and the layer [Q8], [E0]                                       */
/* ------------------------------------------------------------------------ */

/* An NVFP4 expert's blob ends with a 256-byte tail: its tensor scales gate, up,
 * down (fp32, little-endian), then zero bytes [NV]. */
static size_t expert_bytes(const orc_desc* d) {
    int kin = d->latent ? d->latent : d->hidden;
    int kout = kin;
    return 2 * d->n_ff * row_bytes(d->expert_fmt, kin / ORC_QK) +
           (size_t)kout * row_bytes(d->expert_fmt, d->n_ff / ORC_QK) +
           (d->expert_fmt == ORC_NVFP4 ? 256 : 0);
}

static double rdf32(const uint8_t* p) {
    uint32_t u = (uint32_t)p[0] | (uint32_t)p[1] << 8 | (uint32_t)p[2] << 16 | (uint32_t)p[3] << 24;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

size_t orc_expert_bytes(const orc_desc* d) { return expert_bytes(d); }

/*
 * One expert on one quantised input aq (Kin/32 Q8_1 blocks):
 *   g = W_gate aq, u = W_up aq (float), h = silu(g) * u = g / (1 + e^-g) * u
 *   (double from the float g and u, rounded to float), hq = Q8_1(h) per 32,
 *   y = W_down hq (float).  SwiGLU with the gate first is the reading taken.
 */
static void expert_ffn(const orc_desc* d, const uint8_t* blob, const uint8_t* aq,
                       const uint8_t* given_hq, float* h, uint8_t* hq, float* y, int32_t* isum_gu,
                       int32_t* isum_dn) {
    int fmt = d->expert_fmt, F = d->n_ff;
    int kin = d->latent ? d->latent : d->hidden, kout = kin;
    int nbi = kin / ORC_QK, nbf = F / ORC_QK;
    size_t rbi = row_bytes(fmt, nbi);
    const uint8_t* gate = blob;
    const uint8_t* up = gate + (size_t)F * rbi;
    const uint8_t* down = up + (size_t)F * rbi;
    const int nv = fmt == ORC_NVFP4;
    size_t rbf = row_bytes(fmt, nbf);
    const uint8_t* ts = down + (size_t)kout * rbf;    /* NVFP4 tensor scales */
    for (int r = 0; r < F; ++r) {
        int32_t* tg = isum_gu ? isum_gu + (size_t)r * nbi : NULL;
        int32_t* tu = isum_gu ? isum_gu + (size_t)(F + r) * nbi : NULL;
        float g = nv ? orc_row_dot_nvfp4(gate + r * rbi, aq, nbi, rdf32(ts), tg)
                     : orc_row_dot(fmt, gate + r * rbi, aq, nbi, tg);
        float u = nv ? orc_row_dot_nvfp4(up + r * rbi, aq, nbi, rdf32(ts + 4), tu)
                     : orc_row_dot(fmt, up + r * rbi, aq, nbi, tu);
        double gd = (double)g;
        h[r] = (float)(gd / (1.0 + exp(-gd)) * (double)u);
    }
    if (given_hq)
        memcpy(hq, given_hq, (size_t)nbf * ORC_Q8_1_BYTES);
    else
        orc_quantize_q8_1(h, F, hq);
    if (nv) {
        for (int r = 0; r < kout; ++r)
            y[r] = orc_row_dot_nvfp4(down + r * rbf, hq, nbf, rdf32(ts + 8),
                                     isum_dn ? isum_dn + (size_t)r * nbf : NULL);
    } else {
        orc_matvec(fmt, kout, nbf, down, hq, y, isum_dn);
    }
}

void orc_expert_ffn(const orc_desc* d, const uint8_t* blob, const uint8_t* aq, float* h,
                    uint8_t* hq, float* y, int32_t* isum_gu, int32_t* isum_dn) {
    expert_ffn(d, blob, aq, NULL, h, hq, y, isum_gu, isum_dn);
}

typedef struct {
    const orc_desc* d;
    const float *x, *Wr, *br;
    const int32_t* groups;
    const uint8_t *experts, *D, *U;
    float* out;
    const orc_taps* taps;
    const orc_given* given;
    const int32_t* list;
    int n;
    int next;
    pthread_mutex_t mu;
} job_t;

#define TAP(ptr, stride) ((ptr) ? (ptr) + (size_t)i * (stride) : NULL)

static void run_token(job_t* J, int i) {
    const orc_desc* d = J->d;
    const orc_taps* tp = J->taps;
    const orc_given* gv = J->given;
    int t = J->list ? J->list[i] : i;
    int H = d->hidden, E = d->n_experts, k = d->top_k, F = d->n_ff, L = d->latent;
    int kin = L ? L : H, kout = kin;
    const float* x = J->x + (size_t)t * H;
    int32_t ids[512];
    float w[512];
    route_token(d, x, J->Wr, J->br, J->groups, gv && gv->ids ? gv->ids + (size_t)i * k : NULL,
                ids, w, tp ? TAP(tp->logits, E) : NULL);
    if (tp && tp->ids) memcpy(tp->ids + (size_t)i * k, ids, sizeof(int32_t) * k);
    if (tp && tp->weights) memcpy(tp->weights + (size_t)i * k, w, sizeof(float) * k);

    uint8_t* xq = (uint8_t*)malloc((size_t)(H / ORC_QK) * ORC_Q8_1_BYTES);
    orc_quantize_q8_1(x, H, xq);
    if (tp && tp->xq) memcpy(tp->xq + (size_t)i * (H / ORC_QK) * ORC_Q8_1_BYTES, xq, (size_t)(H / ORC_QK) * ORC_Q8_1_BYTES);

    const uint8_t* ain = xq;                  /* the experts' quantised input */
    uint8_t* zq = NULL;
    float* z = NULL;
    if (L) {                                   /* latent: z = D Q8_1(x), experts on Q8_1(z) */
        z = (float*)malloc(sizeof(float) * L);
        zq = (uint8_t*)malloc((size_t)(L / ORC_QK) * ORC_Q8_1_BYTES);
        orc_matvec(d->dense_fmt, L, H / ORC_QK, J->D, xq, z, tp ? TAP(tp->isum_d, (size_t)L * (H / ORC_QK)) : NULL);
        if (gv && gv->zq)
            memcpy(zq, gv->zq + (size_t)i * (L / ORC_QK) * ORC_Q8_1_BYTES, (size_t)(L / ORC_QK) * ORC_Q8_1_BYTES);
        else
            orc_quantize_q8_1(z, L, zq);
        if (tp && tp->z) memcpy(tp->z + (size_t)i * L, z, sizeof(float) * L);
        if (tp && tp->zq) memcpy(tp->zq + (size_t)i * (L / ORC_QK) * ORC_Q8_1_BYTES, zq, (size_t)(L / ORC_QK) * ORC_Q8_1_BYTES);
        ain = zq;
    }

    size_t eb = expert_bytes(d);
    float* h = (float*)malloc(sizeof(float) * F);
    uint8_t* hq = (uint8_t*)malloc((size_t)(F / ORC_QK) * ORC_Q8_1_BYTES);
    float* y = (float*)malloc(sizeof(float) * (size_t)k * kout);
    for (int j = 0; j < k; ++j) {
        size_t a = (size_t)i * k + j;
        expert_ffn(d, J->experts + (size_t)ids[j] * eb, ain,
                   gv && gv->hq ? gv->hq + a * (F / ORC_QK) * ORC_Q8_1_BYTES : NULL, h, hq,
                   y + (size_t)j * kout, tp && tp->isum_gu ? tp->isum_gu + a * 2 * F * (kin / ORC_QK) : NULL,
                   tp && tp->isum_dn ? tp->isum_dn + a * kout * (F / ORC_QK) : NULL);
        if (tp && tp->h) memcpy(tp->h + a * F, h, sizeof(float) * F);
        if (tp && tp->hq) memcpy(tp->hq + a * (F / ORC_QK) * ORC_Q8_1_BYTES, hq, (size_t)(F / ORC_QK) * ORC_Q8_1_BYTES);
        if (tp && tp->y) memcpy(tp->y + a * kout, y + (size_t)j * kout, sizeof(float) * kout);
    }
    /* combine: out = sum_j w_j y_j, in rank order, in double */
    float* comb = L ? (float*)malloc(sizeof(float) * L) : J->out + (size_t)i * H;
    for (int r = 0; r < kout; ++r) {
        double acc = 0.0;
        for (int j = 0; j < k; ++j) acc += (double)w[j] * (double)y[(size_t)j * kout + r];
        comb[r] = (float)acc;
    }
    if (L) {                                   /* out = U Q8_1(y_lat) */
        uint8_t* ylq = (uint8_t*)malloc((size_t)(L / ORC_QK) * ORC_Q8_1_BYTES);
        if (gv && gv->ylq)
            memcpy(ylq, gv->ylq + (size_t)i * (L / ORC_QK) * ORC_Q8_1_BYTES, (size_t)(L / ORC_QK) * ORC_Q8_1_BYTES);
        else
            orc_quantize_q8_1(comb, L, ylq);
        if (tp && tp->ylat) memcpy(tp->ylat + (size_t)i * L, comb, sizeof(float) * L);
        if (tp && tp->ylq) memcpy(tp->ylq + (size_t)i * (L / ORC_QK) * ORC_Q8_1_BYTES, ylq, (size_t)(L / ORC_QK) * ORC_Q8_1_BYTES);
        orc_matvec(d->dense_fmt, H, L / ORC_QK, J->U, ylq, J->out + (size_t)i * H,
                   tp ? TAP(tp->isum_u, (size_t)H * (L / ORC_QK)) : NULL);
        free(ylq);
        free(comb);
        free(z);
        free(zq);
    }
    free(xq);
    free(h);
    free(hq);
    free(y);
}

static void* worker(void* p) {
    job_t* J = (job_t*)p;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int i = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (i >= J->n) break;
        run_token(J, i);
    }
    return NULL;
}

/*
 * The layer for the tokens in list[0..n) (all of 0..n-1 when list is NULL):
 * route on x; Q8_1(x); latent: z = D Q8_1(x), experts on Q8_1(z); every chosen
 * expert's FFN; combine in rank order; latent: out = U Q8_1(y_lat).
 * out and every tap are indexed by position in the list.  Tokens are spread
 * over nthreads threads; each token is computed by one thread alone.
 * Returns 0, or -1 on a bad argument.
 */
int orc_layer_forward_given(const orc_desc* d, const float* x, const float* Wr,
                            const float* br, const int32_t* groups, const uint8_t* experts,
                            const uint8_t* D, const uint8_t* U, const int32_t* list, int n,
                            float* out, const orc_taps* taps, const orc_given* given,
                            int nthreads) {
    if (!d || !x || !Wr || !experts || !out || n < 0) return -1;
    if (d->top_k < 1 || d->top_k > d->n_experts || d->top_k > 512) return -1;
    if (d->latent && (!D || !U)) return -1;
    if (d->expert_fmt != ORC_Q8_0 && d->expert_fmt != ORC_Q4_0 && d->expert_fmt != ORC_Q5_1 &&
        d->expert_fmt != ORC_Q4_K && d->expert_fmt != ORC_Q5_K && d->expert_fmt != ORC_Q3_K &&
        d->expert_fmt != ORC_NVFP4)
        return -1;
    if (is_kq(d->expert_fmt) &&
        ((d->latent ? d->latent : d->hidden) % 256 || d->n_ff % 256))
        return -1;
    if (d->latent && d->dense_fmt != ORC_Q8_0 && d->dense_fmt != ORC_Q4_0) return -1;
    if (d->n_groups > 0) {                     /* every group holds E / n_groups experts */
        int G = d->n_groups;
        if (!groups || d->n_experts % G || d->topk_groups < 1 || d->topk_groups > G ||
            d->topk_groups * (d->n_experts / G) < d->top_k) return -1;
        int* cnt = (int*)calloc(G, sizeof(int));
        int bad = 0;
        for (int e = 0; e < d->n_experts; ++e) {
            if (groups[e] < 0 || groups[e] >= G) { bad = 1; break; }
            cnt[groups[e]]++;
        }
        for (int g = 0; g < G && !bad; ++g) bad = cnt[g] != d->n_experts / G;
        free(cnt);
        if (bad) return -1;
    }
    job_t J;
    J.d = d; J.x = x; J.Wr = Wr; J.br = br; J.groups = groups; J.experts = experts;
    if (given && given->ids) {                 /* given experts: distinct and in range */
        for (int i = 0; i < n; ++i)
            for (int j = 0; j < d->top_k; ++j) {
                int32_t e = given->ids[(size_t)i * d->top_k + j];
                if (e < 0 || e >= d->n_experts) return -1;
                for (int m = 0; m < j; ++m)
                    if (given->ids[(size_t)i * d->top_k + m] == e) return -1;
            }
    }
    J.D = D; J.U = U; J.out = out; J.taps = taps; J.given = given; J.list = list; J.n = n;
    J.next = 0;
    pthread_mutex_init(&J.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads == 1) {
        worker(&J);
    } else {
        pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
        for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &J);
        for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
        free(th);
    }
    pthread_mutex_destroy(&J.mu);
    return 0;
}

int orc_layer_forward(const orc_desc* d, const float* x, const float* Wr, const float* br,
                      const int32_t* groups, const uint8_t* experts, const uint8_t* D,
                      const uint8_t* U, const int32_t* list, int n, float* out,
                      const orc_taps* taps, int nthreads) {
    return orc_layer_forward_given(d, x, Wr, br, groups, experts, D, U, list, n, out, taps, NULL,
                                   nthreads);
}
