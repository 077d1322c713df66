/*
 * CPU oracle for the blockwise-int8 ("q8") Muon momentum update.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code with the HIP library.
 *
 * Built with gcc -O2 -fopenmp -ffp-contract=off (no fast-math, no FTZ), so
 * every float expression below is evaluated in IEEE binary32 with one
 * rounding per operation, in exactly the order written.
 *
 * Source: "Quantized Muon Momentum" (cppmega docs), sections
 *   - "What Exists": state = int8 codes (same shape as the momentum) plus
 *     one fp32 absmax per block of 256 elements; symmetric nearest rounding
 *     with effective range [-127, 127];
 *   - "Algorithm": per 256-element block: load codes and absmax, dequantise
 *     in fp32, load the grad, m = beta*old + (1-beta)*grad, store m into the
 *     grad buffer, new block absmax, requantise, store codes and absmax,
 *     optionally accumulate the block sum of m*m;
 *   - "Grouped QKV And Sharding": one sum of squares per logical norm group,
 *     then every block scaled by its group norm.
 *
 * Readings where the page is silent (each listed in the design notes):
 *   - dequantisation order: old = (float)code * (absmax / 127);
 *   - the EMA is two separately rounded products and one rounded sum (no FMA);
 *   - "nearest" rounding is round-half-to-even (rintf in the default mode);
 *   - an all-zero block stores codes 0 and absmax 0;
 *   - requantisation: x = m * (127 / amax), rounded, clamped to [-127, 127]
 *     with fmaxf / fminf (which return the number when the other operand is
 *     NaN, so a NaN m codes as -127); for a block so small (amax < 2^-64)
 *     that 127 / amax could overflow, m and amax are both scaled by 2^64
 *     first, which is exact and leaves x unchanged wherever 127 / amax is
 *     finite (a zero element then stays 0 instead of 0 * inf);
 *   - the new absmax is taken over the fp32 m (before rounding m to the grad
 *     dtype), and so is the block sum of squares;
 *   - block sums of squares are accumulated in fp64 (squares of fp32 values
 *     are exact in fp64); group sums add block sums in ascending block order;
 *   - group inverse norm = (float)(1 / (sqrt(S_g) + eps)) computed in fp64;
 *   - the scale pass rounds float(stored grad) * inv to the grad dtype
 *     (round to nearest even).
 *
 * Stochastic rounding ("Known Limitations" names it as not implemented on
 * the page; this is the reading taken for it):
 *   - x = m * (127 / amax) exactly as for nearest rounding; q = floor(x) + 1
 *     with probability frac(x) = x - floor(x), else floor(x); clamped to
 *     [-127, 127].  floor(x) is exact; x - floor(x) is one binary32
 *     subtraction (exact for x >= 0, rounded once for some negative x);
 *   - the uniform u in [0, 1) is (r >> 8) * 2^-24 for a 32-bit word r of
 *     Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers:
 *     as easy as 1, 2, 3", SC 2011): counter (e / 4 low word, e / 4 high
 *     word, offset, tensor index), key (seed low word, seed high word), r is
 *     output word e mod 4; round up iff u < frac(x).
 */
#include <math.h>
#include <stdlib.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define OR_BLOCK 256

enum { OR_F32 = 0, OR_BF16 = 1, OR_F16 = 2 };

/* ----------------------------------------------------------- requantise */

/* x = (m * s) * inv with s and inv from here: s = 2^64 for amax < 2^-64
 * (amax * s is exact), else 1; inv = 127 / (amax * s). */
static inline void requant_scale(float amax, float *s, float *inv) {
    *s = amax < 0x1p-64f ? 0x1p64f : 1.0f;
    *inv = 127.0f / (amax * *s);
}

/* A rounded value clamped to [-127, 127] (NaN -> -127). */
static inline int8_t code_of(float q) { return (int8_t)fminf(fmaxf(q, -127.0f), 127.0f); }

/* ---------------------------------------------------------------- dtypes */

static uint32_t bits_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float float_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* binary32 -> bfloat16, round to nearest, ties to even; NaN stays NaN (quiet). */
uint16_t or_bf16_from_f32(float f)
{
    uint32_t u = bits_of(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep = u >> 16;
    uint32_t rest = u & 0xffffu;
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u)))
        keep += 1u;            /* carries into the exponent correctly, incl. to inf */
    return (uint16_t)keep;
}

float or_f32_from_bf16(uint16_t h) { return float_of((uint32_t)h << 16); }

/* binary32 -> binary16, round to nearest, ties to even, with subnormals. */
uint16_t or_f16_from_f32(float f)
{
    const uint32_t u = bits_of(f);
    const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u)                 /* NaN: quiet */
        return (uint16_t)(sign | 0x7e00u);
    if (a >= 0x477ff000u)                /* |f| >= 65520 rounds to infinity */
        return (uint16_t)(sign | 0x7c00u);
    if (a >= 0x38800000u) {              /* |f| >= 2^-14: normal binary16 */
        const uint32_t r = a - 0x38000000u;   /* exponent bias 127 -> 15 */
        uint32_t q = r >> 13;
        const uint32_t rem = r & 0x1fffu;
        if (rem > 0x1000u || (rem == 0x1000u && (q & 1u)))
            q += 1u;                     /* a carry moves into the exponent */
        return (uint16_t)(sign | q);
    }
    if (a < 0x33000000u)                 /* |f| < 2^-25 rounds to zero */
        return sign;
    /* binary16 subnormal: |f| = sig * 2^(E-150); the unit is 2^-24 */
    const uint32_t E = a >> 23;
    const uint32_t sig = (a & 0x7fffffu) | 0x800000u;
    const uint32_t s = 126u - E;         /* 14 .. 24 */
    uint32_t q = sig >> s;
    const uint32_t rem = sig & ((1u << s) - 1u);
    const uint32_t half = 1u << (s - 1u);
    if (rem > half || (rem == half && (q & 1u)))
        q += 1u;
    return (uint16_t)(sign | q);
}

float or_f32_from_f16(uint16_t h)
{
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t ex = (h >> 10) & 0x1fu;
    uint32_t man = h & 0x3ffu;
    if (ex == 0x1fu)
        return float_of(sign | 0x7f800000u | (man << 13));
    if (ex == 0) {
        /* subnormal: man * 2^-24, exact in binary32 */
        float v = (float)man * 5.9604644775390625e-08f;
        return sign ? -v : v;
    }
    return float_of(sign | ((ex - 15 + 127) << 23) | (man << 13));
}

static float load_grad(const void *grad, int dtype, int64_t i)
{
    if (dtype == OR_F32) return ((const float *)grad)[i];
    if (dtype == OR_BF16) return or_f32_from_bf16(((const uint16_t *)grad)[i]);
    return or_f32_from_f16(((const uint16_t *)grad)[i]);
}

static void store_grad(void *grad, int dtype, int64_t i, float v)
{
    if (dtype == OR_F32) ((float *)grad)[i] = v;
    else if (dtype == OR_BF16) ((uint16_t *)grad)[i] = or_bf16_from_f32(v);
    else ((uint16_t *)grad)[i] = or_f16_from_f32(v);
}

/* ---------------------------------------------------------- Philox4x32 */

/* Philox4x32 with 10 rounds, from the SC 2011 paper: each round multiplies
 * counter words 0 and 2 by two fixed 32-bit constants, forms the new counter
 * from the high halves xor-ed with the other words and the key and the low
 * halves, and the key is advanced by the two Weyl constants between rounds. */
void or_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; r++) {
        if (r > 0) {
            k0 += W0;
            k1 += W1;
        }
        const uint64_t p0 = (uint64_t)M0 * c[0];
        const uint64_t p1 = (uint64_t)M1 * c[2];
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
        const uint32_t n1 = (uint32_t)p1;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
        const uint32_t n3 = (uint32_t)p0;
        c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
    }
    for (int i = 0; i < 4; i++) out[i] = c[i];
}

/* The uniform of element e for stochastic rounding (see the header). */
static float sr_uniform(int64_t e, uint64_t seed, uint32_t offset, uint32_t tensor)
{
    const uint64_t q = (uint64_t)e >> 2;
    const uint32_t ctr[4] = {(uint32_t)q, (uint32_t)(q >> 32), offset, tensor};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t r[4];
    or_philox4x32_10(ctr, key, r);
    return (float)(r[e & 3] >> 8) * 0x1p-24f;
}

/* ------------------------------------------------------------ q8 update */

enum { OR_ROUND_NEAREST = 0, OR_ROUND_STOCHASTIC = 1 };

/*
 * One tensor of `numel` elements.  codes/absmax hold the prior state and are
 * overwritten with the new state; grad holds g and is overwritten with m
 * rounded to its dtype.  block_sumsq (nullable) receives one fp64 sum of m*m
 * per block.  Blocks are [256 b, min(numel, 256 b + 256)): the last block of
 * a tensor covers the remainder.  rounding: nearest, or stochastic with
 * (seed, offset, tensor) selecting the random stream (header).
 */
void or_q8_update_ex(int8_t *codes, float *absmax, void *grad, int dtype,
                     int64_t numel, float beta, double *block_sumsq,
                     int rounding, uint64_t seed, uint32_t offset, uint32_t tensor)
{
    const int64_t nblk = (numel + OR_BLOCK - 1) / OR_BLOCK;
    const float omb = 1.0f - beta;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblk; b++) {
        const int64_t lo = b * OR_BLOCK;
        const int64_t hi = (lo + OR_BLOCK < numel) ? lo + OR_BLOCK : numel;
        float m[OR_BLOCK];
        /* dequantise the old momentum, apply the EMA */
        const float step = absmax[b] / 127.0f;
        float amax = 0.0f;
        for (int64_t i = lo; i < hi; i++) {
            const float old = (float)codes[i] * step;
            const float g = load_grad(grad, dtype, i);
            const float t1 = beta * old;
            const float t2 = omb * g;
            const float mi = t1 + t2;
            m[i - lo] = mi;
            const float a = fabsf(mi);
            if (a > amax) amax = a;
        }
        /* m goes back into the grad buffer */
        for (int64_t i = lo; i < hi; i++)
            store_grad(grad, dtype, i, m[i - lo]);
        /* requantise against the new block absmax */
        if (amax == 0.0f) {
            for (int64_t i = lo; i < hi; i++) codes[i] = 0;
        } else {
            float sc, inv;
            requant_scale(amax, &sc, &inv);
            for (int64_t i = lo; i < hi; i++) {
                const float x = (m[i - lo] * sc) * inv;
                float q;
                if (rounding == OR_ROUND_STOCHASTIC) {
                    const float fl = floorf(x);
                    q = sr_uniform(i, seed, offset, tensor) < x - fl ? fl + 1.0f : fl;
                } else {
                    q = rintf(x);
                }
                codes[i] = code_of(q);
            }
        }
        absmax[b] = amax;
        if (block_sumsq) {
            double s = 0.0;
            for (int64_t i = lo; i < hi; i++) {
                const double d = (double)m[i - lo];
                s += d * d;
            }
            block_sumsq[b] = s;
        }
    }
}

void or_q8_update(int8_t *codes, float *absmax, void *grad, int dtype,
                  int64_t numel, float beta, double *block_sumsq)
{
    or_q8_update_ex(codes, absmax, grad, dtype, numel, beta, block_sumsq, OR_ROUND_NEAREST, 0, 0, 0);
}

/* -------------------------------------------------------- MXFP8 carrier */

/*
 * "Quantized Muon Momentum", section "Wave18B MXFP8 Carrier Probe": the
 * update emits, instead of writing m into the grad buffer, a row-wise MXFP8
 * carrier (E4M3 payload bytes, one E8M0 scale byte per 32 elements of a row)
 * plus one fp32 inverse Frobenius norm.  Readings (design notes): the payload
 * encodes the fp32 m of the update (one pass; inv_norm beside it carries the
 * normalisation); the scale of a 32-element block is 2^(floor(log2 amax) - 8)
 * (the OCP Microscaling rule for E4M3, whose largest exponent is 8), E8M0
 * byte = that exponent + 127, clamped to [0, 254]; an all-zero block has
 * scale byte 0 and zero payload; elements are m / scale rounded to E4M3
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no
 * infinities) to nearest even, saturating at +-448.
 */
uint8_t or_e4m3_from_f32(float v)
{
    const uint32_t u = bits_of(v);
    const uint8_t sign = (uint8_t)((u >> 24) & 0x80u);
    const float a = fabsf(v);
    if (a != a) return (uint8_t)(sign | 0x7Fu);            /* NaN */
    if (a >= 0x1p-6f) {                                     /* normal range */
        uint32_t w = bits_of(a);
        w += 0x7FFFFu + ((w >> 20) & 1u);                   /* round to 3 mantissa bits, ties to even */
        w &= 0xFFF00000u;
        const float r = float_of(w);
        if (r > 448.0f) return (uint8_t)(sign | 0x7Eu);     /* saturate */
        const uint32_t e = ((w >> 23) & 0xFFu) - 127u + 7u;  /* 1 .. 15 */
        const uint32_t m = (w >> 20) & 7u;
        return (uint8_t)(sign | (e << 3) | m);
    }
    /* subnormal: multiples of 2^-9 (a rounds to 8 = the smallest normal) */
    const float n = rintf(a * 512.0f);
    return (uint8_t)(sign | (uint8_t)n);
}

float or_f32_from_e4m3(uint8_t c)
{
    const float s = (c & 0x80u) ? -1.0f : 1.0f;
    const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
    if (e == 0xFu && m == 7u) return s * NAN;
    if (e == 0) return s * (float)m * 0x1p-9f;
    return s * ldexpf(1.0f + (float)m / 8.0f, (int)e - 7);
}

/* E8M0 scale byte of a block with absolute maximum amax (finite, >= 0). */
uint8_t or_mx_scale_byte(float amax)
{
    if (amax == 0.0f) return 0;
    int e2;
    frexpf(amax, &e2);                 /* amax = f * 2^e2, f in [0.5, 1): floor(log2 amax) = e2 - 1 */
    int e = (e2 - 1) - 8;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return (uint8_t)(e + 127);
}

/*
 * The q8 update with the carrier in place of writing m: codes/absmax as
 * or_q8_update (nearest rounding), grad only read, payload [numel] and
 * scales [numel / 32] written; numel and cols multiples of 32.
 */
void or_q8_update_carrier(int8_t *codes, float *absmax, const void *grad, int dtype,
                          int64_t numel, float beta, uint8_t *payload, uint8_t *scales,
                          double *block_sumsq)
{
    const int64_t nblk = (numel + OR_BLOCK - 1) / OR_BLOCK;
    const float omb = 1.0f - beta;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblk; b++) {
        const int64_t lo = b * OR_BLOCK;
        const int64_t hi = (lo + OR_BLOCK < numel) ? lo + OR_BLOCK : numel;
        float m[OR_BLOCK];
        const float step = absmax[b] / 127.0f;
        float amax = 0.0f;
        for (int64_t i = lo; i < hi; i++) {
            const float old = (float)codes[i] * step;
            const float g = load_grad(grad, dtype, i);
            const float t1 = beta * old;
            const float t2 = omb * g;
            const float mi = t1 + t2;
            m[i - lo] = mi;
            const float a = fabsf(mi);
            if (a > amax) amax = a;
        }
        /* carrier: 32-element MX blocks inside this 256-block */
        for (int64_t k = lo; k < hi; k += 32) {
            float bm = 0.0f;
            for (int64_t i = k; i < k + 32; i++) {
                const float a = fabsf(m[i - lo]);
                if (a > bm) bm = a;
            }
            const uint8_t sb = or_mx_scale_byte(bm);
            scales[k / 32] = sb;
            const float inv_scale = ldexpf(1.0f, -((int)sb - 127));   /* 1 / 2^(sb - 127), exact */
            for (int64_t i = k; i < k + 32; i++)
                payload[i] = bm == 0.0f ? 0 : or_e4m3_from_f32(m[i - lo] * inv_scale);
        }
        if (amax == 0.0f) {
            for (int64_t i = lo; i < hi; i++) codes[i] = 0;
        } else {
            float sc, inv;
            requant_scale(amax, &sc, &inv);
            for (int64_t i = lo; i < hi; i++) codes[i] = code_of(rintf((m[i - lo] * sc) * inv));
        }
        absmax[b] = amax;
        if (block_sumsq) {
            double s = 0.0;
            for (int64_t i = lo; i < hi; i++) {
                const double d = (double)m[i - lo];
                s += d * d;
            }
            block_sumsq[b] = s;
        }
    }
}

/*
 * The carrier of a tall matrix handed over transposed (reading R29): the q8
 * update of a rows x cols row-major tensor (codes/absmax/block sums exactly
 * as or_q8_update, nearest rounding; the grad only read), with the MXFP8
 * carrier of m^T in place of m's: payload_t is cols x rows row-major (byte
 * [c][r] codes m[r][c]) and scales_t is cols x rows/32, one E8M0 byte per 32
 * consecutive rows of a column, each with the rule of or_q8_update_carrier.
 * rows a multiple of 32.
 */
void or_q8_update_carrier_t(int8_t *codes, float *absmax, const void *grad, int dtype,
                            int64_t rows, int64_t cols, float beta, uint8_t *payload_t,
                            uint8_t *scales_t, double *block_sumsq)
{
    const int64_t numel = rows * cols;
    const int64_t nblk = (numel + OR_BLOCK - 1) / OR_BLOCK;
    const float omb = 1.0f - beta;
    float *m = malloc((size_t)numel * sizeof(float));
    if (!m) return;
    /* the update, block by block (the same operations as or_q8_update) */
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblk; b++) {
        const int64_t lo = b * OR_BLOCK;
        const int64_t hi = (lo + OR_BLOCK < numel) ? lo + OR_BLOCK : numel;
        const float step = absmax[b] / 127.0f;
        float amax = 0.0f;
        for (int64_t i = lo; i < hi; i++) {
            const float old = (float)codes[i] * step;
            const float g = load_grad(grad, dtype, i);
            const float t1 = beta * old;
            const float t2 = omb * g;
            m[i] = t1 + t2;
            const float a = fabsf(m[i]);
            if (a > amax) amax = a;
        }
        if (amax == 0.0f) {
            for (int64_t i = lo; i < hi; i++) codes[i] = 0;
        } else {
            float sc, inv;
            requant_scale(amax, &sc, &inv);
            for (int64_t i = lo; i < hi; i++) codes[i] = code_of(rintf((m[i] * sc) * inv));
        }
        absmax[b] = amax;
        if (block_sumsq) {
            double sum = 0.0;
            for (int64_t i = lo; i < hi; i++) sum += (double)m[i] * (double)m[i];
            block_sumsq[b] = sum;
        }
    }
    /* the carrier of m^T: 32 consecutive rows of one column per MX block */
    const int64_t nrb = rows / 32;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; c++) {
        for (int64_t g = 0; g < nrb; g++) {
            float bm = 0.0f;
            for (int64_t r = 32 * g; r < 32 * g + 32; r++) {
                const float a = fabsf(m[r * cols + c]);
                if (a > bm) bm = a;
            }
            const uint8_t sb = or_mx_scale_byte(bm);
            scales_t[c * nrb + g] = sb;
            const float inv_scale = ldexpf(1.0f, -((int)sb - 127));
            for (int64_t r = 32 * g; r < 32 * g + 32; r++)
                payload_t[c * rows + r] = bm == 0.0f ? 0 : or_e4m3_from_f32(m[r * cols + c] * inv_scale);
        }
    }
    free(m);
}

/* --------------------------------------------------------- group norms */

/* S_g = sum of block sums of group g, blocks visited in ascending order. */
void or_group_sums(const double *block_sumsq, const int32_t *block_group,
                   int64_t nblk, int32_t ngroups, double *group_sums)
{
    for (int32_t g = 0; g < ngroups; g++) group_sums[g] = 0.0;
    for (int64_t b = 0; b < nblk; b++)
        group_sums[block_group[b]] += block_sumsq[b];
}

/* inv_g = 1 / (||M_g||_F + eps), evaluated in fp64 and rounded to fp32. */
void or_group_inv_norm(const double *group_sums, int32_t ngroups, float eps,
                       float *inv)
{
    for (int32_t g = 0; g < ngroups; g++)
        inv[g] = (float)(1.0 / (sqrt(group_sums[g]) + (double)eps));
}

/* Scale pass: grad <- round_dtype(float(grad) * inv[group of its block]). */
void or_scale_by_group(void *grad, int dtype, int64_t numel,
                       const int32_t *block_group, const float *inv)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < numel; i++) {
        const float s = inv[block_group[i / OR_BLOCK]];
        store_grad(grad, dtype, i, load_grad(grad, dtype, i) * s);
    }
}

/* Round an fp32 array to bf16 / f16 bit patterns (used to build inputs). */
void or_round_array(const float *src, int64_t n, int dtype, uint16_t *dst)
{
    for (int64_t i = 0; i < n; i++)
        dst[i] = dtype == OR_BF16 ? or_bf16_from_f32(src[i]) : or_f16_from_f32(src[i]);
}

void or_widen_array(const uint16_t *src, int64_t n, int dtype, float *dst)
{
    for (int64_t i = 0; i < n; i++)
        dst[i] = dtype == OR_BF16 ? or_f32_from_bf16(src[i]) : or_f32_from_f16(src[i]);
}

/* Threads an OpenMP region of this library uses (reported with timings). */
int or_num_threads(void) { return omp_get_max_threads(); }
