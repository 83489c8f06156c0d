/*
 * tq_oracle.c -- plain, slow, scalar fp32 CPU oracle of the TurboQuant
 * KV-cache codec.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library. The HIP codec never links, includes or
 * calls anything here, and this file shares no code with it.
 *
 * Sources (pages, cited by title and the function or table on them):
 *   [ops]    "@mlx-bun/inference 0.0.0-stage -> 1.0.0",
 *            package/src/kernels/turboquant/ops.ts
 *   [tables] "mlx-bun 0.0.9 -> 0.0.11", src/mlx/turboquant-tables.ts
 *
 * Every step is written in the order the pages apply it, one element at a
 * time, in binary32 arithmetic. Build with -O2 -ffp-contract=off and without
 * any fast-math flag: products are rounded before they are added and every
 * division and square root is the IEEE one.
 *
 * Readings where the pages leave a step open (each listed in the design
 * notes of the repository):
 *   - rounding of ops.round is round-half-to-even (rintf);
 *   - the Hadamard transform is the natural (Sylvester) order transform,
 *     computed as radix-2 butterflies with span h = 1, 2, 4, ..., d/2 and
 *     then multiplied once by binary32(1/sqrt(d));
 *   - the per-group mean of squares sums k = 0..31 in order;
 *   - float -> fp16 and float -> bf16 conversions round to nearest even and
 *     overflow to infinity.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "tq_oracle_tables.h"

#define TQO_BLOCK 32 /* [ops] TURBOQUANT_BLOCK_SIZE: groups of 32 along head_dim */

enum { TQO_OK = 0, TQO_E_ARG = 1 };
enum { TQO_F32 = 0, TQO_BF16 = 1 };

/* ------------------------------------------------------------------ */
/* binary16 / bfloat16 conversions, written from the IEEE 754 format   */
/* definitions (sign, biased exponent, fraction).                      */
/* ------------------------------------------------------------------ */

static uint32_t bits_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float float_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* Round the finite value v (exact in double) to a grid of spacing
 * 2^q_exp, ties to even. */
static double round_to_quantum(double v, int q_exp)
{
    double q = ldexp(1.0, q_exp);
    double n = v / q;              /* exact: q is a power of two */
    double r = nearbyint(n);       /* default mode: nearest, ties to even */
    return r * q;
}

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Normal numbers 2^-14 .. 65504; subnormal spacing 2^-24. */
uint16_t tqo_f32_to_f16(float f)
{
    uint32_t u = bits_of(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(f)) return (uint16_t)(sign | 0x7e00u);
    double a = fabs((double)f);
    if (isinf(f)) return (uint16_t)(sign | 0x7c00u);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                       /* a = m 2^e, m in [0.5, 1) */
    int E = e - 1;                      /* a in [2^E, 2^(E+1)) */
    int q_exp = (E < -14) ? -24 : E - 10;
    double r = round_to_quantum(a, q_exp);
    if (r >= 65536.0) return (uint16_t)(sign | 0x7c00u);   /* overflow -> inf */
    if (r == 0.0) return sign;
    frexp(r, &e);
    E = e - 1;
    if (E < -14) {                      /* subnormal: r = f * 2^-24 */
        return (uint16_t)(sign | (uint16_t)(r / ldexp(1.0, -24)));
    }
    uint32_t frac = (uint32_t)((r / ldexp(1.0, E) - 1.0) * 1024.0);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)frac);
}

float tqo_f16_to_f32(uint16_t h)
{
    int s = (h >> 15) & 1, E = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (E == 0x1f) v = m ? NAN : INFINITY;
    else if (E == 0) v = ldexp((double)m, -24);
    else v = ldexp(1.0 + m / 1024.0, E - 15);
    return (float)(s ? -v : v);
}

/* bfloat16: the upper 16 bits of binary32 (8 exponent bits, 7 fraction
 * bits). Normal numbers from 2^-126; subnormal spacing 2^-133; largest
 * finite (2 - 2^-7) 2^127. */
uint16_t tqo_f32_to_bf16(float f)
{
    uint32_t u = bits_of(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(f)) return (uint16_t)(sign | 0x7fc0u);
    if (isinf(f)) return (uint16_t)(sign | 0x7f80u);
    double a = fabs((double)f);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);
    int E = e - 1;
    int q_exp = (E < -126) ? -133 : E - 7;
    double r = round_to_quantum(a, q_exp);
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7f80u);
    /* r is now a bfloat16 value, hence exactly a binary32 whose low 16
     * bits are zero. */
    return (uint16_t)(sign | (uint16_t)(bits_of((float)r) >> 16));
}

float tqo_bf16_to_f32(uint16_t b) { return float_of((uint32_t)b << 16); }

/* ------------------------------------------------------------------ */
/* tables                                                              */
/* ------------------------------------------------------------------ */

/* [ops] isSupportedHeadDim / [tables] TURBOQUANT_HEAD_DIMS, SIGN_VECTORS */
const float *tqo_signs(int32_t d)
{
    switch (d) {
    case 64: return TQO_SIGN_64;
    case 128: return TQO_SIGN_128;
    case 256: return TQO_SIGN_256;
    case 512: return TQO_SIGN_512;
    default: return 0;
    }
}

/* [ops] centroidsFor / boundariesFor; [tables] TURBOQUANT_VALUE_BITS,
 * LLOYD_MAX. Returns the number of centroids (2^bits) or 0. */
int32_t tqo_lloyd_max(int32_t bits, const float **centroids, const float **boundaries)
{
    switch (bits) {
    case 2: *centroids = TQO_CENTROIDS_2; *boundaries = TQO_BOUNDARIES_2; return 4;
    case 3: *centroids = TQO_CENTROIDS_3; *boundaries = TQO_BOUNDARIES_3; return 8;
    case 4: *centroids = TQO_CENTROIDS_4; *boundaries = TQO_BOUNDARIES_4; return 16;
    case 5: *centroids = TQO_CENTROIDS_5; *boundaries = TQO_BOUNDARIES_5; return 32;
    case 8: *centroids = TQO_CENTROIDS_8; *boundaries = TQO_BOUNDARIES_8; return 256;
    default: *centroids = 0; *boundaries = 0; return 0;
    }
}

/* [ops] packedDim: bytes for dim elements at bits each; -1 when dim*bits is
 * not a multiple of 8. */
int64_t tqo_packed_dim(int32_t dim, int32_t bits)
{
    if (dim < 0 || bits <= 0) return -1;
    if (((int64_t)dim * bits) % 8 != 0) return -1;
    return ((int64_t)dim * bits) / 8;
}

static int supported_key_bits(int32_t bits)
{
    return bits == 2 || bits == 3 || bits == 4 || bits == 5 || bits == 8;
}

/* ------------------------------------------------------------------ */
/* rotation                                                            */
/* ------------------------------------------------------------------ */

/* binary32 value of 1/sqrt(d): the normalisation the Hadamard transform
 * applies ([ops] fwht() doc comment). */
float tqo_hadamard_scale(int32_t d) { return (float)(1.0 / sqrt((double)d)); }

/* Normalised fast Walsh-Hadamard transform of one row, in place. */
void tqo_hadamard(float *y, int32_t d)
{
    for (int32_t h = 1; h < d; h *= 2) {
        for (int32_t i = 0; i < d; i += 2 * h) {
            for (int32_t j = i; j < i + h; ++j) {
                float a = y[j];
                float b = y[j + h];
                y[j] = a + b;
                y[j + h] = a - b;
            }
        }
    }
    float r = tqo_hadamard_scale(d);
    for (int32_t i = 0; i < d; ++i) y[i] = y[i] * r;
}

/* [ops] fwht(x, encode): encode multiplies by the sign vector and then
 * transforms; decode transforms and then multiplies by the signs. */
int32_t tqo_fwht(float *y, int32_t d, int32_t encode)
{
    const float *s = tqo_signs(d);
    if (!s) return TQO_E_ARG;
    if (encode) {
        for (int32_t i = 0; i < d; ++i) y[i] = y[i] * s[i];
        tqo_hadamard(y, d);
    } else {
        tqo_hadamard(y, d);
        for (int32_t i = 0; i < d; ++i) y[i] = y[i] * s[i];
    }
    return TQO_OK;
}

/* ------------------------------------------------------------------ */
/* value path                                                          */
/* ------------------------------------------------------------------ */

/* [ops] searchsorted: index = number of boundaries strictly below z,
 * counted by comparing against every boundary. */
int32_t tqo_bin_index(float z, int32_t bits)
{
    const float *c, *b;
    int32_t n = tqo_lloyd_max(bits, &c, &b);
    int32_t idx = 0;
    for (int32_t j = 0; j < n - 1; ++j)
        if (z > b[j]) idx += 1;
    return idx;
}

/* [ops] encodeValues for one row x[0..d): rotate, per-32 RMS scale, divide
 * by (scale + 1e-8), count boundaries. idx[d] receives the unpacked
 * indices, scale16[d/32] the fp16 scales. z (optional, d floats) receives
 * the normalised values that were binned. */
int32_t tqo_value_encode_row(const float *x, int32_t d, int32_t bits,
                             uint8_t *idx, uint16_t *scale16, float *z)
{
    float y[512];
    const float *c, *b;
    if (!tqo_signs(d) || !tqo_lloyd_max(bits, &c, &b)) return TQO_E_ARG;
    for (int32_t i = 0; i < d; ++i) y[i] = x[i];
    tqo_fwht(y, d, 1);
    const float eps = 1e-8f;
    for (int32_t g = 0; g < d / TQO_BLOCK; ++g) {
        const float *yg = y + g * TQO_BLOCK;
        float ss = 0.0f;
        for (int32_t k = 0; k < TQO_BLOCK; ++k) {
            float sq = yg[k] * yg[k];
            ss = ss + sq;
        }
        float mean_sq = ss / (float)TQO_BLOCK;
        float scale = sqrtf(mean_sq);
        float scale_eps = scale + eps;
        for (int32_t k = 0; k < TQO_BLOCK; ++k) {
            float zn = yg[k] / scale_eps;
            if (z) z[g * TQO_BLOCK + k] = zn;
            idx[g * TQO_BLOCK + k] = (uint8_t)tqo_bin_index(zn, bits);
        }
        scale16[g] = tqo_f32_to_f16(scale);
    }
    return TQO_OK;
}

/* [ops] dequantScaled: centroid times the fp16 scale, still rotated. */
int32_t tqo_value_dequant_rotated_row(const uint8_t *idx, const uint16_t *scale16,
                                      int32_t d, int32_t bits, float *out)
{
    const float *c, *b;
    int32_t n = tqo_lloyd_max(bits, &c, &b);
    if (!n || !tqo_signs(d)) return TQO_E_ARG;
    for (int32_t i = 0; i < d; ++i) {
        int32_t k = idx[i];
        if (k >= n) return TQO_E_ARG;
        out[i] = c[k] * tqo_f16_to_f32(scale16[i / TQO_BLOCK]);
    }
    return TQO_OK;
}

/* [ops] decodeValues: dequantScaled, then the inverse rotation. Output in
 * binary32 (the caller rounds to bf16 for the reference output dtype). */
int32_t tqo_value_decode_row(const uint8_t *idx, const uint16_t *scale16,
                             int32_t d, int32_t bits, float *out)
{
    int32_t st = tqo_value_dequant_rotated_row(idx, scale16, d, bits, out);
    if (st) return st;
    return tqo_fwht(out, d, 0);
}

/* ------------------------------------------------------------------ */
/* key path                                                            */
/* ------------------------------------------------------------------ */

/* [ops] encodeKeys for one row: per-32 min/max affine quantisation in
 * binary32. q[d] receives bytes (two's complement int8 when is_signed,
 * else uint8), scale16/zero16[d/32] the fp16 scale and zero point. */
int32_t tqo_key_encode_row(const float *x, int32_t d, int32_t bits, int32_t is_signed,
                           uint8_t *q, uint16_t *scale16, uint16_t *zero16)
{
    if (d % TQO_BLOCK != 0 || d <= 0) return TQO_E_ARG;
    if (!supported_key_bits(bits)) return TQO_E_ARG;
    if (is_signed && bits != 8) return TQO_E_ARG;
    const float eps = 1e-8f;
    const int32_t max_val = is_signed ? (1 << (bits - 1)) - 1 : (1 << bits) - 1;
    for (int32_t g = 0; g < d / TQO_BLOCK; ++g) {
        const float *xg = x + g * TQO_BLOCK;
        float mn = xg[0], mx = xg[0];
        for (int32_t k = 1; k < TQO_BLOCK; ++k) {
            if (xg[k] < mn) mn = xg[k];
            if (xg[k] > mx) mx = xg[k];
        }
        float scale, zp, lo, hi;
        if (is_signed) {
            float range = mx - mn;
            scale = range / (float)(2.0 * max_val);
            float scale_eps = scale + eps;
            float denom = 2.0f * scale_eps;
            float sum_mm = mx + mn;
            zp = rintf(sum_mm / denom);
            lo = (float)(-max_val);
            hi = (float)max_val;
        } else {
            float range = mx - mn;
            scale = range / (float)max_val;
            float scale_eps = scale + eps;
            zp = rintf(mn / scale_eps);
            lo = 0.0f;
            hi = (float)max_val;
        }
        float scale_eps = scale + eps;
        for (int32_t k = 0; k < TQO_BLOCK; ++k) {
            float over = xg[k] / scale_eps;
            float shifted = over - zp;
            float r = rintf(shifted);
            if (r < lo) r = lo;
            if (r > hi) r = hi;
            int32_t qi = (int32_t)r;
            q[g * TQO_BLOCK + k] = (uint8_t)(qi & 0xff);
        }
        scale16[g] = tqo_f32_to_f16(scale);
        zero16[g] = tqo_f32_to_f16(zp);
    }
    return TQO_OK;
}

/* [ops] decodeKeys: (q + zero) * scale in binary32, per element. */
int32_t tqo_key_decode_row(const uint8_t *q, const uint16_t *scale16, const uint16_t *zero16,
                           int32_t d, int32_t is_signed, float *out)
{
    if (d % TQO_BLOCK != 0 || d <= 0) return TQO_E_ARG;
    for (int32_t i = 0; i < d; ++i) {
        float qf = is_signed ? (float)(int8_t)q[i] : (float)q[i];
        float zero = tqo_f16_to_f32(zero16[i / TQO_BLOCK]);
        float scale = tqo_f16_to_f32(scale16[i / TQO_BLOCK]);
        float sum = qf + zero;
        out[i] = sum * scale;
    }
    return TQO_OK;
}

/* ------------------------------------------------------------------ */
/* bit packing                                                         */
/* ------------------------------------------------------------------ */

/* [ops] bit-packing section: a flat little-endian bit stream in which
 * element i occupies bits [i*bits, i*bits + bits), bit 0 being the least
 * significant bit of byte 0. bits == 8 stores one byte per element. */
int32_t tqo_pack_bits(const uint8_t *vals, int64_t n, int32_t bits, uint8_t *out)
{
    int64_t nbytes = ((int64_t)n * bits) / 8;
    if (bits < 1 || bits > 8 || ((int64_t)n * bits) % 8 != 0) return TQO_E_ARG;
    for (int64_t i = 0; i < nbytes; ++i) out[i] = 0;
    for (int64_t i = 0; i < n; ++i) {
        for (int32_t t = 0; t < bits; ++t) {
            int64_t pos = i * bits + t;
            uint8_t bit = (uint8_t)((vals[i] >> t) & 1u);
            out[pos / 8] = (uint8_t)(out[pos / 8] | (bit << (pos % 8)));
        }
    }
    return TQO_OK;
}

int32_t tqo_unpack_bits(const uint8_t *packed, int64_t n, int32_t bits, uint8_t *vals)
{
    if (bits < 1 || bits > 8 || ((int64_t)n * bits) % 8 != 0) return TQO_E_ARG;
    for (int64_t i = 0; i < n; ++i) {
        uint8_t v = 0;
        for (int32_t t = 0; t < bits; ++t) {
            int64_t pos = i * bits + t;
            uint8_t bit = (uint8_t)((packed[pos / 8] >> (pos % 8)) & 1u);
            v = (uint8_t)(v | (bit << t));
        }
        vals[i] = v;
    }
    return TQO_OK;
}

/* ------------------------------------------------------------------ */
/* whole-tensor encode / decode over rows = tokens * heads             */
/* ------------------------------------------------------------------ */

static float load_elem(const void *base, int32_t dtype, int64_t i)
{
    if (dtype == TQO_BF16) return tqo_bf16_to_f32(((const uint16_t *)base)[i]);
    return ((const float *)base)[i];
}

/* Encode rows x [rows, d] of K and/or V (either may be NULL) into the five
 * planes: k_codes [rows, d*k_bits/8], k_scale/k_zero [rows, d/32] (fp16
 * bits), v_codes [rows, d*v_bits/8], v_scale [rows, d/32]. */
int32_t tqo_encode_kv(const void *k, const void *v, int32_t in_dtype, int64_t rows, int32_t d,
                      int32_t k_bits, int32_t k_signed, int32_t v_bits,
                      uint8_t *k_codes, uint16_t *k_scale, uint16_t *k_zero,
                      uint8_t *v_codes, uint16_t *v_scale)
{
    float x[512];
    uint8_t idx[512];
    if (!tqo_signs(d) || rows < 0) return TQO_E_ARG;
    if (in_dtype != TQO_F32 && in_dtype != TQO_BF16) return TQO_E_ARG;
    const int32_t G = d / TQO_BLOCK;
    if (k) {
        if (!supported_key_bits(k_bits) || (k_signed && k_bits != 8)) return TQO_E_ARG;
        int64_t kb = tqo_packed_dim(d, k_bits);
        for (int64_t r = 0; r < rows; ++r) {
            for (int32_t i = 0; i < d; ++i) x[i] = load_elem(k, in_dtype, r * d + i);
            int32_t st = tqo_key_encode_row(x, d, k_bits, k_signed, idx, k_scale + r * G, k_zero + r * G);
            if (st) return st;
            tqo_pack_bits(idx, d, k_bits, k_codes + r * kb);
        }
    }
    if (v) {
        const float *c, *b;
        if (!tqo_lloyd_max(v_bits, &c, &b)) return TQO_E_ARG;
        int64_t vb = tqo_packed_dim(d, v_bits);
        for (int64_t r = 0; r < rows; ++r) {
            for (int32_t i = 0; i < d; ++i) x[i] = load_elem(v, in_dtype, r * d + i);
            int32_t st = tqo_value_encode_row(x, d, v_bits, idx, v_scale + r * G, 0);
            if (st) return st;
            tqo_pack_bits(idx, d, v_bits, v_codes + r * vb);
        }
    }
    return TQO_OK;
}

static void store_elem(void *base, int32_t dtype, int64_t i, float f)
{
    if (dtype == TQO_BF16) ((uint16_t *)base)[i] = tqo_f32_to_bf16(f);
    else ((float *)base)[i] = f;
}

/* Decode the planes back to K and/or V rows [rows, d] in binary32 or bf16.
 * rotated_v != 0 stops the value path before the inverse rotation
 * ([ops] decodeValuesRotated). */
int32_t tqo_decode_kv(const uint8_t *k_codes, const uint16_t *k_scale, const uint16_t *k_zero,
                      const uint8_t *v_codes, const uint16_t *v_scale,
                      int64_t rows, int32_t d, int32_t k_bits, int32_t k_signed, int32_t v_bits,
                      void *k_out, void *v_out, int32_t out_dtype, int32_t rotated_v)
{
    float y[512];
    uint8_t idx[512];
    if (!tqo_signs(d) || rows < 0) return TQO_E_ARG;
    if (out_dtype != TQO_F32 && out_dtype != TQO_BF16) return TQO_E_ARG;
    const int32_t G = d / TQO_BLOCK;
    if (k_out) {
        if (!supported_key_bits(k_bits) || (k_signed && k_bits != 8)) return TQO_E_ARG;
        int64_t kb = tqo_packed_dim(d, k_bits);
        for (int64_t r = 0; r < rows; ++r) {
            tqo_unpack_bits(k_codes + r * kb, d, k_bits, idx);
            int32_t st = tqo_key_decode_row(idx, k_scale + r * G, k_zero + r * G, d, k_signed, y);
            if (st) return st;
            for (int32_t i = 0; i < d; ++i) store_elem(k_out, out_dtype, r * d + i, y[i]);
        }
    }
    if (v_out) {
        const float *c, *b;
        if (!tqo_lloyd_max(v_bits, &c, &b)) return TQO_E_ARG;
        int64_t vb = tqo_packed_dim(d, v_bits);
        for (int64_t r = 0; r < rows; ++r) {
            tqo_unpack_bits(v_codes + r * vb, d, v_bits, idx);
            int32_t st = rotated_v
                ? tqo_value_dequant_rotated_row(idx, v_scale + r * G, d, v_bits, y)
                : tqo_value_decode_row(idx, v_scale + r * G, d, v_bits, y);
            if (st) return st;
            for (int32_t i = 0; i < d; ++i) store_elem(v_out, out_dtype, r * d + i, y[i]);
        }
    }
    return TQO_OK;
}

/* [ops] unrotateValues: inverse rotation of rows [rows, d] in binary32,
 * returned in the input's dtype. */
int32_t tqo_unrotate(const void *x, void *out, int32_t dtype, int64_t rows, int32_t d)
{
    float y[512];
    if (!tqo_signs(d) || rows < 0) return TQO_E_ARG;
    if (dtype != TQO_F32 && dtype != TQO_BF16) return TQO_E_ARG;
    for (int64_t r = 0; r < rows; ++r) {
        for (int32_t i = 0; i < d; ++i) y[i] = load_elem(x, dtype, r * d + i);
        tqo_fwht(y, d, 0);
        for (int32_t i = 0; i < d; ++i) store_elem(out, dtype, r * d + i, y[i]);
    }
    return TQO_OK;
}
