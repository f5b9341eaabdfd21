/*
 * CPU oracle for the quantized-weight matmul  out[t][r] = sum_i W[r][i] * x[t][i]
 * with W in GGUF-style Q4_K / Q6_K super-blocks and x quantized to int8 blocks
 * of 32 (an f32 scale d and the f32 product s = d * sum(q) per block).
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
 * baseline leg may load or run this code.  It shares nothing with the HIP path:
 * no headers, helpers, tables or constants.  Plain, slow and written to be read
 * against the pages; f64 wherever a value is combined.
 *
 * Pages cited (by title; section in brackets):
 *   [GEMM]  "The quantized GEMM" (mojo-dllm kernels page)
 *   [MMQ]   "llama.cpp MMQ -- quantized-weight int8 tensor-core matmul: structure,
 *            numerics, SASS census, and minfer contrast"
 *   [CH04]  "04 - Reading minfer's kernels II -- from GEMV to tiled GEMM"
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes of the repository):
 *   R1  Q6_K element-to-bit map inside the low-nibble / high-2-bit planes: the
 *       pages name the planes and their order only; the public GGUF arrangement
 *       is used (two halves of 128; see q6k_decode).  PARITY UNPINNED by the
 *       pages for that map: pinned only by internal consistency and special cases.
 *   R2  Activation scale d = amax / 127 (IEEE f32 divide), codes
 *       q = roundf(x / d) (IEEE f32 divide, ties away from zero), so |q| <= 127.
 *   R3  All-zero block (d == 0): q = 0, s = 0.
 *   R4  s = d * (float)sum(q), one f32 multiply, round to nearest even.
 *   R5  Q6_K group scales are signed int8; Q6_K d sits in the last two bytes.
 *   R17 RMS norm in f32 with one fixed order (the pages fix neither formula nor
 *       order, only that the fused and unfused kernels agree bit for bit): 256
 *       lane partials, lane t taking the values i with (i / 4) mod 256 == t in
 *       increasing i, each by one fused multiply-add of the square; the partials
 *       combined by halving (stride 128, 64, ..., 1); r = 1 / sqrtf(ss / n + eps);
 *       y = (x * r) * w.  See oracle_rmsnorm.
 *   R18 silu(g) * u evaluated in f64 as (g / (1 + exp(-g))) * u and rounded once
 *       to f32 (the value the quantizer then reads).
 *
 *   R20 Q8_0 block: f16 d then 32 int8 codes, w = d * q (the pages give the
 *       34-byte size only; the public GGUF layout).
 *   R21 Q4_0 / Q8_0 rows are read in groups of eight blocks (256 weights); a row
 *       length must be a multiple of 256 like the K-quants.
 *   R22 Q5_K block (the pages name the type only): the public GGUF layout -- d,
 *       dmin, the 12 scale bytes of Q4_K, 32 bytes qh, 128 bytes qs; element
 *       32j + l has low nibble as Q4_K's code and high bit = bit j of qh[l];
 *       code = nibble | 16 * bit (0..31), w = d * sc_j * code - dmin * m_j.
 *   R19 Q8_K activations: the per-32 rules R2/R3 applied to blocks of 256
 *       (d = amax / 127, q = roundf(x / d), zero block -> 0); the 16-value group
 *       sums are the exact integer sums of the codes, stored as f32.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp (no -ffast-math, no -march).
 *
 * OQ_MUTATE (default 0) plants one known mistake, for the tests that show the
 * pins catch it: 1 swapped nibble halves, 2 Q6_K offset 32 dropped, 3 Q4_K min
 * term dropped, 4 scale and min swapped, 5 Q6_K scale per 32 instead of per 16,
 * 6 RMS mean over n - 1, 7 eps added after the square root, 8 squares summed in
 * one running sum, 9 silu with exp(+g), 10 Q8_K scale from the first 32 values of
 * the block only, 11 Q8_K min term from the first 16-value sum of each sub-block,
 * 12 Q4_0 offset 8 dropped, 13 Q4_0 nibbles read interleaved (element 2l low, 2l+1
 * high nibble of byte l) instead of element l low, l + 16 high, 14 Q5_K high bit
 * dropped.
 */
#ifndef OQ_MUTATE
#define OQ_MUTATE 0
#endif
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OQ_TYPE_Q4_K 1
#define OQ_TYPE_Q6_K 2
/* Q6_K stored with each 210-byte block padded to 224 bytes ([GEMM, "The GPU path",
 * "Weights stay in GGUF blocks"]: the upload pads each Q6_K block so every 16-byte
 * piece is aligned).  The first 210 bytes are the block; the pad is ignored. */
#define OQ_TYPE_Q6_K_P224 3
/* 32-weight block formats ([CH03, section 3.2] Q4_0; Q8_0 named there by its
 * 34-byte block), read in groups of eight consecutive blocks = 256 weights. */
#define OQ_TYPE_Q4_0 4
#define OQ_TYPE_Q8_0 5
/* Q5_K (R22): 176 bytes = f16 d | f16 dmin | 12 scale bytes packed as Q4_K's | 32
 * bytes of high bits | 128 bytes of low nibbles arranged as Q4_K's codes. */
#define OQ_TYPE_Q5_K 6

/* f16 bits -> f64, exact (normal, subnormal, zero; inf/nan kept as such). */
static double f16_bits_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1F;
    int man = h & 0x3FF;
    double v;
    if (ex == 0)
        v = ldexp((double)man, -24);               /* subnormal: man * 2^-24 */
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(man | 0x400), ex - 25); /* (1024 + man) * 2^(ex-25) */
    return sign ? -v : v;
}

static uint16_t rd_u16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* ---- O1. Q4_K super-block (144 bytes) ------------------------------------
 * [GEMM, "The GPU path", "Q4_K: packed in shared memory"]: a row's super-block is
 * a 16-byte header (d, dmin, packed scales) then 128 bytes of codes; in code
 * chunk p (32 bytes) byte l carries sub-block 2p in its low nibble and sub-block
 * 2p+1 in its high nibble, at position l.
 * [MMQ, section 6, get_scale_min_k4 semantics]: the 12 scale bytes decode to a
 * (scale, min) pair per sub-block of 32; for j < 4 scale = s[j] & 63,
 * min = s[j+4] & 63; otherwise scale = (s[j+4] & 0xF) | ((s[j-4] >> 6) << 4) and
 * min = (s[j+4] >> 4) | ((s[j] >> 6) << 4).  A code v in 0..15 stands for
 * d*scale*v - dmin*min.  Codes are never centred [MMQ, section 11.4]. */
typedef struct {
    double d, dmin;
    int sc[8], m[8];
    int q[256];
} q4k_block;

static void q4k_scale_min(const uint8_t* s, int j, int* sc, int* m)
{
    if (j < 4) {
        *sc = s[j] & 63;
        *m = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 0xF) | ((s[j - 4] >> 6) << 4);
        *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
#if OQ_MUTATE == 4
    int t = *sc;
    *sc = *m;
    *m = t;
#endif
}

static void q4k_decode(const uint8_t* B, q4k_block* o)
{
    o->d = f16_bits_to_f64(rd_u16(B + 0));
    o->dmin = f16_bits_to_f64(rd_u16(B + 2));
    const uint8_t* s12 = B + 4;
    const uint8_t* qs = B + 16;
    for (int j = 0; j < 8; ++j)
        q4k_scale_min(s12, j, &o->sc[j], &o->m[j]);
    for (int j = 0; j < 8; ++j) {
        int p = j >> 1;
        for (int l = 0; l < 32; ++l) {
            uint8_t byte = qs[32 * p + l];
#if OQ_MUTATE == 1
            o->q[32 * j + l] = (j & 1) ? (byte & 0x0F) : (byte >> 4);
#else
            o->q[32 * j + l] = (j & 1) ? (byte >> 4) : (byte & 0x0F);
#endif
        }
    }
}

static void q5k_decode(const uint8_t* B, q4k_block* o)
{
    o->d = f16_bits_to_f64(rd_u16(B + 0));
    o->dmin = f16_bits_to_f64(rd_u16(B + 2));
    const uint8_t* s12 = B + 4;
    const uint8_t* qh = B + 16;
    const uint8_t* qs = B + 48;
    for (int j = 0; j < 8; ++j)
        q4k_scale_min(s12, j, &o->sc[j], &o->m[j]);
    for (int j = 0; j < 8; ++j) {
        int p = j >> 1;
        for (int l = 0; l < 32; ++l) {
            uint8_t byte = qs[32 * p + l];
            int lo = (j & 1) ? (byte >> 4) : (byte & 0x0F);
#if OQ_MUTATE == 14
            int hi = 0;
#else
            int hi = (qh[l] >> j) & 1;
#endif
            o->q[32 * j + l] = lo | (hi << 4);
        }
    }
}

static void k4_decode(int type, const uint8_t* B, q4k_block* o)
{
    if (type == OQ_TYPE_Q5_K)
        q5k_decode(B, o);
    else
        q4k_decode(B, o);
}

/* ---- O2. Q6_K super-block (210 bytes) ------------------------------------
 * [GEMM, "Q6_K: the same layout and prefetch"]: low nibbles, high bits, 16 int8
 * group scales, d -- in that order; [GEMM, "Weights: 8 rows per register"]: the
 * stored Q6_K code is the value plus 32.  [MMQ, section 4, Q6_K specialization]: the 6-bit
 * code is (low | high) and the value is d * scale * (code - 32), one int8 scale per
 * 16 values.  Element-to-bit map: reading R1 (two halves h of 128 elements; half
 * h uses low bytes 64h.., high bytes 32h.., scales 8h..): for l in 0..31,
 *   element 128h+l      <- low nibble of ql[64h+l],    bits 0-1 of qh[32h+l]
 *   element 128h+32+l   <- low nibble of ql[64h+32+l], bits 2-3 of qh[32h+l]
 *   element 128h+64+l   <- high nibble of ql[64h+l],   bits 4-5 of qh[32h+l]
 *   element 128h+96+l   <- high nibble of ql[64h+32+l],bits 6-7 of qh[32h+l]. */
typedef struct {
    double d;
    int sc[16];
    int q6[256]; /* stored code, 0..63 (value uses q6 - 32) */
} q6k_block;

static void q6k_decode(const uint8_t* B, q6k_block* o)
{
    const uint8_t* ql = B;
    const uint8_t* qh = B + 128;
    const int8_t* sc = (const int8_t*)(B + 192);
    o->d = f16_bits_to_f64(rd_u16(B + 208));
    for (int g = 0; g < 16; ++g)
        o->sc[g] = sc[g];
    for (int h = 0; h < 2; ++h) {
        for (int l = 0; l < 32; ++l) {
            int hb = qh[32 * h + l];
            int a = ql[64 * h + l];
            int b = ql[64 * h + 32 + l];
            o->q6[128 * h + l] = (a & 0xF) | (((hb >> 0) & 3) << 4);
            o->q6[128 * h + 32 + l] = (b & 0xF) | (((hb >> 2) & 3) << 4);
            o->q6[128 * h + 64 + l] = (a >> 4) | (((hb >> 4) & 3) << 4);
            o->q6[128 * h + 96 + l] = (b >> 4) | (((hb >> 6) & 3) << 4);
        }
    }
}

/* ---- O3. Activation quantizer --------------------------------------------
 * [GEMM, "The GPU path", "Activations get one scale per 32"]: int8 codes with one
 * f32 scale per 32 values, with the product of the scale and the code sum stored
 * beside it.  [CH04, section 2.1]: largest magnitude, then scale, then rounding.
 * Readings R2, R3, R4.  Per token t, block k of 32:
 *   amax = max |x|;  d = amax / 127;  q = roundf(x / d);  s = d * sum(q). */
int oracle_quantize(const float* x, int nt, int id, int8_t* q, float* d, float* s)
{
    if (!x || !q || !d || !s || nt < 0 || id < 0 || id % 32)
        return -1;
    int nblk = id / 32;
    for (int t = 0; t < nt; ++t) {
        for (int k = 0; k < nblk; ++k) {
            const float* xb = x + (size_t)t * id + 32 * k;
            int8_t* qb = q + (size_t)t * id + 32 * k;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float a = fabsf(xb[i]);
                if (a > amax)
                    amax = a;
            }
            float dk = amax / 127.0f;
            int sum = 0;
            if (dk == 0.0f) {
                for (int i = 0; i < 32; ++i)
                    qb[i] = 0;
            } else {
                for (int i = 0; i < 32; ++i) {
                    float r = roundf(xb[i] / dk);
                    int qi = (int)r;
                    if (qi > 127 || qi < -127)
                        return -2; /* cannot happen for finite input; kept as a check */
                    qb[i] = (int8_t)qi;
                    sum += qi;
                }
            }
            d[(size_t)t * nblk + k] = dk;
            s[(size_t)t * nblk + k] = dk * (float)sum;
        }
    }
    return 0;
}

/* ---- O6. Producer-side elementwise steps that feed the quantizer -----------
 * [GEMM, "The GPU path", "Fused elementwise kernels"]: each RMS norm and the FFN
 * activation ends in the quantizer; one step adds the projection output into the
 * residual stream and normalizes the sum, one normalizes without the add (first
 * layer), one forms silu(g) * u.  These functions produce the f32 values that
 * oracle_quantize then quantizes; the fused products are checked as
 * oracle_quantize(oracle_rmsnorm(...)) and so on.
 *
 * Reading R17 (sum order).  The norm's f32 result depends on the order in which
 * the squares are added, and the quantized codes depend on its last bit, so the
 * order is part of the operation: lane t (0..255) accumulates, in increasing i,
 * fma(x_i, x_i, p_t) over the i whose group of four, i / 4, is congruent to t
 * modulo 256; the lanes are then combined by halving, p_t += p_{t+s} for
 * s = 128, 64, ..., 1, and ss = p_0. */
static float rms_sum_squares(const float* x, int n)
{
    float p[256];
    for (int t = 0; t < 256; ++t)
        p[t] = 0.0f;
#if OQ_MUTATE == 8
    for (int i = 0; i < n; ++i)
        p[0] = fmaf(x[i], x[i], p[0]);
#else
    for (int i = 0; i < n; ++i) {
        int t = (i / 4) % 256;
        p[t] = fmaf(x[i], x[i], p[t]);
    }
#endif
    for (int stride = 128; stride >= 1; stride /= 2)
        for (int t = 0; t < stride; ++t)
            p[t] = p[t] + p[t + stride];
    return p[0];
}

/* r = 1 / sqrt(mean(x^2) + eps), three correctly rounded f32 operations. */
static float rms_scale(float ss, int n, float eps)
{
#if OQ_MUTATE == 6
    float mean = ss / (float)(n - 1);
#else
    float mean = ss / (float)n;
#endif
#if OQ_MUTATE == 7
    return 1.0f / (sqrtf(mean) + eps);
#else
    return 1.0f / sqrtf(mean + eps);
#endif
}

/* y[t][i] = (x[t][i] * r_t) * w[i] with r_t from row t (reading R17). */
int oracle_rmsnorm(const float* x, const float* w, float eps, int nt, int id, float* y)
{
    if (!x || !w || !y || nt < 0 || id < 1 || !(eps >= 0.0f))
        return -1;
    for (int t = 0; t < nt; ++t) {
        const float* xr = x + (size_t)t * id;
        float* yr = y + (size_t)t * id;
        float r = rms_scale(rms_sum_squares(xr, id), id, eps);
        for (int i = 0; i < id; ++i)
            yr[i] = (xr[i] * r) * w[i];
    }
    return 0;
}

/* The residual update h_new = h + o (one f32 add per element), written to h_new,
 * then y = rmsnorm(h_new) as above. */
int oracle_add_rmsnorm(const float* h, const float* o, const float* w, float eps, int nt, int id,
                       float* h_new, float* y)
{
    if (!h || !o || !h_new)
        return -1;
    for (size_t i = 0; i < (size_t)nt * (size_t)(id > 0 ? id : 0); ++i)
        h_new[i] = h[i] + o[i];
    return oracle_rmsnorm(h_new, w, eps, nt, id, y);
}

/* y = silu(g) * u, silu(g) = g / (1 + e^-g) = g * sigmoid(g); reading R18: every
 * operation in f64 in that order, one rounding to f32 at the end. */
int oracle_silu_mul(const float* g, const float* u, size_t n, float* y)
{
    if (!g || !u || !y)
        return -1;
    for (size_t i = 0; i < n; ++i) {
        double gd = (double)g[i];
#if OQ_MUTATE == 9
        double e = exp(gd);
#else
        double e = exp(-gd);
#endif
        double sg = gd / (1.0 + e);
        y[i] = (float)(sg * (double)u[i]);
    }
    return 0;
}

/* ---- O4. Per-scale-group integer dots --------------------------------------
 * [GEMM, "The GPU path"]: a 32-weight Q4_K sub-block meets exactly one activation
 * scale and is reduced as sum(q * qx) in integers; Q6_K reduces per 16-weight
 * group.  Q4_K: S[t][r][b][j] = sum_{l<32} q(32j+l) * qx[t][256b+32j+l], codes
 * 0..15 uncentred.  Q6_K: S[t][r][b][g] = sum_{l<16} (q6(16g+l) - 32) *
 * qx[t][256b+16g+l]. */
static int32_t dot_q4k_sub(const q4k_block* w, const int8_t* qx, int j)
{
    int32_t acc = 0;
    for (int l = 0; l < 32; ++l)
        acc += w->q[32 * j + l] * (int32_t)qx[32 * j + l];
    return acc;
}

static int32_t dot_q6k_group(const q6k_block* w, const int8_t* qx, int g)
{
    int32_t acc = 0;
    for (int l = 0; l < 16; ++l) {
#if OQ_MUTATE == 2
        acc += w->q6[16 * g + l] * (int32_t)qx[16 * g + l];
#else
        acc += (w->q6[16 * g + l] - 32) * (int32_t)qx[16 * g + l];
#endif
    }
    return acc;
}

/* bytes per 256 weights */
static size_t blk_bytes(int type)
{
    switch (type) {
    case OQ_TYPE_Q4_K: return 144;
    case OQ_TYPE_Q6_K: return 210;
    case OQ_TYPE_Q6_K_P224: return 224;
    case OQ_TYPE_Q4_0: return 8 * 18;
    case OQ_TYPE_Q5_K: return 176;
    default: return 8 * 34;
    }
}
static int known_type(int type)
{
    return type == OQ_TYPE_Q4_K || type == OQ_TYPE_Q6_K || type == OQ_TYPE_Q6_K_P224 || type == OQ_TYPE_Q4_0 ||
           type == OQ_TYPE_Q8_0 || type == OQ_TYPE_Q5_K;
}
/* Q4_K and Q5_K: sub-blocks of 32 with a 6-bit scale and min, uncentred codes */
static int is_k4(int type) { return type == OQ_TYPE_Q4_K || type == OQ_TYPE_Q5_K; }
static int is_k6(int type) { return type == OQ_TYPE_Q6_K || type == OQ_TYPE_Q6_K_P224; }
static int is_b32(int type) { return type == OQ_TYPE_Q4_0 || type == OQ_TYPE_Q8_0; }

/* ---- O8. 32-weight block formats ------------------------------------------
 * Q4_0 ([CH03, section 3.2]): 18 bytes = f16 d, then 16 bytes in which byte l
 * holds element l in its low nibble and element l + 16 in its high nibble; the
 * stored nibble is round(v / d) + 8, so w = d * (nibble - 8).  Q8_0 (R20): 34
 * bytes = f16 d, then 32 int8 codes, w = d * q.  A group is eight consecutive
 * blocks (256 weights); codes are returned centred (Q4_0: nibble - 8). */
typedef struct {
    double d[8];
    int q[256];
} b32_group;

static void b32_decode(int type, const uint8_t* B, b32_group* o)
{
    for (int j = 0; j < 8; ++j) {
        if (type == OQ_TYPE_Q4_0) {
            const uint8_t* b = B + 18 * j;
            o->d[j] = f16_bits_to_f64(rd_u16(b));
            for (int l = 0; l < 16; ++l) {
#if OQ_MUTATE == 13
                o->q[32 * j + 2 * l] = (b[2 + l] & 0xF) - 8;
                o->q[32 * j + 2 * l + 1] = (b[2 + l] >> 4) - 8;
#elif OQ_MUTATE == 12
                o->q[32 * j + l] = b[2 + l] & 0xF;
                o->q[32 * j + 16 + l] = b[2 + l] >> 4;
#else
                o->q[32 * j + l] = (b[2 + l] & 0xF) - 8;
                o->q[32 * j + 16 + l] = (b[2 + l] >> 4) - 8;
#endif
            }
        } else {
            const uint8_t* b = B + 34 * j;
            o->d[j] = f16_bits_to_f64(rd_u16(b));
            for (int l = 0; l < 32; ++l)
                o->q[32 * j + l] = (int8_t)b[2 + l];
        }
    }
}

static int32_t dot_b32(const b32_group* w, const int8_t* qx, int j)
{
    int32_t acc = 0;
    for (int l = 0; l < 32; ++l)
        acc += w->q[32 * j + l] * (int32_t)qx[32 * j + l];
    return acc;
}

int oracle_subblock_dots(int type, const uint8_t* W, const int8_t* q, int nt, int od, int id,
                         int32_t* S)
{
    if (!W || !q || !S || nt < 0 || od < 0 || id < 0 || id % 256)
        return -1;
    if (!known_type(type))
        return -2;
    int nsb = id / 256;
    int ng = is_k6(type) ? 16 : 8;
    size_t bb = blk_bytes(type);
#pragma omp parallel for schedule(static)
    for (int r = 0; r < od; ++r) {
        for (int b = 0; b < nsb; ++b) {
            const uint8_t* B = W + ((size_t)r * nsb + b) * bb;
            q4k_block w4;
            q6k_block w6;
            b32_group w3;
            if (is_k4(type))
                k4_decode(type, B, &w4);
            else if (is_k6(type))
                q6k_decode(B, &w6);
            else
                b32_decode(type, B, &w3);
            for (int t = 0; t < nt; ++t) {
                const int8_t* qx = q + (size_t)t * id + 256 * b;
                int32_t* dst = S + (((size_t)t * od + r) * nsb + b) * ng;
                for (int g = 0; g < ng; ++g)
                    dst[g] = is_k4(type) ? dot_q4k_sub(&w4, qx, g)
                             : is_k6(type)        ? dot_q6k_group(&w6, qx, g)
                                                  : dot_b32(&w3, qx, g);
            }
        }
    }
    return 0;
}

/* ---- O5. Combine one output ------------------------------------------------
 * [GEMM, "The GPU path"]: sum w x = d*sc*dx * sum(q*qx) - dmin*m * (dx*sum(qx)) per
 * 32-weight sub-block; the second factor of the min term is the stored s.
 * [GEMM, "Weights: 8 rows per register"]: the mins stay out of the integer
 * loop.  Q6_K: d*sc_g*dx * sum((q6-32)*qx), dx the scale of the 32-block holding
 * group g.  Every term in f64, summed in f64, one rounding to f32 at the end.
 * mag receives sum |term| (used for the comparison tolerance). */
static void one_output(int type, const uint8_t* Wrow, const int8_t* qx_t, const float* d_t,
                       const float* s_t, int nsb, float* out, double* mag)
{
    double acc = 0.0, am = 0.0;
    size_t bb = blk_bytes(type);
    for (int b = 0; b < nsb; ++b) {
        const uint8_t* B = Wrow + (size_t)b * bb;
        const int8_t* qx = qx_t + 256 * b;
        if (is_k4(type)) {
            q4k_block w;
            k4_decode(type, B, &w);
            for (int j = 0; j < 8; ++j) {
                double dx = (double)d_t[8 * b + j];
                double sx = (double)s_t[8 * b + j];
                double S = (double)dot_q4k_sub(&w, qx, j);
                double tmain = (w.d * (double)w.sc[j]) * dx * S;
#if OQ_MUTATE == 3
                double tmin = 0.0 * sx;
#else
                double tmin = (w.dmin * (double)w.m[j]) * sx;
#endif
                acc += tmain - tmin;
                am += fabs(tmain) + fabs(tmin);
            }
        } else if (is_b32(type)) {
            /* 32-weight blocks: d_w * dx * sum(qc * qx), codes centred -- exact, no
             * stored sum enters */
            b32_group w;
            b32_decode(type, B, &w);
            for (int j = 0; j < 8; ++j) {
                double tm = w.d[j] * (double)d_t[8 * b + j] * (double)dot_b32(&w, qx, j);
                acc += tm;
                am += fabs(tm);
            }
        } else {
            q6k_block w;
            q6k_decode(B, &w);
            for (int g = 0; g < 16; ++g) {
                double dx = (double)d_t[8 * b + g / 2];
                double S = (double)dot_q6k_group(&w, qx, g);
#if OQ_MUTATE == 5
                double tm = (w.d * (double)w.sc[g / 2]) * dx * S;
#else
                double tm = (w.d * (double)w.sc[g]) * dx * S;
#endif
                acc += tm;
                am += fabs(tm);
            }
        }
    }
    *out = (float)acc;
    if (mag)
        *mag = am;
}

int oracle_matmul_q8(int type, const uint8_t* W, const int8_t* q, const float* d, const float* s,
                     int nt, int od, int id, float* out, double* mag)
{
    if (!W || !q || !d || !s || !out || nt < 0 || od < 0 || id < 0 || id % 256)
        return -1;
    if (!known_type(type))
        return -2;
    int nsb = id / 256;
    size_t row_bytes = (size_t)nsb * blk_bytes(type);
    long total = (long)nt * od;
#pragma omp parallel for schedule(static)
    for (long e = 0; e < total; ++e) {
        int t = (int)(e / od), r = (int)(e % od);
        one_output(type, W + (size_t)r * row_bytes, q + (size_t)t * id, d + (size_t)t * (id / 32),
                   s + (size_t)t * (id / 32), nsb, out + (size_t)t * od + r, mag ? mag + (size_t)t * od + r : NULL);
    }
    return 0;
}

/* ---- O7. Q8_K activations (one scale per 256 values) ----------------------
 * [GEMM, "Activations: int8 with a scale per 256"]: each activation row is
 * quantized to int8 with one f32 scale per 256 values, and the sum of every group
 * of 16 values is kept as a float; [GEMM, "The zero points do not touch the inner
 * loop"]: the Q4_K min term is dmin * m times the activation sum of the
 * sub-block, taken from those stored sums.  Reading R19.  Per token t, block b of
 * 256: amax = max |x|; d = amax / 127; q = roundf(x / d); bsum[g] = sum of the 16
 * codes of group g (exact integer, stored as f32). */
int oracle_quantize_q8k(const float* x, int nt, int id, int8_t* q, float* d, float* bsum)
{
    if (!x || !q || !d || !bsum || nt < 0 || id < 0 || id % 256)
        return -1;
    int nsb = id / 256;
    for (int t = 0; t < nt; ++t) {
        for (int b = 0; b < nsb; ++b) {
            const float* xb = x + (size_t)t * id + 256 * b;
            int8_t* qb = q + (size_t)t * id + 256 * b;
            float amax = 0.0f;
#if OQ_MUTATE == 10
            for (int i = 0; i < 32; ++i) {
#else
            for (int i = 0; i < 256; ++i) {
#endif
                float a = fabsf(xb[i]);
                if (a > amax)
                    amax = a;
            }
            float db = amax / 127.0f;
            for (int i = 0; i < 256; ++i) {
                int qi = 0;
                if (db != 0.0f) {
                    float r = roundf(xb[i] / db);
                    if (r > 127.0f || r < -127.0f) {
                        if (OQ_MUTATE != 10)
                            return -2; /* cannot happen: |x| <= amax */
                        r = r > 0 ? 127.0f : -127.0f;
                    }
                    qi = (int)r;
                }
                qb[i] = (int8_t)qi;
            }
            d[(size_t)t * nsb + b] = db;
            for (int g = 0; g < 16; ++g) {
                int sum = 0;
                for (int l = 0; l < 16; ++l)
                    sum += qb[16 * g + l];
                bsum[(size_t)t * (id / 16) + 16 * b + g] = (float)sum;
            }
        }
    }
    return 0;
}

/* One output from Q8_K activations.  Q4_K, per super-block b and sub-block j:
 *   d * sc_j * dx_b * sum(q * qx)  -  dmin * m_j * dx_b * (bsum_{2j} + bsum_{2j+1});
 * Q6_K, per group g: d * sc_g * dx_b * sum((q6 - 32) * qx).  Every term in f64,
 * summed in f64, one rounding to f32; mag = sum |term|. */
static void one_output_q8k(int type, const uint8_t* Wrow, const int8_t* qx_t, const float* d_t,
                           const float* bs_t, int nsb, float* out, double* mag)
{
    double acc = 0.0, am = 0.0;
    size_t bb = blk_bytes(type);
    for (int b = 0; b < nsb; ++b) {
        const uint8_t* B = Wrow + (size_t)b * bb;
        const int8_t* qx = qx_t + 256 * b;
        double dx = (double)d_t[b];
        if (is_k4(type)) {
            q4k_block w;
            k4_decode(type, B, &w);
            for (int j = 0; j < 8; ++j) {
#if OQ_MUTATE == 11
                double bs = 2.0 * (double)bs_t[16 * b + 2 * j];
#else
                double bs = (double)bs_t[16 * b + 2 * j] + (double)bs_t[16 * b + 2 * j + 1];
#endif
                double tmain = (w.d * (double)w.sc[j]) * dx * (double)dot_q4k_sub(&w, qx, j);
                double tmin = (w.dmin * (double)w.m[j]) * dx * bs;
                acc += tmain - tmin;
                am += fabs(tmain) + fabs(tmin);
            }
        } else {
            q6k_block w;
            q6k_decode(B, &w);
            for (int g = 0; g < 16; ++g) {
                double tm = (w.d * (double)w.sc[g]) * dx * (double)dot_q6k_group(&w, qx, g);
                acc += tm;
                am += fabs(tm);
            }
        }
    }
    *out = (float)acc;
    if (mag)
        *mag = am;
}

int oracle_matmul_q8k(int type, const uint8_t* W, const int8_t* q, const float* d, const float* bsum,
                      int nt, int od, int id, float* out, double* mag)
{
    if (!W || !q || !d || !bsum || !out || nt < 0 || od < 0 || id < 0 || id % 256)
        return -1;
    if (!known_type(type) || is_b32(type))
        return -2;
    int nsb = id / 256;
    size_t row_bytes = (size_t)nsb * blk_bytes(type);
    long total = (long)nt * od;
#pragma omp parallel for schedule(static)
    for (long e = 0; e < total; ++e) {
        int t = (int)(e / od), r = (int)(e % od);
        one_output_q8k(type, W + (size_t)r * row_bytes, q + (size_t)t * id, d + (size_t)t * nsb,
                       bsum + (size_t)t * (id / 16), nsb, out + (size_t)t * od + r,
                       mag ? mag + (size_t)t * od + r : NULL);
    }
    return 0;
}

/* The integer stage of the Q8_K matmul: per token t, row r, super-block b,
 *   S[..][0] = sum_j sc_j * sum(q * qx)                     (Q4_K; Q6_K: sum_g sc_g *
 *              sum((q6 - 32) * qx)),
 *   S[..][1] = sum_j m_j * (bsum_{2j} + bsum_{2j+1})         (Q4_K; Q6_K: 0),
 * exact integers (the group sums are integers stored as f32).  S: [nt][od][id/256][2]. */
int oracle_q8k_superblock_sums(int type, const uint8_t* W, const int8_t* q, const float* bsum, int nt, int od,
                               int id, int32_t* S)
{
    if (!W || !q || !bsum || !S || nt < 0 || od < 0 || id < 0 || id % 256)
        return -1;
    if (!known_type(type) || is_b32(type))
        return -2;
    int nsb = id / 256;
    size_t bb = blk_bytes(type);
#pragma omp parallel for schedule(static)
    for (int r = 0; r < od; ++r) {
        for (int b = 0; b < nsb; ++b) {
            const uint8_t* B = W + ((size_t)r * nsb + b) * bb;
            q4k_block w4;
            q6k_block w6;
            if (is_k4(type))
                k4_decode(type, B, &w4);
            else
                q6k_decode(B, &w6);
            for (int t = 0; t < nt; ++t) {
                const int8_t* qx = q + (size_t)t * id + 256 * b;
                const float* bs = bsum + (size_t)t * (id / 16) + 16 * b;
                long s1 = 0, s2 = 0;
                if (is_k4(type)) {
                    for (int j = 0; j < 8; ++j) {
                        s1 += (long)w4.sc[j] * dot_q4k_sub(&w4, qx, j);
                        s2 += (long)w4.m[j] * ((long)bs[2 * j] + (long)bs[2 * j + 1]);
                    }
                } else {
                    for (int g = 0; g < 16; ++g)
                        s1 += (long)w6.sc[g] * dot_q6k_group(&w6, qx, g);
                }
                int32_t* dst = S + (((size_t)t * od + r) * nsb + b) * 2;
                dst[0] = (int32_t)s1;
                dst[1] = (int32_t)s2;
            }
        }
    }
    return 0;
}

/* Selected outputs only, as oracle_matmul_q8_points. */
int oracle_matmul_q8k_points(int type, const uint8_t* W, const int8_t* q, const float* d, const float* bsum,
                             int nt, int od, int id, int n, const int* t_idx, const int* r_idx, float* out,
                             double* mag)
{
    if (!W || !q || !d || !bsum || !out || !t_idx || !r_idx || nt < 0 || od < 0 || id < 0 || id % 256 || n < 0)
        return -1;
    if (!known_type(type) || is_b32(type))
        return -2;
    int nsb = id / 256;
    size_t row_bytes = (size_t)nsb * blk_bytes(type);
#pragma omp parallel for schedule(static)
    for (int k = 0; k < n; ++k) {
        int t = t_idx[k], r = r_idx[k];
        if (t < 0 || t >= nt || r < 0 || r >= od) {
            out[k] = 0.0f;
            if (mag)
                mag[k] = -1.0;
            continue;
        }
        one_output_q8k(type, W + (size_t)r * row_bytes, q + (size_t)t * id, d + (size_t)t * nsb,
                       bsum + (size_t)t * (id / 16), nsb, out + k, mag ? mag + k : NULL);
    }
    return 0;
}

/* Selected outputs only: out[k] = output (t_idx[k], r_idx[k]). */
int oracle_matmul_q8_points(int type, const uint8_t* W, const int8_t* q, const float* d, const float* s,
                            int nt, int od, int id, int npts, const int* t_idx, const int* r_idx,
                            float* out, double* mag)
{
    if (!W || !q || !d || !s || !out || !t_idx || !r_idx || id % 256 || npts < 0)
        return -1;
    if (!known_type(type))
        return -2;
    int nsb = id / 256;
    size_t row_bytes = (size_t)nsb * blk_bytes(type);
    for (int k = 0; k < npts; ++k)
        if (t_idx[k] < 0 || t_idx[k] >= nt || r_idx[k] < 0 || r_idx[k] >= od)
            return -3;
#pragma omp parallel for schedule(static)
    for (int k = 0; k < npts; ++k) {
        int t = t_idx[k], r = r_idx[k];
        one_output(type, W + (size_t)r * row_bytes, q + (size_t)t * id, d + (size_t)t * (id / 32),
                   s + (size_t)t * (id / 32), nsb, out + k, mag ? mag + k : NULL);
    }
    return 0;
}

/* The whole path: quantize the activations, then combine.  q, d, s are scratch
 * buffers the caller provides (nt*id int8, nt*id/32 floats each). */
int oracle_matmul(int type, const uint8_t* W, const float* x, int nt, int od, int id, int8_t* q,
                  float* d, float* s, float* out, double* mag)
{
    int rc = oracle_quantize(x, nt, id, q, d, s);
    if (rc)
        return rc;
    return oracle_matmul_q8(type, W, q, d, s, nt, od, id, out, mag);
}

/* Decoded fields of one super-block, for the pins: Q4_K fills d, dmin, sc[8], m[8],
 * codes[256]; Q6_K fills d, sc[16], codes[256] (stored 0..63). */
int oracle_decode_block(int type, const uint8_t* B, double* d, double* dmin, int* sc, int* m, int* codes)
{
    if (is_k4(type)) {
        q4k_block w;
        k4_decode(type, B, &w);
        *d = w.d;
        *dmin = w.dmin;
        memcpy(sc, w.sc, sizeof w.sc);
        memcpy(m, w.m, sizeof w.m);
        memcpy(codes, w.q, sizeof w.q);
        return 0;
    }
    if (type == OQ_TYPE_Q6_K || type == OQ_TYPE_Q6_K_P224) {
        q6k_block w;
        q6k_decode(B, &w);
        *d = w.d;
        *dmin = 0.0;
        memcpy(sc, w.sc, sizeof w.sc);
        memcpy(codes, w.q6, sizeof w.q6);
        return 0;
    }
    return -2;
}

/* Decoded group of eight 32-weight blocks (types 4, 5): d[8], centred codes[256]. */
int oracle_decode_group32(int type, const uint8_t* B, double* d, int* codes)
{
    if (!is_b32(type))
        return -2;
    b32_group w;
    b32_decode(type, B, &w);
    memcpy(d, w.d, sizeof w.d);
    memcpy(codes, w.q, sizeof w.q);
    return 0;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
