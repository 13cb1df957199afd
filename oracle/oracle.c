/*
 * CPU oracle for block-quantized weight GEMV / MoE / prefill (Q4_0, Q8_0).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this file's library.  The product path (the HIP
 * library and its Python binding) never calls it, and this file shares no
 * code with that library: its binary16 codec, its quantizer and its parser of
 * the packed bytes are written here from the format definition alone.
 *
 * Everything is plain fp64 loops in the order the definitions state.  The
 * only parallelism is an OpenMP loop over independent output rows, which
 * changes no arithmetic.
 *
 * ORC_PLANT_* macros build deliberately broken copies for the tests that show
 * the pins catch plausible mistakes (a swapped nibble order, a dropped offset,
 * the wrong tie rule or divisor, a shifted index, a dropped term, a codec
 * slip, a sign slip in silu, gate and up swapped, the activation quantizer's
 * tie rule, a shifted activation scale).  The default build defines none of
 * them.
 *
 * What is computed, and where it is defined:
 *  - Q4_0 block: 32 weights share one binary16 scale d and carry 4-bit codes
 *    q; the weight is (q - 8) * d.  Byte j of a block's 16 code bytes holds
 *    element j in its low nibble and element j + 16 in its high nibble (the
 *    GGUF Q4_0 layout with group size 32) [sm8x-bench, "our kernel" and the
 *    Q4_0 table; volta-kernel-bakeoff, "What's in the race"].
 *  - Quantizer: d = fp16(fl32(absmax / 7)); q = clamp(round(w / d) + 8, 0, 15)
 *    with round half away from zero and w / d taken in fp64 against the
 *    stored binary16 d; an all-zero (or underflowing) block has d = 0, q = 8.
 *  - Q8_0 block: 32 int8 codes q and one binary16 scale d, weight q * d;
 *    d = fp16(fl32(absmax / 127)), q = clamp(round(w / d), -127, 127)
 *    [H100-KERNEL-5X-ROADMAP, "Why the decode gap is bandwidth" and Lever 1
 *    (int8 codes plus a per-block scale); the scale is binary16 here].
 *  - GEMV: y[m][n] = sum_k w[n][k] * x[m][k] in fp64 on the exactly
 *    dequantized weights, plus s[m][n] = sum_k |w[n][k] * x[m][k]| for the
 *    acceptance bound [volta-kernel-bakeoff, "Making it fair": a CPU
 *    double-precision reference of the same quantized weights].
 *  - MoE: expert e uses pool matrix idx[e] and its own token x[e]
 *    [volta-kernel-bakeoff, "What's in the race" (moe_*) and "Making it fair"].
 *  - Prefill: the GEMV definition for M token rows (same sums).
 *  - fp32 activations: each is rounded to binary16 (nearest, ties to even,
 *    overflow to infinity) and the GEMV definition applies to the rounded
 *    values [volta-kernel-bakeoff, "Results", the like-for-like bullets:
 *    fp32 activations in, their conversion counted; values beyond binary16's
 *    range become infinity].
 *  - SwiGLU on a stacked table: rows 0..N-1 of one packed 2N x K matrix are
 *    the gate rows, rows N..2N-1 the up rows; the output is silu(g) * u with
 *    g, u the two GEMVs and silu(v) = v / (1 + e^-v) [volta-kernel-bakeoff,
 *    "Results", the few-tokens bullet: gate and up stacked into one table,
 *    the activations converted once; the FFN fusion step of the CUDA-kernel
 *    diary: gate, up and SwiGLU in one kernel, the activations read once].
 *  - Plain 2-bit block (q2w): 32 weights share one binary16 scale d and
 *    carry codes c in -2..1, the weight is c * d; stored as u = c + 2 in two
 *    bits, byte j of the block's 8 code bytes holding elements j, j + 8,
 *    j + 16, j + 24 in bits 0-1, 2-3, 4-5, 6-7 (2.5 bits per weight)
 *    [volta-kernel-bakeoff, "What's in the race": q2w, codes -2..1, one fp16
 *    scale per 32].  The pages give no quantizer; the reading here: m = the
 *    block's weight of largest magnitude (the first on ties), d =
 *    fp16(fl32(m / -2)), so m lands exactly on code -2 and all four codes are
 *    used, c = clamp(round(w / d), -2, 1) with w / d in fp64 against the
 *    stored d and round half away from zero as for Q4_0; d = 0 gives c = 0.
 *  - 8-bit activations: each 32-block of a token's fp16 activations becomes
 *    int8 codes qx with one binary32 scale dx: amax = the block's largest
 *    |x|, dx = amax / 127 and inv = 127 / amax (binary32 divisions),
 *    qx = rint(x * inv) with a binary32 product and ties to even (an
 *    all-zero block: qx = 0, dx = 0).  The GEMV then takes, per block, the
 *    exact integer sum of (q - 8) * qx times dw * dx [sm8x-bench, "our
 *    kernel": the activations quantized to 8-bit blocks once, then an int8
 *    dot with 4-way multiply-accumulate; the pages fix neither the rounding
 *    nor the precision of that quantizer, so both are this reading's, taken
 *    in binary32 as the kernel takes them].
 *
 * Packed buffer layout (one N x K matrix, K % 32 == 0, blocks along K, block
 * index i = n * (K / 32) + b):
 *   codes  : at byte 0; 16 bytes per Q4_0 block / 32 per Q8_0 block / 8 per
 *            q2w block, block i at byte 16 * i / 32 * i / 8 * i.  Q8_0 codes
 *            are two's complement int8.
 *   scales : binary16 little-endian, scale i at byte S0 + 2 * i, where S0 is
 *            the code-region size rounded up to a multiple of 256.
 *   total  : (S0 + 2 * N * K / 32) rounded up to a multiple of 256.
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define ORC_Q4_0 0
#define ORC_Q8_0 1
#define ORC_Q2W 2

/* ---------------------------------------------------------------- binary16 */

/* Decode IEEE 754 binary16 bits to the exact double value. */
double orc_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
#if defined(ORC_PLANT_HALF)
        v = ldexp((double)(1024 + m), -24);
#else
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
#endif
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);     /* 1.m * 2^(e-15) */
    return sign ? -v : v;
}

/* Round a double to the nearest binary16, ties to even, subnormals kept,
 * overflow to infinity.  rint() rounds to nearest-even in the default mode. */
uint16_t orc_double_to_half(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (isnan(v))
        return (uint16_t)(sign | 0x7e00u);
    /* 65520 lies half-way between 65504 (odd mantissa) and 2^16: rounds up */
    if (a >= 65520.0)
        return (uint16_t)(sign | 0x7c00u);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: quantum 2^-24; a result of 1024 is the smallest
         * normal, whose bit pattern is exactly 1024 as well */
        double r = rint(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)r);
    }
    int e2;
    frexp(a, &e2);                  /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;                 /* a in [2^E, 2^(E+1)) */
    double r = rint(ldexp(a, 10 - E));   /* significand scaled to [1024, 2048] */
    if (r >= 2048.0) {
        r = 1024.0;
        E += 1;
    }
    int biased = E + 15;
    if (biased >= 31)
        return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | (uint16_t)(biased << 10) | (uint16_t)((int)r - 1024));
}

uint16_t orc_float_to_half(float f) { return orc_double_to_half((double)f); }

/* ------------------------------------------------------------- the layout */

static size_t round256(size_t v) { return (v + 255u) & ~(size_t)255u; }

static size_t code_bytes_per_block(int fmt) { return fmt == ORC_Q4_0 ? 16u : fmt == ORC_Q2W ? 8u : 32u; }

size_t orc_packed_bytes(int fmt, int64_t N, int64_t K)
{
    if (N <= 0 || K <= 0 || K % 32 != 0 || (fmt != ORC_Q4_0 && fmt != ORC_Q8_0 && fmt != ORC_Q2W))
        return 0;
    size_t nb = (size_t)N * (size_t)(K / 32);
    size_t s0 = round256(nb * code_bytes_per_block(fmt));
    return round256(s0 + 2u * nb);
}

static size_t scale_offset(int fmt, int64_t N, int64_t K)
{
    size_t nb = (size_t)N * (size_t)(K / 32);
    return round256(nb * code_bytes_per_block(fmt));
}

/* Signed weight multiplier of element k (0..31) of block i:
 * Q4_0 -> q - 8, Q8_0 -> q, q2w -> u - 2. */
static int code_value(int fmt, const uint8_t *p, size_t i, int k)
{
    if (fmt == ORC_Q2W) {
        const uint8_t *blk = p + 8u * i;
#if defined(ORC_PLANT_Q2ORDER)
        int u = (blk[k / 4] >> (2 * (k % 4))) & 3;
#else
        int u = (blk[k % 8] >> (2 * (k / 8))) & 3;
#endif
        return u - 2;
    }
    if (fmt == ORC_Q4_0) {
        const uint8_t *blk = p + 16u * i;
#if defined(ORC_PLANT_NIBBLE)
        int q = (k < 16) ? (blk[k] >> 4) : (blk[k - 16] & 0x0f);
#else
        int q = (k < 16) ? (blk[k] & 0x0f) : (blk[k - 16] >> 4);
#endif
#if defined(ORC_PLANT_OFFSET)
        return q;
#else
        return q - 8;
#endif
    }
    const uint8_t *blk = p + 32u * i;
    return (int)(int8_t)blk[k];
}

static double scale_value(int fmt, const uint8_t *p, int64_t N, int64_t K, size_t i)
{
#if defined(ORC_PLANT_SCALEIDX)
    if (i + 1 < (size_t)N * (size_t)(K / 32)) i += 1;
#endif
    const uint8_t *s = p + scale_offset(fmt, N, K) + 2u * i;
    uint16_t h = (uint16_t)(s[0] | (s[1] << 8));
    return orc_half_to_double(h);
}

/* ------------------------------------------------------------- quantizer */

/* One q2w block (the reading in the header): codes into c[8], scale bits
 * into *d16; sets *err to 4 for a non-finite weight or scale. */
static void quantize_q2w_block(const float *blk, uint8_t *c, uint16_t *d16, int *err)
{
    float m = 0.0f;
    for (int k = 0; k < 32; ++k) {
        if (!isfinite(blk[k]))
            *err = 4;
        if (fabsf(blk[k]) > fabsf(m))
            m = blk[k];
    }
    float d32 = m / -2.0f;   /* binary32 division */
    *d16 = orc_float_to_half(d32);
    if ((*d16 & 0x7c00u) == 0x7c00u)
        *err = 4;
    double d = orc_half_to_double(*d16);
    int u[32];
    for (int k = 0; k < 32; ++k) {
        int v = 0;
        if (d != 0.0 && isfinite(d)) {
            double r = round((double)blk[k] / d);   /* half away from zero */
            if (r > 1.0) r = 1.0;
            if (r < -2.0) r = -2.0;
            v = (int)r;
        }
        u[k] = v + 2;
    }
    for (int j = 0; j < 8; ++j)
        c[j] = (uint8_t)(u[j] | (u[j + 8] << 2) | (u[j + 16] << 4) | (u[j + 24] << 6));
}

/* Returns 0 on success, 4 (range error) if a weight is non-finite or a scale
 * overflows binary16, 2 on a bad shape, 5 if `out_bytes` is too small. */
int orc_quantize(int fmt, const float *w, int64_t N, int64_t K, uint8_t *out, size_t out_bytes)
{
    size_t need = orc_packed_bytes(fmt, N, K);
    if (need == 0)
        return 2;
    if (out_bytes < need)
        return 5;
    memset(out, 0, need);
    const int qmax = (fmt == ORC_Q4_0) ? 7 : 127;
    const int64_t KB = K / 32;
    size_t s0 = scale_offset(fmt, N, K);
    int err = 0;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < KB; ++b) {
            const float *blk = w + n * K + b * 32;
            size_t i = (size_t)(n * KB + b);
            if (fmt == ORC_Q2W) {
                uint16_t d2;
                quantize_q2w_block(blk, out + 8u * i, &d2, &err);
                out[s0 + 2u * i] = (uint8_t)(d2 & 0xff);
                out[s0 + 2u * i + 1] = (uint8_t)(d2 >> 8);
                continue;
            }
            float a = 0.0f;
            for (int k = 0; k < 32; ++k) {
                if (!isfinite(blk[k]))
                    err = 4;
                float m = fabsf(blk[k]);
                if (m > a)
                    a = m;
            }
            float d32 = a / (float)qmax;          /* binary32 division */
            uint16_t d16 = orc_float_to_half(d32);
            if ((d16 & 0x7c00u) == 0x7c00u)
                err = 4;
            double d = orc_half_to_double(d16);
            int q[32];
            for (int k = 0; k < 32; ++k) {
                int v;
                if (d == 0.0 || !isfinite(d)) {
                    v = 0;
                } else {
#if defined(ORC_PLANT_ROUND)
                    double r = rint((double)blk[k] / d);
#elif defined(ORC_PLANT_D32)
                    double r = round((double)blk[k] / (double)d32);
#else
                    double r = round((double)blk[k] / d);   /* half away from zero */
#endif
                    if (r > qmax) r = qmax;
                    if (r < -qmax - (fmt == ORC_Q4_0 ? 1 : 0)) r = -qmax - (fmt == ORC_Q4_0 ? 1 : 0);
                    v = (int)r;
                }
                q[k] = v;
            }
            if (fmt == ORC_Q4_0) {
                uint8_t *c = out + 16u * i;
                for (int j = 0; j < 16; ++j)
                    c[j] = (uint8_t)((q[j] + 8) | ((q[j + 16] + 8) << 4));
            } else {
                uint8_t *c = out + 32u * i;
                for (int k = 0; k < 32; ++k)
                    c[k] = (uint8_t)(int8_t)q[k];
            }
            out[s0 + 2u * i] = (uint8_t)(d16 & 0xff);
            out[s0 + 2u * i + 1] = (uint8_t)(d16 >> 8);
        }
    }
    return err;
}

/* ----------------------------------------------------------- dequantizer */

/* Exact dequantized value of every weight as double: (q - 8) * d or q * d. */
void orc_dequant_f64(int fmt, const uint8_t *p, int64_t N, int64_t K, double *out)
{
    const int64_t KB = K / 32;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < KB; ++b) {
            size_t i = (size_t)(n * KB + b);
            double d = scale_value(fmt, p, N, K, i);
            for (int k = 0; k < 32; ++k)
                out[n * K + b * 32 + k] = (double)code_value(fmt, p, i, k) * d;
        }
}

/* binary32 output: the exact value is representable (at most 15 significant
 * bits for Q4_0, 18 for Q8_0), so the conversion does not round. */
void orc_dequant_f32(int fmt, const uint8_t *p, int64_t N, int64_t K, float *out)
{
    const int64_t KB = K / 32;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < KB; ++b) {
            size_t i = (size_t)(n * KB + b);
            double d = scale_value(fmt, p, N, K, i);
            for (int k = 0; k < 32; ++k)
                out[n * K + b * 32 + k] = (float)((double)code_value(fmt, p, i, k) * d);
        }
}

/* binary16 output bits: the exact value rounded to nearest-even. */
void orc_dequant_f16(int fmt, const uint8_t *p, int64_t N, int64_t K, uint16_t *out)
{
    const int64_t KB = K / 32;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < KB; ++b) {
            size_t i = (size_t)(n * KB + b);
            double d = scale_value(fmt, p, N, K, i);
            for (int k = 0; k < 32; ++k)
                out[n * K + b * 32 + k] = orc_double_to_half((double)code_value(fmt, p, i, k) * d);
        }
}

/* ----------------------------------------------------------------- GEMV */

/* One output element: row n of the packed matrix against token row xm. */
static void dot_row(int fmt, const uint8_t *p, int64_t N, int64_t K, int64_t n,
                    const uint16_t *xm, double *y, double *s)
{
    const int64_t KB = K / 32;
    double acc = 0.0, sabs = 0.0;
#if defined(ORC_PLANT_DROP)
    for (int64_t b = 0; b + 1 < KB; ++b) {
#else
    for (int64_t b = 0; b < KB; ++b) {
#endif
        size_t i = (size_t)(n * KB + b);
        double d = scale_value(fmt, p, N, K, i);
        for (int k = 0; k < 32; ++k) {
            double w = (double)code_value(fmt, p, i, k) * d;
#if defined(ORC_PLANT_XINDEX)
            double x = orc_half_to_double(xm[b * 32 + (k ^ 1)]);
#else
            double x = orc_half_to_double(xm[b * 32 + k]);
#endif
            double t = w * x;
            acc += t;
            sabs += fabs(t);
        }
    }
    *y = acc;
    *s = sabs;
}

/* y[m][n], s[m][n] for all N rows and M tokens (x is binary16 bits [M][K]). */
void orc_gemv(int fmt, const uint8_t *p, int64_t N, int64_t K, const uint16_t *x, int64_t M,
              double *y, double *s)
{
    for (int64_t m = 0; m < M; ++m) {
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < N; ++n)
            dot_row(fmt, p, N, K, n, x + m * K, &y[m * N + n], &s[m * N + n]);
    }
}

/* The same definition on a chosen subset of rows: y[m][r], s[m][r] for
 * row rows[r], r < R.  Used to check large matrices on sampled outputs. */
void orc_gemv_rows(int fmt, const uint8_t *p, int64_t N, int64_t K, const uint16_t *x, int64_t M,
                   const int64_t *rows, int64_t R, double *y, double *s)
{
    for (int64_t m = 0; m < M; ++m) {
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < R; ++r)
            dot_row(fmt, p, N, K, rows[r], x + m * K, &y[m * R + r], &s[m * R + r]);
    }
}

/* MoE: expert e multiplies pool matrix idx[e] (stride = packed bytes of one
 * N x K matrix) with its own token x[e]; y, s are [E][N]. */
void orc_moe(int fmt, const uint8_t *pool, int64_t P, const int32_t *idx, int64_t E,
             const uint16_t *x, int64_t N, int64_t K, double *y, double *s)
{
    size_t stride = orc_packed_bytes(fmt, N, K);
    for (int64_t e = 0; e < E; ++e) {
        int64_t j = idx[e];
        if (j < 0 || j >= P) {
            for (int64_t n = 0; n < N; ++n) {
                y[e * N + n] = NAN;
                s[e * N + n] = NAN;
            }
            continue;
        }
        orc_gemv(fmt, pool + (size_t)j * stride, N, K, x + e * K, 1, y + e * N, s + e * N);
    }
}

/* ------------------------------------------------ fp32 input and SwiGLU */

/* Round n fp32 activations to binary16 bits (the codec above). */
void orc_floats_to_half(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_float_to_half(x[i]);
}

/* silu(v) = v * sigmoid(v) = v / (1 + e^-v). */
double orc_silu(double v)
{
#if defined(ORC_PLANT_SILU)
    return v / (1.0 + exp(v));
#else
    return v / (1.0 + exp(-v));
#endif
}

/* y[i] = silu(g[i]) * u[i] for the gate and up halves of a stacked GEMV. */
void orc_swiglu(const double *g, const double *u, int64_t n, double *y)
{
    for (int64_t i = 0; i < n; ++i)
#if defined(ORC_PLANT_GLU)
        y[i] = orc_silu(u[i]) * g[i];
#else
        y[i] = orc_silu(g[i]) * u[i];
#endif
}

/* ------------------------------------------------------ 8-bit activations */

/* Quantize M x K fp16 activations (bits) per 32-block: qx int8 [M][K],
 * dx binary32 [M][K / 32] (the definition in the header).  Every step is one
 * IEEE binary32 operation, as written. */
void orc_quantize_act8(const uint16_t *x, int64_t M, int64_t K, int8_t *qx, float *dx)
{
    const int64_t KB = K / 32;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t b = 0; b < KB; ++b) {
            const uint16_t *xb = x + m * K + b * 32;
            float v[32];
            float amax = 0.0f;
            for (int k = 0; k < 32; ++k) {
                v[k] = (float)orc_half_to_double(xb[k]);   /* exact */
                float a = fabsf(v[k]);
                if (a > amax)
                    amax = a;
            }
            float d = 0.0f, inv = 0.0f;
            if (amax > 0.0f) {
                d = amax / 127.0f;
                inv = 127.0f / amax;
            }
            for (int k = 0; k < 32; ++k) {
                float t = v[k] * inv;
#if defined(ORC_PLANT_ACTROUND)
                float r = roundf(t);
#else
                float r = rintf(t);
#endif
                if (r > 127.0f)
                    r = 127.0f;
                if (r < -127.0f)
                    r = -127.0f;
                qx[m * K + b * 32 + k] = (int8_t)r;
            }
            dx[m * KB + b] = d;
        }
}

/* Q4_0 (or q2w) weights against 8-bit activations (qx, dx from
 * orc_quantize_act8):
 *   y[m][n] = sum_b dw[n][b] * dx[m][b] * sum_k c_k * qx_k   (fp64)
 *   s[m][n] = sum_b |dw dx| * sum_k |c_k qx_k|
 * with c the signed multiplier of the weight format (q - 8, or u - 2).
 * The integer sums are exact; the products of the three factors are exact
 * in fp64 (11 + 24 + 16 significant bits), so y is the exact value up to
 * the fp64 rounding of the sum over blocks. */
void orc_gemv_q8act(int fmt, const uint8_t *p, int64_t N, int64_t K, const int8_t *qx, const float *dx,
                    int64_t M, double *y, double *s)
{
    const int64_t KB = K / 32;
    for (int64_t m = 0; m < M; ++m) {
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, sabs = 0.0;
            for (int64_t b = 0; b < KB; ++b) {
                size_t i = (size_t)(n * KB + b);
                double dw = scale_value(fmt, p, N, K, i);
#if defined(ORC_PLANT_ACTSCALE)
                double d = (double)dx[m * KB + (b + 1) % KB];
#else
                double d = (double)dx[m * KB + b];
#endif
                int64_t isum = 0, iabs = 0;
                for (int k = 0; k < 32; ++k) {
                    int64_t t = (int64_t)code_value(fmt, p, i, k) * (int64_t)qx[m * K + b * 32 + k];
                    isum += t;
                    iabs += t < 0 ? -t : t;
                }
                acc += dw * d * (double)isum;
                sabs += fabs(dw * d) * (double)iabs;
            }
            y[m * N + n] = acc;
            s[m * N + n] = sabs;
        }
    }
}

/* ------------------------------------------------------ thread control */

/* OpenMP threads for the loops over output rows (changes no arithmetic). */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int orc_max_threads(void) { return omp_get_max_threads(); }
