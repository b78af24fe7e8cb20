/*
 * pqo.c -- CPU oracle for the block-scaled quantizers and dequantizer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the package's smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code, header, table or
 * constant generator with the HIP library.
 *
 * Style: plain and slow on purpose.  Every rounding decision is taken by
 * exact comparisons in binary64, where each product compared against is
 * exactly representable (the bit counts are stated at each use and checked
 * at run time with an FMA residual).  Build with
 *     gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC
 * so that no operation is contracted or approximated.
 *
 * Sources (titles of the pages the method is described on):
 *   [BW]  "Towards Blackwell-Native 8-bit and 4-bit RL" (Miles / LMSYS blog)
 *   [MT]  "miniTE technical report: stable training and efficient
 *          implementation of native NVFP4 RL"
 *   [PR]  "PR #2396 report: docs: refresh MXFP8 and NVFP4 RL guide"
 *
 * Where the pages are silent, the reading taken is marked "reading" at the
 * code that takes it.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Element grids.                                                            */
/* ------------------------------------------------------------------------ */

/* bf16 bit pattern -> exact value (bf16 is the top half of a binary32). */
static double bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* E4M3 ([BW] Format background: MXFP8 and NVFP4 both use FP8 E4M3; the bit
 * layout is the OCP one: 1 sign, 4 exponent bits with bias 7, 3 mantissa
 * bits, exponent field 0 is subnormal, code 0x7F is NaN and never produced).
 * Magnitude code c in 0..126 -> value. */
static double e4m3_magnitude(int c)
{
    int e = (c >> 3) & 15, m = c & 7;
    if (e == 0)
        return ldexp((double)m, -9);
    return ldexp(1.0 + m / 8.0, e - 7);
}

/* E2M1 ([BW] Format background: NVFP4 stores FP4 E2M1 values): magnitude
 * code 0..7 -> 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
static double e2m1_magnitude(int c)
{
    static const double v[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    return v[c & 7];
}

/* E8M0 ([BW] Format background: MXFP8 scale is a power of two): byte b ->
 * 2^(b-127); 0xFF is NaN and never produced. */
static double e8m0_value(int b) { return ldexp(1.0, b - 127); }

/* Count of products that were not exact; must stay 0 (checked by tests). */
static long g_inexact;

/* mid * den, checking with an FMA residual that the product is exact. */
static double exact_mul(double mid, double den)
{
    double p = mid * den;
    if (fma(mid, den, -p) != 0.0) {
#pragma omp atomic
        g_inexact++;
    }
    return p;
}

/*
 * Round the exact real num/den (num >= 0, den > 0) to the nearest point of
 * an ascending grid g[0..n-1], ties to the even code, values beyond the top
 * saturating to g[n-1].  The code of grid point k is k for both E4M3 and
 * E2M1 magnitudes, so "even code" is "even index".
 *
 * The decision compares num against midpoint*den.  The midpoint of two
 * adjacent E4M3 points has at most 5 significant bits and an E2M1 midpoint
 * at most 3; every den passed in has at most 28 significant bits, so each
 * product has at most 33 bits and is exact in binary64.
 *
 * Binary search for the first midpoint that num does not exceed.
 */
static int rne_grid(double num, double den, const double *g, int n)
{
    int lo = 0, hi = n - 1; /* answer index in [lo, hi] */
    while (lo < hi) {
        int k = (lo + hi) / 2; /* midpoint between g[k] and g[k+1] */
        double mid = 0.5 * (g[k] + g[k + 1]);
        double t = exact_mul(mid, den);
        if (num < t)
            hi = k;
        else if (num > t)
            lo = k + 1;
        else
            return (k % 2 == 0) ? k : k + 1; /* exact tie: even code */
    }
    return lo;
}

static double g_e4m3[127];
static double g_e2m1[8];
static int g_init;

static void init_grids(void)
{
    if (g_init)
        return;
    for (int c = 0; c < 127; ++c)
        g_e4m3[c] = e4m3_magnitude(c);
    for (int c = 0; c < 8; ++c)
        g_e2m1[c] = e2m1_magnitude(c);
    g_init = 1;
}

/* Signed E4M3 byte nearest to x/den (den > 0), saturating at 448.  The sign
 * bit follows the sign of x, zero results included (a negative input that
 * rounds to zero gives 0x80: the pages do not say; IEEE conversions keep the
 * sign of zero, and that reading is taken). */
static uint8_t e4m3_encode(double x, double den)
{
    int neg = signbit(x) ? 1 : 0;
    int c = rne_grid(fabs(x), den, g_e4m3, 127);
    return (uint8_t)((neg << 7) | c);
}

/* Signed E2M1 nibble nearest to x/den (den > 0), saturating at 6; sign bit
 * is bit 3 and follows the sign of x as for E4M3. */
static uint8_t e2m1_encode(double x, double den)
{
    int neg = signbit(x) ? 1 : 0;
    int c = rne_grid(fabs(x), den, g_e2m1, 8);
    return (uint8_t)((neg << 3) | c);
}

/* ------------------------------------------------------------------------ */
/* MXFP8 ([BW] Format background: MXFP8; Recipe 1: training).               */
/* ------------------------------------------------------------------------ */

/*
 * Scale exponent of one block with absolute maximum a: the power-of-two
 * scale is rounded up so that the block maximum is not clipped, i.e. the
 * smallest e with a <= 448 * 2^e (448 is the E4M3 maximum).  The E8M0 range
 * limits e to [-127, 127]; an all-zero block takes the smallest scale
 * (reading: the pages are silent; any scale decodes zero to zero).
 */
static int mx_scale_exponent(double a)
{
    for (int e = -127; e <= 127; ++e)
        if (a <= 448.0 * ldexp(1.0, e))
            return e;
    return 127; /* unreachable for finite bf16 input */
}

/* One 1x32 block: v[i*stride] for i < 32 -> q[i*qstride], scale byte. */
static void mx_block(const uint16_t *x, long stride, uint8_t *q, long qstride,
                     uint8_t *scale)
{
    double a = 0.0;
    for (int i = 0; i < 32; ++i) {
        double v = fabs(bf16_value(x[i * stride]));
        if (v > a)
            a = v;
    }
    int e = mx_scale_exponent(a);
    double den = ldexp(1.0, e); /* one significant bit */
    for (int i = 0; i < 32; ++i)
        q[i * qstride] = e4m3_encode(bf16_value(x[i * stride]), den);
    *scale = (uint8_t)(e + 127);
}

/*
 * Row-wise copy: 1x32 blocks along each row of x[R, C] (leading dim ld).
 * q[R, C] row-major, s[R, C/32] row-major.  C must be a multiple of 32.
 */
void pqo_quantize_mxfp8_rowwise(const uint16_t *x, long R, long C, long ld,
                                uint8_t *q, uint8_t *s)
{
    init_grids();
#pragma omp parallel for schedule(static)
    for (long r = 0; r < R; ++r)
        for (long b = 0; b < C / 32; ++b)
            mx_block(x + r * ld + b * 32, 1, q + r * C + b * 32, 1,
                     s + r * (C / 32) + b);
}

/*
 * Column-wise copy: 32x1 blocks down each column of the same bf16 input,
 * quantized from the full-precision data and not from the row-wise copy
 * ([BW] Recipe 1: training -- row-wise and column-wise blocks differ
 * numerically and are each quantized from the high-precision tensor).
 * Stored transposed (reading): qT[C, R] and sT[C, R/32], so that each 32-row
 * block is contiguous, as the contraction over rows needs.  R must be a
 * multiple of 32.
 */
void pqo_quantize_mxfp8_colwise(const uint16_t *x, long R, long C, long ld,
                                uint8_t *qT, uint8_t *sT)
{
    init_grids();
#pragma omp parallel for schedule(static)
    for (long c = 0; c < C; ++c)
        for (long b = 0; b < R / 32; ++b)
            mx_block(x + (b * 32) * ld + c, ld, qT + c * R + b * 32, 1,
                     sT + c * (R / 32) + b);
}

/* ------------------------------------------------------------------------ */
/* NVFP4 ([BW] Format background: NVFP4; Recipe 2: per-token activation      */
/* scaling; [MT] 2.2 decode x^ = q * s_b * s_g; [MT] 5.6 gs = gamax / 2688). */
/* ------------------------------------------------------------------------ */

/*
 * x[R, C] (leading dim ld) is split into scope groups of rows_per_group
 * consecutive rows; each group has one FP32 outer scale.  rows_per_group = 1
 * is the per-token scope; rows_per_group = R/G views x as G stacked tensors
 * (one per expert); for fused gate/up weights, one group spans both halves,
 * so gate and up share one outer scale ([BW] Recipe 2, gate/up pairing).
 *
 *   A     = max |x| over the group
 *   s_g   = fp32(A / 2688), one correctly rounded binary32 division
 *           (2688 = 6 * 448, E2M1 max times E4M3 max)
 *   s_b   = E4M3 nearest to a_b / (6 s_g) for each 1x16 block with block max
 *           a_b, rounded to nearest, saturating at 448; s_b = 0 when s_g = 0
 *   q_i   = E2M1 nearest to x_i / (s_b s_g), saturating at 6; +-0 when s_b = 0
 *
 * Outputs: q[R, C/2] with element 2j in the low nibble of byte j (reading),
 * sb[R, C/16] E4M3 bytes, sg[R / rows_per_group] binary32 decode scales.
 * C must be a multiple of 16 and R a multiple of rows_per_group.
 */
/*
 * The 1x16 blocks of one row xr[0..C) under a given outer scale s_g: block
 * scale s_b, then the E2M1 codes, as described above.  qr gets C/2 bytes and
 * sbr C/16 bytes.
 */
static void nvfp4_encode_row(const uint16_t *xr, long C, float s_g,
                             uint8_t *qr, uint8_t *sbr)
{
    for (long b = 0; b < C / 16; ++b) {
        const uint16_t *xb = xr + b * 16;
        uint8_t *qb = qr + b * 8;
        double ab = 0.0;
        for (int i = 0; i < 16; ++i) {
            double v = fabs(bf16_value(xb[i]));
            if (v > ab)
                ab = v;
        }
        int sbc = 0;
        if (s_g != 0.0f) /* 6 * s_g: at most 26 significant bits */
            sbc = rne_grid(ab, 6.0 * (double)s_g, g_e4m3, 127);
        sbr[b] = (uint8_t)sbc;
        double dec = g_e4m3[sbc] * (double)s_g; /* <= 28 bits */
        for (int j = 0; j < 8; ++j) {
            uint8_t lo, hi;
            double x0 = bf16_value(xb[2 * j]);
            double x1 = bf16_value(xb[2 * j + 1]);
            if (sbc == 0) {
                lo = signbit(x0) ? 0x8 : 0x0;
                hi = signbit(x1) ? 0x8 : 0x0;
            } else {
                lo = e2m1_encode(x0, dec);
                hi = e2m1_encode(x1, dec);
            }
            qb[j] = (uint8_t)(lo | (hi << 4));
        }
    }
}

void pqo_quantize_nvfp4(const uint16_t *x, long R, long C, long ld,
                        long rows_per_group, uint8_t *q, uint8_t *sb,
                        float *sg)
{
    init_grids();
    long G = R / rows_per_group;
#pragma omp parallel for schedule(dynamic)
    for (long g = 0; g < G; ++g) {
        long r0 = g * rows_per_group;
        float A = 0.0f;
        for (long r = r0; r < r0 + rows_per_group; ++r)
            for (long c = 0; c < C; ++c) {
                float v = (float)fabs(bf16_value(x[r * ld + c]));
                if (v > A)
                    A = v;
            }
        volatile float denom = 2688.0f; /* keep the division in binary32 */
        float s_g = A / denom;
        sg[g] = s_g;
        for (long r = r0; r < r0 + rows_per_group; ++r)
            nvfp4_encode_row(x + r * ld, C, s_g, q + r * (C / 2), sb + r * (C / 16));
    }
}

/*
 * The same block encoding of each row r of x[R, C] under an outer scale
 * sg[r] given by the caller instead of taken from the row's own maximum.
 * The online amax loop of [MT] 5.6 encodes each activation tile with the
 * outer scale of the running row maximum, which may exceed the tile's own
 * maximum; with sg[r] = fp32(max|x[r]| / 2688) this is the per-token
 * quantizer above.  Every |x| must be at most 2688 sg[r] (not checked:
 * larger values saturate the block scale at 448).
 */
void pqo_quantize_nvfp4_given_scale(const uint16_t *x, long R, long C, long ld,
                                    const float *sg, uint8_t *q, uint8_t *sb)
{
    init_grids();
#pragma omp parallel for schedule(static)
    for (long r = 0; r < R; ++r)
        nvfp4_encode_row(x + r * ld, C, sg[r], q + r * (C / 2), sb + r * (C / 16));
}

/* ------------------------------------------------------------------------ */
/* Block-scaled FP8, the DeepSeek-V3 style ([BW] Why Blackwell-native       */
/* recipes: 128x128 weight blocks and 1x128 activation tiles, each with an  */
/* FP32 scale computed online and applied around the matrix core; [PR]      */
/* Choose a precision: FP8 block-wise, 128x128, FP32 scales).               */
/* ------------------------------------------------------------------------ */

/*
 * Blocks of br rows x 128 columns (br = 1: activation tiles; br = 128:
 * weight blocks).  For a block with absolute maximum A:
 *   s = A / 448 rounded once to binary32 (reading: the block maximum maps
 *       to the E4M3 maximum; the pages give the block shapes and FP32
 *       scales, not the formula);
 *   q = nearest E4M3 to x / s, ties to even, saturating at 448; A = 0
 *       gives s = 0 and q = +-0.
 * s [R/br, C/128] binary32, q [R, C] bytes.
 */
void pqo_quantize_fp8_block(const uint16_t *x, long R, long C, long ld, long br,
                            uint8_t *q, float *s)
{
    init_grids();
    long RB = R / br, CB = C / 128;
#pragma omp parallel for schedule(dynamic)
    for (long blk = 0; blk < RB * CB; ++blk) {
        long rb = blk / CB, cb = blk % CB;
        float A = 0.0f;
        for (long r = rb * br; r < (rb + 1) * br; ++r)
            for (long c = cb * 128; c < cb * 128 + 128; ++c) {
                float v = (float)fabs(bf16_value(x[r * ld + c]));
                if (v > A)
                    A = v;
            }
        volatile float d = 448.0f; /* keep the division in binary32 */
        float sc = A / d;
        s[blk] = sc;
        for (long r = rb * br; r < (rb + 1) * br; ++r)
            for (long c = cb * 128; c < cb * 128 + 128; ++c) {
                double v = bf16_value(x[r * ld + c]);
                q[r * C + c] = sc == 0.0f ? (uint8_t)(signbit(v) ? 0x80 : 0x00)
                                          : e4m3_encode(v, (double)sc);
            }
    }
}

/* Exact binary64 values q * s of a block-scaled FP8 tensor. */
void pqo_decode_fp8_block(const uint8_t *q, const float *s, long R, long C, long br,
                          double *out)
{
    long CB = C / 128;
#pragma omp parallel for
    for (long r = 0; r < R; ++r)
        for (long c = 0; c < C; ++c) {
            uint8_t b = q[r * C + c];
            double v = e4m3_magnitude(b & 0x7F) * (double)s[(r / br) * CB + c / 128];
            out[r * C + c] = (b & 0x80) ? -v : v;
        }
}

/* ------------------------------------------------------------------------ */
/* Dequantize ([BW] High-precision and dequantized backward: the backward   */
/* GEMMs read the BF16 dequantization of the exact forward operands).       */
/* ------------------------------------------------------------------------ */

/* Nearest bf16 to the exact binary64 value v, ties to even, overflow to
 * infinity: a single rounding.  Returns the bit pattern. */
static uint16_t bf16_round(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    int E;
    frexp(a, &E); /* a = f * 2^E, f in [0.5, 1) -> a in [2^(E-1), 2^E) */
    int ex = E - 1;
    if (ex < -126)
        ex = -126;                 /* bf16 subnormal quantum is 2^-133 */
    double quantum = ldexp(1.0, ex - 7);
    double n = nearbyint(a / quantum); /* a / quantum exact; RNE */
    double r = n * quantum;
    if (r >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80); /* overflow -> inf */
    float f = (float)r;                   /* exact: r is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | ((u >> 16) & 0x7FFF));
}

/* MXFP8 dequantize of a [R, C] copy with 1x32 scales s[R, C/32]. */
void pqo_dequantize_mxfp8(const uint8_t *q, const uint8_t *s, long R, long C,
                          uint16_t *y)
{
    init_grids();
#pragma omp parallel for schedule(static)
    for (long r = 0; r < R; ++r)
        for (long c = 0; c < C; ++c) {
            uint8_t b = q[r * C + c];
            double v = g_e4m3[b & 0x7F] * e8m0_value(s[r * (C / 32) + c / 32]);
            y[r * C + c] = bf16_round((b & 0x80) ? -v : v);
        }
}

/* NVFP4 dequantize: q[R, C/2], sb[R, C/16], sg[R / rows_per_group]; the
 * product q * s_b * s_g has at most 2 + 4 + 24 bits and is exact. */
void pqo_dequantize_nvfp4(const uint8_t *q, const uint8_t *sb, const float *sg,
                          long R, long C, long rows_per_group, uint16_t *y)
{
    init_grids();
#pragma omp parallel for schedule(static)
    for (long r = 0; r < R; ++r)
        for (long c = 0; c < C; ++c) {
            uint8_t byte = q[r * (C / 2) + c / 2];
            uint8_t nib = (c % 2 == 0) ? (byte & 0xF) : (byte >> 4);
            double v = g_e2m1[nib & 7] * g_e4m3[sb[r * (C / 16) + c / 16] & 0x7F] *
                       (double)sg[r / rows_per_group];
            y[r * C + c] = bf16_round((nib & 8) ? -v : v);
        }
}

/* Exact operand values for the grouped-GEMM oracle, in binary64. */
void pqo_decode_mxfp8(const uint8_t *q, const uint8_t *s, long R, long C,
                      double *out)
{
    init_grids();
#pragma omp parallel for schedule(static)
    for (long r = 0; r < R; ++r)
        for (long c = 0; c < C; ++c) {
            uint8_t b = q[r * C + c];
            double v = g_e4m3[b & 0x7F] * e8m0_value(s[r * (C / 32) + c / 32]);
            out[r * C + c] = (b & 0x80) ? -v : v;
        }
}

void pqo_decode_nvfp4(const uint8_t *q, const uint8_t *sb, const float *sg,
                      long R, long C, long rows_per_group, double *out)
{
    init_grids();
#pragma omp parallel for schedule(static)
    for (long r = 0; r < R; ++r)
        for (long c = 0; c < C; ++c) {
            uint8_t byte = q[r * (C / 2) + c / 2];
            uint8_t nib = (c % 2 == 0) ? (byte & 0xF) : (byte >> 4);
            double v = g_e2m1[nib & 7] * g_e4m3[sb[r * (C / 16) + c / 16] & 0x7F] *
                       (double)sg[r / rows_per_group];
            out[r * C + c] = (nib & 8) ? -v : v;
        }
}

/* ------------------------------------------------------------------------ */
/* Scalar entry points, for the pins.                                        */
/* ------------------------------------------------------------------------ */

uint8_t pqo_e4m3_encode(double x, double den) { init_grids(); return e4m3_encode(x, den); }
uint8_t pqo_e2m1_encode(double x, double den) { init_grids(); return e2m1_encode(x, den); }
double pqo_e4m3_decode(uint8_t b) { double v = e4m3_magnitude(b & 0x7F); return (b & 0x80) ? -v : v; }
double pqo_e2m1_decode(uint8_t n) { double v = e2m1_magnitude(n & 7); return (n & 8) ? -v : v; }
int pqo_mx_scale_exponent(double a) { return mx_scale_exponent(a); }
uint16_t pqo_bf16_round(double v) { return bf16_round(v); }
long pqo_inexact_count(void) { return g_inexact; }
void pqo_reset_inexact(void) { g_inexact = 0; }
float pqo_fp32_div(float a, float b) { volatile float d = b; return a / d; }

void pqo_bf16_round_array(const double *v, long n, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (long i = 0; i < n; ++i)
        out[i] = bf16_round(v[i]);
}

int pqo_omp_threads(void) { return omp_get_max_threads(); }
void pqo_set_threads(int n) { omp_set_num_threads(n); }
