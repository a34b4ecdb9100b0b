/*
 * CPU oracle for MXFP8 block-scaled quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the
 * GPU path is checked against.  Only the test suite, the package smoke check
 * and the benchmark's CPU-baseline leg may load it.  It shares no code with
 * the HIP kernels: no headers, no tables, no helpers.
 *
 * What is computed (the pages fix the block size, the formats and the two
 * copies; the scale rule and the rounding are the OCP MX rule):
 *
 *  - Blocks of 32 consecutive elements along the reduction direction
 *    (page "[Common] Experimental CuTeDSL MXFP8 backends in C++ via TVM-FFI",
 *    review thread on 32-divisible shapes: the block size is 32).
 *  - One E8M0 shared scale per block (page "Experimental FlyDSL GEMM backend
 *    for TE PyTorch (BF16/FP16/FP32/FP8/MXFP8)", commit notes on the fused
 *    scale-pack kernel: per-block E8M0 scales), a bare biased exponent
 *    (page "frost(gemm): Add Rubin kernel pipelines", nitpick on the ue8m0
 *    readback: the byte shifted into the fp32 exponent field is the value).
 *  - Shared exponent X = floor(log2(amax)) - 8, clamped to [-127, 127],
 *    stored as the byte X + 127; an all-zero block stores byte 0.
 *  - Elements become E4M3 (OCP "FN" variant, largest finite 448) of
 *    x * 2^-X, rounded to nearest with ties to even, saturating at +-448,
 *    keeping the sign of zero and of values that round to zero.
 *  - Rowwise copy: blocks along each row, q[R][C], s[R][C/32].
 *    Columnwise copy: blocks along each column, stored transposed as
 *    qT[C][R], sT[C][R/32] (page "Experimental FlyDSL GEMM backend ...",
 *    commit notes: columnwise storage is the materialised transpose).
 *  - dbias: the fp32 column sum of the unquantized input (page "[Common]
 *    Experimental CuTeDSL MXFP8 backends ...", Greptile summary: the dbias
 *    workspace and its reduction).  Summed here in double, rounded once.
 *
 * Every value is handled in double precision: a BF16 value times a power of
 * two in [2^-127, 2^127] is exact in double, so the rounding decision below is
 * the exact one.  No libm transcendental is used; floor(log2) comes from
 * frexp, which is exact.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define MX_BLOCK 32

/* BF16 is the upper half of an IEEE binary32: widen the bit pattern. */
static double bf16_value(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double oracle_bf16_to_double(uint16_t h) { return bf16_value(h); }

/* E4M3 (OCP FN) decode: sign | 4-bit exponent (bias 7) | 3-bit mantissa.
 * Exponent field 0 is subnormal m * 2^-9; the pattern S.1111.111 is NaN;
 * every other pattern is (1 + m/8) * 2^(e-7).  There is no infinity. */
double oracle_e4m3_decode(uint8_t c)
{
    int s = (c >> 7) & 1;
    int e = (c >> 3) & 0xF;
    int m = c & 0x7;
    double mag;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp((double)(8 + m), e - 10);
    return s ? -mag : mag;
}

/* E8M0 decode: byte b encodes 2^(b-127); 0xFF is NaN and never produced. */
double oracle_e8m0_decode(uint8_t b)
{
    if (b == 0xFF)
        return NAN;
    return ldexp(1.0, (int)b - 127);
}

/* E4M3 encode of an exact value v: nearest representable, ties to even,
 * magnitudes at or above 448 saturate to 448, sign always kept. */
uint8_t oracle_e4m3_encode(double v)
{
    uint8_t s = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    int e2, E;
    double n;

    if (a >= 448.0)
        return (uint8_t)(s | 0x7E);
    if (a < 0x1p-6) {
        /* subnormal grid: multiples of 2^-9; a result of 8 is the smallest
         * normal 2^-6, whose code is 0x08 as well. */
        n = nearbyint(a * 512.0);
        return (uint8_t)(s | (uint8_t)n);
    }
    frexp(a, &e2);          /* a = f * 2^e2, f in [0.5, 1) */
    E = e2 - 1;             /* floor(log2 a), in [-6, 8] */
    n = nearbyint(ldexp(a, 3 - E)); /* 4 significant bits: in [8, 16] */
    if (n == 16.0) {
        n = 8.0;
        E += 1;
    }
    return (uint8_t)(s | (uint8_t)(((E + 7) << 3) | ((int)n - 8)));
}

/* Shared-scale byte of a block from its amax (OCP MX): X = floor(log2 amax)
 * - 8 clamped to [-127, 127], byte X + 127; amax 0 gives byte 0. */
uint8_t oracle_scale_byte(double amax)
{
    int e2, X;
    if (amax == 0.0)
        return 0;
    frexp(amax, &e2);
    X = (e2 - 1) - 8;
    if (X < -127)
        X = -127;
    if (X > 127)
        X = 127;
    return (uint8_t)(X + 127);
}

/* Quantize one block of n values given in double. */
static void quantize_block(const double *v, int n, uint8_t *codes, uint8_t *scale)
{
    double amax = 0.0;
    int i, X;
    uint8_t b;
    for (i = 0; i < n; i++)
        if (fabs(v[i]) > amax)
            amax = fabs(v[i]);
    b = oracle_scale_byte(amax);
    X = (int)b - 127;
    for (i = 0; i < n; i++)
        codes[i] = oracle_e4m3_encode(ldexp(v[i], -X));
    *scale = b;
}

/* Rowwise copy: x[R][ld_x] BF16 -> q[R][C], s[R][C/32]. */
void oracle_quantize_rows(const uint16_t *x, int64_t R, int64_t C, int64_t ld_x,
                          uint8_t *q, uint8_t *s)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < R; r++) {
        double v[MX_BLOCK];
        int64_t b;
        int i;
        for (b = 0; b < C / MX_BLOCK; b++) {
            for (i = 0; i < MX_BLOCK; i++)
                v[i] = bf16_value(x[r * ld_x + b * MX_BLOCK + i]);
            quantize_block(v, MX_BLOCK, q + r * C + b * MX_BLOCK, s + r * (C / MX_BLOCK) + b);
        }
    }
}

/* Columnwise copy, stored transposed: blocks of 32 rows of one column.
 * x[R][ld_x] BF16 -> qT[C][R], sT[C][R/32]. */
void oracle_quantize_cols(const uint16_t *x, int64_t R, int64_t C, int64_t ld_x,
                          uint8_t *qT, uint8_t *sT)
{
    int64_t c;
#pragma omp parallel for schedule(static)
    for (c = 0; c < C; c++) {
        double v[MX_BLOCK];
        int64_t b;
        int i;
        for (b = 0; b < R / MX_BLOCK; b++) {
            for (i = 0; i < MX_BLOCK; i++)
                v[i] = bf16_value(x[(b * MX_BLOCK + i) * ld_x + c]);
            quantize_block(v, MX_BLOCK, qT + c * R + b * MX_BLOCK, sT + c * (R / MX_BLOCK) + b);
        }
    }
}

/* The same two copies for fp32 values v[R][ld] (an activation's output,
 * computed in fp32 by the caller). */
void oracle_quantize_rows_f32(const float *x, int64_t R, int64_t C, int64_t ld,
                              uint8_t *q, uint8_t *s)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < R; r++) {
        double v[MX_BLOCK];
        int64_t b;
        int i;
        for (b = 0; b < C / MX_BLOCK; b++) {
            for (i = 0; i < MX_BLOCK; i++)
                v[i] = (double)x[r * ld + b * MX_BLOCK + i];
            quantize_block(v, MX_BLOCK, q + r * C + b * MX_BLOCK, s + r * (C / MX_BLOCK) + b);
        }
    }
}

void oracle_quantize_cols_f32(const float *x, int64_t R, int64_t C, int64_t ld,
                              uint8_t *qT, uint8_t *sT)
{
    int64_t c;
#pragma omp parallel for schedule(static)
    for (c = 0; c < C; c++) {
        double v[MX_BLOCK];
        int64_t b;
        int i;
        for (b = 0; b < R / MX_BLOCK; b++) {
            for (i = 0; i < MX_BLOCK; i++)
                v[i] = (double)x[(b * MX_BLOCK + i) * ld + c];
            quantize_block(v, MX_BLOCK, qT + c * R + b * MX_BLOCK, sT + c * (R / MX_BLOCK) + b);
        }
    }
}

/* Column sums of fp32 values, accumulated in double, rounded once. */
void oracle_dbias_f32(const float *x, int64_t R, int64_t C, int64_t ld, float *dbias)
{
    int64_t c;
#pragma omp parallel for schedule(static)
    for (c = 0; c < C; c++) {
        double acc = 0.0;
        int64_t r;
        for (r = 0; r < R; r++)
            acc += (double)x[r * ld + c];
        dbias[c] = (float)acc;
    }
}

/* dbias[c] = sum over rows of x[r][c], accumulated in double, rounded once to
 * float. */
void oracle_dbias(const uint16_t *x, int64_t R, int64_t C, int64_t ld_x, float *dbias)
{
    int64_t c;
#pragma omp parallel for schedule(static)
    for (c = 0; c < C; c++) {
        double acc = 0.0;
        int64_t r;
        for (r = 0; r < R; r++)
            acc += bf16_value(x[r * ld_x + c]);
        dbias[c] = (float)acc;
    }
}

/* Dequantize a [R][C] code matrix with its [R][C/32] scales into double. */
void oracle_dequantize(const uint8_t *q, const uint8_t *s, int64_t R, int64_t C, double *out)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < R; r++) {
        int64_t c;
        for (c = 0; c < C; c++)
            out[r * C + c] = oracle_e4m3_decode(q[r * C + c]) *
                             oracle_e8m0_decode(s[r * (C / MX_BLOCK) + c / MX_BLOCK]);
    }
}

/* Elementwise encode of an array of exact values (used by the pins). */
void oracle_e4m3_encode_array(const double *v, int64_t n, uint8_t *out)
{
    int64_t i;
    for (i = 0; i < n; i++)
        out[i] = oracle_e4m3_encode(v[i]);
}

/* Scale packing: s[dim][ld_s] bytes (K/32 of them used per row) become
 * packed[K/128][dim] 32-bit words whose byte j (little-endian) is the scale of
 * K-block 4t + j of that row: the [K/128, dim] word layout of the page
 * "Experimental FlyDSL GEMM backend ...", commit notes on the fused
 * scale-pack kernel, with four consecutive 32-blocks (one 128-wide K slab) per
 * word. */
void oracle_pack_scales(const uint8_t *s, int64_t dim, int64_t kblocks, int64_t ld_s,
                        uint8_t *packed)
{
    int64_t t, r;
    int j;
    for (t = 0; t < kblocks / 4; t++)
        for (r = 0; r < dim; r++)
            for (j = 0; j < 4; j++)
                packed[(t * dim + r) * 4 + j] = s[r * ld_s + 4 * t + j];
}

/* Scale bytes of an array of block amax values (the oracle_scale_byte rule). */
void oracle_scale_byte_array(const double *amax, int64_t n, uint8_t *out)
{
    int64_t i;
    for (i = 0; i < n; i++)
        out[i] = oracle_scale_byte(amax[i]);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
