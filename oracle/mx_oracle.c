/*
 * mx_oracle.c -- CPU oracle for the MX quantize / block-Hadamard / MX-GEMM path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's cpu_baseline leg may load this library.  The product path (the
 * HIP library under precision_block_amax_amd/) never calls it, and the two
 * share no code, headers, tables or constants.
 *
 * What it computes, and where that is stated:
 *   - MX micro-scaling: a tensor is cut into 32-element blocks along the
 *     reduction dimension, each block carrying its own dynamic power-of-two
 *     exponent (MXFP4 as described in the hzrcw.cc FP4-training article,
 *     section 02; block size 32: MindSpeed-LLM FSDP2 quantization page,
 *     recipe dynamic_MX-1-1-32 and --model.quant_block_size 32).
 *   - E4M3 / E5M2 element formats (Lumen page, section 1) and MXFP4 = E2M1
 *     (FP4-training article, sections 02 and 04), encoded as in the OCP
 *     8-bit float and MX definitions: E4M3 "FN" (bias 7, max 448, no Inf),
 *     E5M2 (bias 15, max normal 57344), E2M1 (bias 1, max 6).
 *   - E8M0 shared scale: S = clamp(floor(log2 amax) - emax_elem, -127, 127) + 127,
 *     elements cast as v * 2^-(S-127) with round-to-nearest-even and
 *     saturation to the largest normal.
 *   - The deterministic fixed-sign 32-point Hadamard rotation applied along
 *     tokens on the weight-gradient path (FP4-training article, section 02):
 *     y = RN32(1/sqrt 32) * H32 * diag(s) * x, H32 the Sylvester matrix,
 *     s_i = -1 where bit i of the sign mask is set.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - scale exponent uses floor(log2 amax); an all-zero block gets S = 0;
 *     e below -127 clamps to S = 0; a block holding Inf/NaN gets S = 0xFF
 *     and all-zero codes;
 *   - overflow saturates to +-max normal; the sign of zero is kept;
 *   - E2M1 packing: element 2i in bits 3:0, element 2i+1 in bits 7:4;
 *   - rotation arithmetic: fp32, one rounding per operation, butterfly
 *     stages h = 1, 2, 4, 8, 16 in that order, each (a, b) -> (a+b, a-b),
 *     then one multiply by c = RN32(1/sqrt 32); no rounding to bf16;
 *   - stochastic rounding (ablation only): the textbook definition taken to
 *     32 fraction bits, random words from Philox4x32-10 (details below).
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math;
 * SSE arithmetic, so every float operation rounds to float).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

enum { ORC_E4M3 = 0, ORC_E5M2 = 1, ORC_E2M1 = 2 };

typedef struct {
    int ebits;       /* exponent field width */
    int mbits;       /* mantissa field width */
    int bias;        /* exponent bias */
    double maxnorm;  /* largest finite magnitude */
    int emax;        /* exponent of the largest normal binade */
} orc_fmt;

/* format parameters, from the OCP element definitions */
static const orc_fmt FMT[3] = {
    {4, 3, 7, 448.0, 8},     /* E4M3: 1.75 * 2^8   */
    {5, 2, 15, 57344.0, 15}, /* E5M2: 1.75 * 2^15  */
    {2, 1, 1, 6.0, 2},       /* E2M1: 1.5  * 2^2   */
};

static int valid_fmt(int f) { return f >= 0 && f <= 2; }

/* exact value of a bf16 bit pattern (1-8-7, bias 127) */
static double bf16_value(uint16_t b)
{
    int s = b >> 15, E = (b >> 7) & 0xFF, m = b & 0x7F;
    double v;
    if (E == 0xFF)
        v = m ? NAN : INFINITY;
    else if (E == 0)
        v = ldexp((double)m, -133);            /* m/128 * 2^-126 */
    else
        v = ldexp((double)(128 + m), E - 134); /* (1 + m/128) * 2^(E-127) */
    return s ? -v : v;
}

/* floor(log2 a) for finite a > 0: frexp gives a = f * 2^x with f in [0.5, 1) */
static int floor_log2(double a)
{
    int x;
    frexp(a, &x);
    return x - 1;
}

/* E8M0 scale byte of a finite block amax */
static int e8m0_of_amax(double amax, const orc_fmt *f)
{
    int e = (amax == 0.0) ? -127 : floor_log2(amax) - f->emax;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e + 127;
}

/* Round q (exact, already divided by the block scale) to the format grid:
 * nearest representable magnitude, ties to even mantissa LSB, saturating at
 * the largest normal; return sign | exponent field | mantissa field. */
static uint8_t encode_elem(double q, const orc_fmt *f)
{
    int neg = signbit(q) ? 1 : 0;
    double a = fabs(q), mag;
    int emin = 1 - f->bias; /* exponent of the smallest normal binade */

    if (a >= f->maxnorm) {
        mag = f->maxnorm;
    } else if (a == 0.0) {
        mag = 0.0;
    } else {
        int k = floor_log2(a);
        int kk = k < emin ? emin : k;           /* subnormals share emin's spacing */
        double quantum = ldexp(1.0, kk - f->mbits);
        mag = nearbyint(a / quantum) * quantum; /* default rounding mode: ties to even */
        if (mag > f->maxnorm) mag = f->maxnorm;
    }

    unsigned field;
    if (mag == 0.0) {
        field = 0;
    } else {
        int k = floor_log2(mag);
        if (k < emin) { /* subnormal: exponent field 0 */
            field = (unsigned)(mag / ldexp(1.0, emin - f->mbits));
        } else {
            unsigned mant = (unsigned)(mag / ldexp(1.0, k - f->mbits)) - (1u << f->mbits);
            field = ((unsigned)(k + f->bias) << f->mbits) | mant;
        }
    }
    return (uint8_t)(((unsigned)neg << (f->ebits + f->mbits)) | field);
}

/* value of one element code (no block scale) */
static double decode_elem(uint8_t code, int fmt)
{
    const orc_fmt *f = &FMT[fmt];
    int nb = f->ebits + f->mbits;
    int s = (code >> nb) & 1;
    int E = (code >> f->mbits) & ((1 << f->ebits) - 1);
    int m = code & ((1 << f->mbits) - 1);
    double v;
    if (fmt == ORC_E4M3 && E == 15 && m == 7)
        v = NAN;
    else if (fmt == ORC_E5M2 && E == 31)
        v = m ? NAN : INFINITY;
    else if (E == 0)
        v = ldexp((double)m, 1 - f->bias - f->mbits);
    else
        v = ldexp((double)((1 << f->mbits) + m), E - f->bias - f->mbits);
    return s ? -v : v;
}

/* One block of 32 exact values -> 32 element codes (unpacked) and a scale. */
static void quantize_block(const double *v, const orc_fmt *f, uint8_t *codes, uint8_t *scale)
{
    double amax = 0.0;
    int finite = 1;
    for (int i = 0; i < 32; i++) {
        if (!isfinite(v[i]))
            finite = 0;
        else if (fabs(v[i]) > amax)
            amax = fabs(v[i]);
    }
    if (!finite) {
        *scale = 0xFF;
        memset(codes, 0, 32);
        return;
    }
    int S = e8m0_of_amax(amax, f);
    int e = S - 127;
    *scale = (uint8_t)S;
    for (int i = 0; i < 32; i++)
        codes[i] = encode_elem(ldexp(v[i], -e), f); /* exact power-of-two scaling */
}

/* store 32 element codes of one block at dst: bytes (FP8) or packed nibbles (E2M1) */
static void store_block(const uint8_t *codes, int fmt, uint8_t *dst)
{
    if (fmt == ORC_E2M1) {
        for (int j = 0; j < 16; j++)
            dst[j] = (uint8_t)((codes[2 * j] & 0xF) | ((codes[2 * j + 1] & 0xF) << 4));
    } else {
        memcpy(dst, codes, 32);
    }
}

static int64_t code_bytes(int64_t n, int fmt) { return fmt == ORC_E2M1 ? n / 2 : n; }

/* ---------------------------------------------------------------------------
 * Fixed-sign 32-point Hadamard rotation in fp32 (reading: one rounding per op,
 * stages ascending).  H32 is the Sylvester matrix H[i][j] = (-1)^popcount(i&j).
 */
static float hadamard_c(void)
{
    return (float)(1.0 / sqrt(32.0)); /* RN32(1/sqrt 32) */
}

static void hadamard32(float *x, uint32_t mask)
{
    for (int i = 0; i < 32; i++)
        if ((mask >> i) & 1u) x[i] = -x[i];
    for (int h = 1; h < 32; h <<= 1)
        for (int j = 0; j < 32; j++)
            if (!(j & h)) {
                float a = x[j], b = x[j + h];
                x[j] = a + b;
                x[j + h] = a - b;
            }
    float c = hadamard_c();
    for (int i = 0; i < 32; i++)
        x[i] = x[i] * c;
}

/* ---------------------------------------------------------------------------
 * Stochastic rounding (the randomised alternative to round-to-nearest that
 * the FP4-training article, section 01, names among the common fixes it
 * argues against; the pages give no definition, so this is the textbook one):
 * with lo <= |q| < hi the two neighbouring magnitudes on the format grid,
 * |q| goes up to hi with probability (|q| - lo) / (hi - lo), else down to lo.
 * The probability is taken to 32 fraction bits, F = floor(2^32 (|q|-lo)/(hi-lo)),
 * and a 32-bit random word r decides: up iff r < F.  Values on the grid never
 * move; magnitudes at or above the largest normal saturate as in the RNE cast;
 * the block scale is the RNE path's.
 *
 * Random words come from Philox4x32-10, the counter-based generator of
 * Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2,
 * 3" (SC 2011): element i of an output array takes word i mod 4 of the block
 * for counter (i / 4 as two 32-bit words, low first, then 0, 0) and key
 * (seed low word, seed high word).
 */
static void philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; round++) {
        if (round > 0) { /* key schedule: Weyl sequence */
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        uint64_t p0 = (uint64_t)0xD2511F53u * x0, p1 = (uint64_t)0xCD9E8D57u * x2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t y0 = hi1 ^ x1 ^ k0, y1 = lo1, y2 = hi0 ^ x3 ^ k1, y3 = lo0;
        x0 = y0; x1 = y1; x2 = y2; x3 = y3;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* random word of element i under a 64-bit seed */
static uint32_t sr_word(uint64_t i, uint64_t seed)
{
    uint32_t ctr[4] = {(uint32_t)(i >> 2), (uint32_t)(i >> 34), 0u, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    philox4x32_10(ctr, key, out);
    return out[i & 3];
}

static uint8_t encode_elem_sr(double q, uint32_t r, const orc_fmt *f)
{
    int neg = signbit(q) ? 1 : 0;
    double a = fabs(q), mag;
    int emin = 1 - f->bias;
    if (a >= f->maxnorm) {
        mag = f->maxnorm;
    } else if (a == 0.0) {
        mag = 0.0;
    } else {
        int k = floor_log2(a);
        int kk = k < emin ? emin : k;
        double quantum = ldexp(1.0, kk - f->mbits); /* grid spacing around a */
        double t = a / quantum;                      /* exact: power-of-two division */
        double n = floor(t);
        double F = floor(ldexp(t - n, 32));          /* < 2^32, exact */
        if ((double)r < F) n += 1.0;
        mag = n * quantum;
        if (mag > f->maxnorm) mag = f->maxnorm;
    }
    return encode_elem(neg ? -mag : mag, f); /* mag is on the grid: no further rounding */
}

/* ---------------------------------------------------------------------------
 * exported API.  Return 0 on success, -1 on a bad argument.
 */

void oracle_philox4x32_10(const uint32_t *ctr, const uint32_t *key, uint32_t *out)
{
    philox4x32_10(ctr, key, out);
}

/* stochastically rounded element codes of v[i] * 2^-e[i] with random words r[i] */
int oracle_cast_sr_many(const double *v, const int32_t *e, const uint32_t *r, int64_t n, int fmt, uint8_t *out)
{
    if (!valid_fmt(fmt)) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = encode_elem_sr(ldexp(v[i], -e[i]), r[i], &FMT[fmt]);
    return 0;
}

/* the random words the stochastic-rounding quantizer uses for elements start .. start+n-1 */
int oracle_sr_words(uint64_t seed, int64_t start, int64_t n, uint32_t *out)
{
    if (n < 0 || start < 0) return -1;
    for (int64_t i = 0; i < n; i++) out[i] = sr_word((uint64_t)(start + i), seed);
    return 0;
}

float oracle_hadamard_c(void) { return hadamard_c(); }

/* y = RN32(1/sqrt32) * H32 * diag(s) * x on 32 floats */
void oracle_hadamard32_f32(const float *x, uint32_t mask, float *y)
{
    float t[32];
    memcpy(t, x, sizeof t);
    hadamard32(t, mask);
    memcpy(y, t, sizeof t);
}

/* scale bytes for an array of finite amax values */
int oracle_e8m0_many(const double *amax, int64_t n, int fmt, uint8_t *out)
{
    if (!valid_fmt(fmt)) return -1;
    for (int64_t i = 0; i < n; i++) out[i] = (uint8_t)e8m0_of_amax(amax[i], &FMT[fmt]);
    return 0;
}

/* element codes of v[i] * 2^-e[i] for arrays of finite v and e in [-127, 127] */
int oracle_cast_many(const double *v, const int32_t *e, int64_t n, int fmt, uint8_t *out)
{
    if (!valid_fmt(fmt)) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = encode_elem(ldexp(v[i], -e[i]), &FMT[fmt]);
    return 0;
}

/* decoded element values (no block scale) of n codes (unpacked, one per byte) */
int oracle_decode_many(const uint8_t *codes, int64_t n, int fmt, double *out)
{
    if (!valid_fmt(fmt)) return -1;
    for (int64_t i = 0; i < n; i++) out[i] = decode_elem(codes[i], fmt);
    return 0;
}

/* Row mode on bf16: blocks x[r, 32b .. 32b+31].
 * codes [rows x cols] (FP8) or [rows x cols/2] (E2M1); scales [rows x cols/32]. */
int oracle_quantize_rows(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                         uint8_t *codes, uint8_t *scales)
{
    if (!valid_fmt(fmt) || rows < 0 || cols < 0 || cols % 32 || ldx < cols) return -1;
    int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        double v[32];
        uint8_t c[32];
        for (int64_t b = 0; b < nb; b++) {
            for (int i = 0; i < 32; i++) v[i] = bf16_value(x[r * ldx + 32 * b + i]);
            quantize_block(v, &FMT[fmt], c, &scales[r * nb + b]);
            store_block(c, fmt, codes + r * code_bytes(cols, fmt) + code_bytes(32 * b, fmt));
        }
    }
    return 0;
}

/* Row mode on exact doubles (rows x cols, contiguous): used to re-quantize
 * dequantized values, which need not be bf16 numbers. */
int oracle_quantize_rows_f64(const double *x, int64_t rows, int64_t cols, int fmt,
                             uint8_t *codes, uint8_t *scales)
{
    if (!valid_fmt(fmt) || rows < 0 || cols < 0 || cols % 32) return -1;
    int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        uint8_t c[32];
        for (int64_t b = 0; b < nb; b++) {
            quantize_block(&x[r * cols + 32 * b], &FMT[fmt], c, &scales[r * nb + b]);
            store_block(c, fmt, codes + r * code_bytes(cols, fmt) + code_bytes(32 * b, fmt));
        }
    }
    return 0;
}

/* Transposed mode on bf16: blocks x[32b .. 32b+31, c]; block b of column c is
 * written to output row c.  codes [cols x rows] (FP8) or [cols x rows/2];
 * scales [cols x rows/32]. */
int oracle_quantize_transpose(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                              uint8_t *codes, uint8_t *scales)
{
    if (!valid_fmt(fmt) || rows < 0 || cols < 0 || rows % 32 || ldx < cols) return -1;
    int64_t nb = rows / 32;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; c++) {
        double v[32];
        uint8_t q[32];
        for (int64_t b = 0; b < nb; b++) {
            for (int i = 0; i < 32; i++) v[i] = bf16_value(x[(32 * b + i) * ldx + c]);
            quantize_block(v, &FMT[fmt], q, &scales[c * nb + b]);
            store_block(q, fmt, codes + c * code_bytes(rows, fmt) + code_bytes(32 * b, fmt));
        }
    }
    return 0;
}

/* Transposed mode after the rotation: each 32-row block of column c is
 * rotated (fp32, as hadamard32 above), then quantized from the fp32 values. */
int oracle_hadamard32_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx,
                               uint32_t mask, int fmt, uint8_t *codes, uint8_t *scales)
{
    if (!valid_fmt(fmt) || rows < 0 || cols < 0 || rows % 32 || ldx < cols) return -1;
    int64_t nb = rows / 32;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; c++) {
        float t[32];
        double v[32];
        uint8_t q[32];
        for (int64_t b = 0; b < nb; b++) {
            for (int i = 0; i < 32; i++) t[i] = (float)bf16_value(x[(32 * b + i) * ldx + c]);
            hadamard32(t, mask);
            for (int i = 0; i < 32; i++) v[i] = (double)t[i];
            quantize_block(v, &FMT[fmt], q, &scales[c * nb + b]);
            store_block(q, fmt, codes + c * code_bytes(rows, fmt) + code_bytes(32 * b, fmt));
        }
    }
    return 0;
}

/* Dequantize an MX operand: out[r, k] = decode(code) * 2^(S - 127);
 * a scale byte of 0xFF (E8M0 NaN) gives NaN. */
int oracle_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                      int fmt, double *out)
{
    if (!valid_fmt(fmt) || rows < 0 || cols < 0 || cols % 32) return -1;
    int64_t nb = cols / 32, rb = code_bytes(cols, fmt);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t k = 0; k < cols; k++) {
            uint8_t byte = (fmt == ORC_E2M1) ? codes[r * rb + k / 2] : codes[r * rb + k];
            uint8_t code = (fmt == ORC_E2M1) ? (uint8_t)((k & 1) ? (byte >> 4) : (byte & 0xF)) : byte;
            int S = scales[r * nb + k / 32];
            out[r * cols + k] = (S == 0xFF) ? NAN : ldexp(decode_elem(code, fmt), S - 127);
        }
    }
    return 0;
}

/* Transposed mode with stochastic rounding, optionally after the rotation:
 * as oracle_quantize_transpose / oracle_hadamard32_quantize (same blocks, same
 * scales), but element t of output row c is rounded with the random word of
 * output index c * rows + t. */
int oracle_quantize_transpose_sr(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx, int rotate,
                                 uint32_t mask, uint64_t seed, int fmt, uint8_t *codes, uint8_t *scales)
{
    if (!valid_fmt(fmt) || rows < 0 || cols < 0 || rows % 32 || ldx < cols || (rotate != 0 && rotate != 1))
        return -1;
    int64_t nb = rows / 32;
    const orc_fmt *f = &FMT[fmt];
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; c++) {
        float t[32];
        double v[32];
        uint8_t q[32];
        for (int64_t b = 0; b < nb; b++) {
            for (int i = 0; i < 32; i++) t[i] = (float)bf16_value(x[(32 * b + i) * ldx + c]);
            if (rotate) hadamard32(t, mask);
            for (int i = 0; i < 32; i++) v[i] = (double)t[i];
            /* the scale and the non-finite rule of the round-to-nearest path */
            quantize_block(v, f, q, &scales[c * nb + b]);
            if (scales[c * nb + b] != 0xFF) {
                int e = scales[c * nb + b] - 127;
                for (int i = 0; i < 32; i++)
                    q[i] = encode_elem_sr(ldexp(v[i], -e), sr_word((uint64_t)(c * rows + 32 * b + i), seed), f);
            }
            store_block(q, fmt, codes + c * code_bytes(rows, fmt) + code_bytes(32 * b, fmt));
        }
    }
    return 0;
}
