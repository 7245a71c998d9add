/*
 * Float64 reference products with a stored int4 g128 matrix, for the oracle.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE: used by the tests (through
 * oracle/cref.py) to evaluate full-size expert matrices that numpy cannot
 * dequantize in reasonable time.  Independent of the HIP library: it decodes
 * the storage format from its definition and converts fp16 itself.
 *
 *   y[t][n] = sum_c q[n][c] * s[n][c / 128] * x[t][c]      (all in double)
 *
 * Quantization: lpnh.cn/news/2730718 §2.1 (symmetric int4, 128 weights per
 * group along in_features, fp16 group scales).  Storage (this library's
 * format): code q stored as nibble q + 8; 8 consecutive columns per 32-bit
 * little-endian word with nibble p holding column {0,2,4,6,1,3,5,7}[p]; rows
 * in tiles of 16, each 16-byte chunk (32 columns) of the 16 rows side by side:
 *     byte(n, chunk c, b) = (n/16)*16*(in/2) + c*256 + (n%16)*16 + b
 *     scale(n, g)         = (n/16)*16*(in/128) + g*16 + n%16
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC w4_matvec.c -o libw4ref.so
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* IEEE binary16 bit pattern -> double (exact). */
static double half_to_double(uint16_t h) {
    const int sign = (h >> 15) & 1;
    const int exp = (h >> 10) & 0x1f;
    const int man = h & 0x3ff;
    double v;
    if (exp == 0)
        v = ldexp((double)man, -24);                 /* zero / subnormal */
    else if (exp == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(man | 0x400), exp - 25);  /* 1.man * 2^(exp-15) */
    return sign ? -v : v;
}

/* column (within 8) held by nibble p of a word */
static const int kNibbleCol[8] = {0, 2, 4, 6, 1, 3, 5, 7};

/* Decode row n of the stored matrix into q_row[in_dim] (codes -8..7) and
 * s_row[in_dim/128]. */
static void decode_row(const uint8_t *q, const uint16_t *s, int64_t n, int64_t in_dim,
                       int8_t *q_row, double *s_row) {
    const int64_t half_in = in_dim / 2, groups = in_dim / 128;
    const uint8_t *tile = q + (n / 16) * 16 * half_in;
    for (int64_t c = 0; c < in_dim / 32; ++c) {          /* 16-byte chunks */
        const uint8_t *chunk = tile + c * 256 + (n % 16) * 16;
        for (int w = 0; w < 4; ++w) {                     /* 32-bit words */
            uint32_t word = (uint32_t)chunk[4 * w] | ((uint32_t)chunk[4 * w + 1] << 8) |
                            ((uint32_t)chunk[4 * w + 2] << 16) |
                            ((uint32_t)chunk[4 * w + 3] << 24);
            for (int p = 0; p < 8; ++p)
                q_row[c * 32 + w * 8 + kNibbleCol[p]] = (int8_t)((word >> (4 * p)) & 15) - 8;
        }
    }
    const uint16_t *stile = s + (n / 16) * 16 * groups;
    for (int64_t g = 0; g < groups; ++g) s_row[g] = half_to_double(stile[g * 16 + n % 16]);
}

/* y [ntok][out_dim] = x [ntok][in_dim] times the dequantized matrix,
 * transposed.  in_dim a multiple of 128 (and at most 262144), out_dim a
 * multiple of 16. */
void w4_matvec(const uint8_t *q, const uint16_t *s, int64_t out_dim, int64_t in_dim,
               const double *x, int64_t ntok, double *y) {
#pragma omp parallel
    {
        static __thread int8_t q_row[262144];
        static __thread double s_row[2048];
#pragma omp for schedule(static)
        for (int64_t n = 0; n < out_dim; ++n) {
            decode_row(q, s, n, in_dim, q_row, s_row);
            for (int64_t t = 0; t < ntok; ++t) {
                const double *xt = x + t * in_dim;
                double acc = 0.0;
                for (int64_t g = 0; g < in_dim / 128; ++g) {
                    double part = 0.0;
                    for (int c = 0; c < 128; ++c) part += (double)q_row[g * 128 + c] * xt[g * 128 + c];
                    acc += s_row[g] * part;
                }
                y[t * out_dim + n] = acc;
            }
        }
    }
}

/* Decode rows [r0, r1) to float64 weights W[r1-r0][in_dim] (for checks). */
void w4_dequant_rows(const uint8_t *q, const uint16_t *s, int64_t in_dim, int64_t r0, int64_t r1,
                     double *out) {
    static __thread int8_t q_row[262144];
    static __thread double s_row[2048];
    for (int64_t n = r0; n < r1; ++n) {
        decode_row(q, s, n, in_dim, q_row, s_row);
        for (int64_t c = 0; c < in_dim; ++c)
            out[(n - r0) * in_dim + c] = (double)q_row[c] * s_row[c / 128];
    }
}
