/*
 * Float64 reference products with a stored int4 g128 matrix, for the oracle.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE: used by the tests (through
 * oracle/cref.py) to evaluate full-size expert matrices that numpy cannot
 * dequantize in reasonable time.  Independent of the HIP library: it decodes
 * the storage format from its definition and converts fp16 itself.
 *
 *   y[t][n] = sum_c q[n][c] * s[n][c / gs] * x[t][c]      (all in double)
 *
 * Quantization: lpnh.cn/news/2730718 §2.1 (symmetric int4, 128 weights per
 * group along in_features, fp16 group scales; the page also compares groups
 * of 64 and 256, so gs is 64, 128 or 256).  Storage (this library's
 * format): code q stored as nibble q + 8; 8 consecutive columns per 32-bit
 * little-endian word with nibble p holding column {0,2,4,6,1,3,5,7}[p]; rows
 * in tiles of 16, each 16-byte chunk (32 columns) of the 16 rows side by side:
 *     byte(n, chunk c, b) = (n/16)*16*(in/2) + c*256 + (n%16)*16 + b
 *     scale(n, g)         = (n/16)*16*(in/gs) + g*16 + n%16
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
 * s_row[in_dim/gs]. */
static void decode_row(const uint8_t *q, const uint16_t *s, int64_t n, int64_t in_dim,
                       int64_t gs, int8_t *q_row, double *s_row) {
    const int64_t half_in = in_dim / 2, groups = in_dim / gs;
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

/* Shapes the decoder handles: group size 64, 128 or 256; in_dim a multiple
 * of 128 and of gs, at most 262144; out_dim a multiple of 16. */
static int shape_ok(int64_t out_dim, int64_t in_dim, int64_t gs) {
    return (gs == 64 || gs == 128 || gs == 256) && in_dim > 0 && in_dim % 128 == 0 &&
           in_dim % gs == 0 && in_dim <= 262144 && out_dim >= 0 && out_dim % 16 == 0;
}

/* y [ntok][out_dim] = x [ntok][in_dim] times the dequantized matrix,
 * transposed, with gs-column scale groups.  Returns 0, or -1 (nothing
 * written) for a shape outside shape_ok. */
int w4_matvec(const uint8_t *q, const uint16_t *s, int64_t out_dim, int64_t in_dim, int64_t gs,
              const double *x, int64_t ntok, double *y) {
    if (!shape_ok(out_dim, in_dim, gs)) return -1;
#pragma omp parallel
    {
        static __thread int8_t q_row[262144];
        static __thread double s_row[4096];
#pragma omp for schedule(static)
        for (int64_t n = 0; n < out_dim; ++n) {
            decode_row(q, s, n, in_dim, gs, q_row, s_row);
            for (int64_t t = 0; t < ntok; ++t) {
                const double *xt = x + t * in_dim;
                double acc = 0.0;
                for (int64_t g = 0; g < in_dim / gs; ++g) {
                    double part = 0.0;
                    for (int64_t c = 0; c < gs; ++c) part += (double)q_row[g * gs + c] * xt[g * gs + c];
                    acc += s_row[g] * part;
                }
                y[t * out_dim + n] = acc;
            }
        }
    }
    return 0;
}

/* Decode rows [r0, r1) to float64 weights W[r1-r0][in_dim] (for checks).
 * Returns 0, or -1 (nothing written) for a shape outside shape_ok. */
int w4_dequant_rows(const uint8_t *q, const uint16_t *s, int64_t in_dim, int64_t gs, int64_t r0,
                    int64_t r1, double *out) {
    if (!shape_ok(16, in_dim, gs) || r0 < 0 || r1 < r0) return -1;
    static __thread int8_t q_row[262144];
    static __thread double s_row[4096];
    for (int64_t n = r0; n < r1; ++n) {
        decode_row(q, s, n, in_dim, gs, q_row, s_row);
        for (int64_t c = 0; c < in_dim; ++c)
            out[(n - r0) * in_dim + c] = (double)q_row[c] * s_row[c / gs];
    }
    return 0;
}
