/*
 * qmv_oracle.c -- plain CPU oracle for the block-quantized matrix-vector product.
 *
 * TEST INFRASTRUCTURE. Only the test-suite, the package's smoke check and the
 * benchmark's CPU-baseline leg may load this library. The GPU library neither
 * links nor calls it, and this file includes nothing from the GPU library.
 *
 * What is computed (rullama 0.5.0, src/backend/matmul.rs: the module doc says
 * each dispatcher takes the weight bytes as stored in GGUF and returns
 * y = x @ W of length n; the test helper `cpu_matmul_f32` defines it as
 * y[j] = sum_i w[j*k + i] * x[i], i.e. W is n rows of k weights):
 *
 *     y[t][j] = sum_{i<k} x[t][i] * w_j[i]
 *     s[t][j] = sum_{i<k} |x[t][i] * w_j[i]|        (the tolerance scale)
 *
 * and the transposed (backward-input) product over a row range, as the
 * backward-input kernels of dispatch/mod.rs compute it (struct
 * MatmulBackInputParams: j_start..j_end bounds the summed row axis; the CPU
 * reference of its parity tests maps dy of length n to dx of length k):
 *
 *     dx[t][i] = sum_{j0<=j<j1} dy[t][j] * w_j[i]
 *     s[t][i]  = sum_{j0<=j<j1} |dy[t][j] * w_j[i]|
 *
 * and the same forward product over affine group-quantized weights (moeflux,
 * tests/graph_diff_oracle.rs: 4-bit or 8-bit codes packed in u32 words, one
 * bf16 scale and one bf16 bias per group of 64 weights, value
 * code * scale + bias).
 *
 * Every weight is first decoded to an f32 value, element by element, then the
 * sum runs serially over i in f64. There is no blocking, no factoring of the
 * block scales and no reordering: the decode of element i of row j looks up
 * its own block and field and nothing else.
 *
 * Block layouts. The pages give the block sizes (Q4_0 18 bytes per 32 weights,
 * Q4_K 144 bytes per 256, Q6_K 210 bytes per 256: matmul.rs, fns matmul_q4_0,
 * matmul_q4_k, matmul_q6_k; Q8_0 and Q5_0 blocks of 32 weights laid out field
 * by field in the expert-matmul tests of dispatch/mod.rs) and where the f16 scale fields sit (dispatch/mod.rs,
 * the backward-input parity tests: Q4_0 d at bytes 0..2, Q4_K d at 0..2 and
 * dmin at 2..4, Q6_K d in the last two bytes). They call the CPU dequantizers
 * "ggml-exact" (matmul.rs, test q4_0_matmul_gpu_vs_cpu_oracle) but do not print
 * them. The field order inside each block below is therefore the ggml block
 * layout that name refers to, restated from its definition. That reading is
 * pinned by hand-built blocks and invariants in the tests; agreement with real
 * GGUF files is "parity unpinned" (no such file is available).
 *
 * Multi-byte fields are little-endian (the pages serialise with to_le_bytes).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F16 1
#define ORACLE_BF16 2
#define ORACLE_Q4_0 3
#define ORACLE_Q4_K 4
#define ORACLE_Q6_K 5
#define ORACLE_Q8_0 6
#define ORACLE_Q5_0 7

/* ---------------------------------------------------------------- scalars */

/* IEEE 754 binary16 -> f32, from the format's definition: 1 sign bit, 5
 * exponent bits (bias 15), 10 fraction bits. Exact for every finite input,
 * subnormals included (every f16 value is an f32 value). */
float oracle_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24); /* subnormal: 0.f * 2^-14 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25); /* 1.f * 2^(e-15) */
    return (float)(sign ? -v : v);
}

/* bfloat16 -> f32: the stored 16 bits are the upper half of an f32
 * (matmul.rs, doc of fn matmul_bf16). */
float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint16_t rd_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* ------------------------------------------------------------ block sizes */

int64_t oracle_block_elems(int fmt)
{
    switch (fmt) {
    case ORACLE_F16:
    case ORACLE_BF16: return 1;
    case ORACLE_Q4_0:
    case ORACLE_Q8_0:
    case ORACLE_Q5_0: return 32;
    case ORACLE_Q4_K:
    case ORACLE_Q6_K: return 256;
    default: return -1;
    }
}

int64_t oracle_block_bytes(int fmt)
{
    switch (fmt) {
    case ORACLE_F16:
    case ORACLE_BF16: return 2;
    case ORACLE_Q4_0: return 18;
    case ORACLE_Q4_K: return 144;
    case ORACLE_Q6_K: return 210;
    case ORACLE_Q8_0: return 34;
    case ORACLE_Q5_0: return 22;
    default: return -1;
    }
}

/* Bytes of one row of k weights, or -1 when k is not a whole number of blocks. */
int64_t oracle_row_bytes(int fmt, int64_t k)
{
    int64_t qk = oracle_block_elems(fmt);
    if (qk <= 0 || k < 0 || k % qk != 0)
        return -1;
    return (k / qk) * oracle_block_bytes(fmt);
}

/* ---------------------------------------------------- per-element decoders */

/* Q4_0, 32 weights in 18 bytes: f16 d, then 16 bytes of 4-bit codes.
 * Element e < 16 is the low nibble of byte e, element e >= 16 the high nibble
 * of byte e-16. Value (q - 8) * d: exact in f32 (11-bit d times a 4-bit
 * integer). */
float oracle_q4_0_elem(const uint8_t *blk, int e)
{
    float d = oracle_f16_to_f32(rd_u16(blk));
    const uint8_t *qs = blk + 2;
    int q = (e < 16) ? (qs[e] & 0x0f) : (qs[e - 16] >> 4);
    return d * (float)(q - 8);
}

/* Q4_K: the 6-bit scale and 6-bit min of sub-block s (0..7) from the 12
 * packed bytes. Sub-blocks 0..3 keep theirs in the low 6 bits of bytes s and
 * s+4; sub-blocks 4..7 take their low 4 bits from the two nibbles of byte s+4
 * and their top 2 bits from the top bits of bytes s-4 (scale) and s (min). */
void oracle_q4_k_scale_min(const uint8_t *sc, int s, int *scale, int *min)
{
    if (s < 4) {
        *scale = sc[s] & 63;
        *min = sc[s + 4] & 63;
    } else {
        *scale = (sc[s + 4] & 0x0f) | ((sc[s - 4] >> 6) << 4);
        *min = (sc[s + 4] >> 4) | ((sc[s] >> 6) << 4);
    }
}

/* Q4_K, 256 weights in 144 bytes: f16 d, f16 dmin, 12 bytes of packed
 * scales/mins, 128 bytes of 4-bit codes. The super-block is four 64-weight
 * chunks; in chunk c, code byte 32c+l carries element 64c+l in its low nibble
 * (sub-block 2c) and element 64c+32+l in its high nibble (sub-block 2c+1).
 * Value (d*scale)*q - dmin*min: both products are exact in f32, the
 * subtraction rounds once. */
float oracle_q4_k_elem(const uint8_t *blk, int e)
{
    float d = oracle_f16_to_f32(rd_u16(blk));
    float dmin = oracle_f16_to_f32(rd_u16(blk + 2));
    const uint8_t *sc = blk + 4;
    const uint8_t *qs = blk + 16;
    int c = e / 64, h = (e % 64) / 32, l = e % 32;
    int q = (qs[32 * c + l] >> (4 * h)) & 0x0f;
    int scale, min;
    oracle_q4_k_scale_min(sc, 2 * c + h, &scale, &min);
    float a = (d * (float)scale) * (float)q;
    float b = dmin * (float)min;
    return a - b;
}

/* Q6_K, 256 weights in 210 bytes: 128 bytes ql (low 4 bits), 64 bytes qh
 * (high 2 bits), 16 signed 8-bit scales, f16 d last. The super-block is two
 * halves of 128; in half h, quarter g (0..3) and position l (0..31) the low
 * bits come from ql[64h + 32*(g%2) + l] (low nibble for g<2, high nibble for
 * g>=2), the high bits are bits 2g..2g+1 of qh[32h + l], and the scale is
 * scales[8h + 2g + l/16]. Value (d*scale)*(q - 32). */
float oracle_q6_k_elem(const uint8_t *blk, int e)
{
    const uint8_t *ql = blk;
    const uint8_t *qh = blk + 128;
    const int8_t *scales = (const int8_t *)(blk + 192);
    float d = oracle_f16_to_f32(rd_u16(blk + 208));
    int h = e / 128, r = e % 128, g = r / 32, l = r % 32;
    int lo = (ql[64 * h + 32 * (g % 2) + l] >> (4 * (g / 2))) & 0x0f;
    int hi = (qh[32 * h + l] >> (2 * g)) & 3;
    int q = lo | (hi << 4);
    float ds = d * (float)scales[8 * h + 2 * g + l / 16];
    return ds * (float)(q - 32);
}

/* Q8_0, 32 weights in 34 bytes: f16 d, then one signed 8-bit code per
 * element in element order. Value d * q: exact in f32.
 * (rullama 0.5.0, src/backend/dispatch/mod.rs, the batched expert-matmul
 * test: blocks of QK8_0 weights with d in bytes 0..2 and the code bytes
 * from byte 2 on; the signed reading is ggml's.) */
float oracle_q8_0_elem(const uint8_t *blk, int e)
{
    float d = oracle_f16_to_f32(rd_u16(blk));
    int q = (int)(int8_t)blk[2 + e];
    return d * (float)q;
}

/* Q5_0, 32 weights in 22 bytes: f16 d, a little-endian 32-bit word qh of
 * fifth bits, 16 bytes of 4-bit codes. Element e takes the low nibble of code
 * byte e (e < 16) or the high nibble of code byte e-16 (e >= 16) as its low
 * four bits and bit e of qh as its fifth bit; value d * (q - 16), exact in
 * f32. (Same page and test module as Q8_0, the Q5_0 expert-matmul test: d in
 * bytes 0..2, qh in bytes 2..6, the 16 code bytes from byte 6 on; the element
 * order and the offset 16 are ggml's.) */
float oracle_q5_0_elem(const uint8_t *blk, int e)
{
    float d = oracle_f16_to_f32(rd_u16(blk));
    uint32_t qh = (uint32_t)blk[2] | ((uint32_t)blk[3] << 8) | ((uint32_t)blk[4] << 16) |
                  ((uint32_t)blk[5] << 24);
    const uint8_t *qs = blk + 6;
    int lo = (e < 16) ? (qs[e] & 0x0f) : (qs[e - 16] >> 4);
    int hi = (int)((qh >> e) & 1u);
    int q = lo | (hi << 4);
    return d * (float)(q - 16);
}

/* Decode weight i of one row (row points at the row's first byte). */
float oracle_elem(int fmt, const uint8_t *row, int64_t i)
{
    switch (fmt) {
    case ORACLE_F16: return oracle_f16_to_f32(rd_u16(row + 2 * i));
    case ORACLE_BF16: return oracle_bf16_to_f32(rd_u16(row + 2 * i));
    case ORACLE_Q4_0: return oracle_q4_0_elem(row + (i / 32) * 18, (int)(i % 32));
    case ORACLE_Q4_K: return oracle_q4_k_elem(row + (i / 256) * 144, (int)(i % 256));
    case ORACLE_Q6_K: return oracle_q6_k_elem(row + (i / 256) * 210, (int)(i % 256));
    case ORACLE_Q8_0: return oracle_q8_0_elem(row + (i / 32) * 34, (int)(i % 32));
    case ORACLE_Q5_0: return oracle_q5_0_elem(row + (i / 32) * 22, (int)(i % 32));
    default: return NAN;
    }
}

/* Decode one whole row of k weights into w[0..k). Returns 0, or -1 on a bad
 * format or k. */
int oracle_dequant_row(int fmt, const uint8_t *row, int64_t k, float *w)
{
    if (oracle_row_bytes(fmt, k) < 0)
        return -1;
    for (int64_t i = 0; i < k; i++)
        w[i] = oracle_elem(fmt, row, i);
    return 0;
}

/* ------------------------------------------------------------------- gemv */

/* For each listed row j = rows[r] and each token t < m:
 *   y[t*nrows + r] = sum_i x[t*k + i] * w_j[i]          (f64, serial in i)
 *   s[t*nrows + r] = sum_i |x[t*k + i] * w_j[i]|
 * W holds n rows of row_bytes(fmt, k) bytes; x is m rows of k f32. s may be
 * NULL. Returns 0, -1 on bad arguments, -2 if out of memory. */
int oracle_gemv_rows(int fmt, const uint8_t *W, const float *x, int64_t k, int64_t n,
                     int64_t m, const int64_t *rows, int64_t nrows, double *y, double *s)
{
    int64_t rb = oracle_row_bytes(fmt, k);
    if (rb < 0 || n < 0 || m < 0 || nrows < 0)
        return -1;
    float *w = (float *)malloc((size_t)(k > 0 ? k : 1) * sizeof(float));
    if (!w)
        return -2;
    for (int64_t r = 0; r < nrows; r++) {
        int64_t j = rows[r];
        if (j < 0 || j >= n) {
            free(w);
            return -1;
        }
        oracle_dequant_row(fmt, W + j * rb, k, w);
        for (int64_t t = 0; t < m; t++) {
            double acc = 0.0, mag = 0.0;
            for (int64_t i = 0; i < k; i++) {
                double p = (double)x[t * k + i] * (double)w[i];
                acc += p;
                mag += fabs(p);
            }
            y[t * nrows + r] = acc;
            if (s)
                s[t * nrows + r] = mag;
        }
    }
    free(w);
    return 0;
}

/* The contiguous-range form: rows j0 <= j < j1, outputs indexed j - j0. */
int oracle_gemv_range(int fmt, const uint8_t *W, const float *x, int64_t k, int64_t n,
                      int64_t m, int64_t j0, int64_t j1, double *y, double *s)
{
    if (j0 < 0 || j1 < j0 || j1 > n)
        return -1;
    int64_t nr = j1 - j0;
    int64_t *rows = (int64_t *)malloc((size_t)(nr > 0 ? nr : 1) * sizeof(int64_t));
    if (!rows)
        return -2;
    for (int64_t r = 0; r < nr; r++)
        rows[r] = j0 + r;
    int rc = oracle_gemv_rows(fmt, W, x, k, n, m, rows, nr, y, s);
    free(rows);
    return rc;
}

/* ------------------------------------------------------- transposed gemv */

/* For each listed column i = cols[c] and each token t < m:
 *   dx[t*ncols + c] = sum_{j0 <= j < j1} dy[t*n + j] * w_j[i]   (f64, serial in j)
 *   s[t*ncols + c]  = sum_{j0 <= j < j1} |dy[t*n + j] * w_j[i]|
 * W holds n rows of row_bytes(fmt, k) bytes; dy is m rows of n f32. Every
 * weight is decoded on its own (oracle_elem). s may be NULL. Returns 0, or -1
 * on bad arguments. */
int oracle_gemv_t_cols(int fmt, const uint8_t *W, const float *dy, int64_t k, int64_t n,
                       int64_t m, int64_t j0, int64_t j1, const int64_t *cols, int64_t ncols,
                       double *dx, double *s)
{
    int64_t rb = oracle_row_bytes(fmt, k);
    if (rb < 0 || n < 0 || m < 0 || ncols < 0 || j0 < 0 || j1 < j0 || j1 > n)
        return -1;
    for (int64_t c = 0; c < ncols; c++) {
        int64_t i = cols[c];
        if (i < 0 || i >= k)
            return -1;
        for (int64_t t = 0; t < m; t++) {
            double acc = 0.0, mag = 0.0;
            for (int64_t j = j0; j < j1; j++) {
                double p = (double)dy[t * n + j] * (double)oracle_elem(fmt, W + j * rb, i);
                acc += p;
                mag += fabs(p);
            }
            dx[t * ncols + c] = acc;
            if (s)
                s[t * ncols + c] = mag;
        }
    }
    return 0;
}

/* ------------------------------------------------------- affine weights */

/* Weight i of one row of affine group-quantized weights (moeflux,
 * tests/graph_diff_oracle.rs, the 4-bit embedding fixture: codes packed into
 * u32 words, k*bits/32 words per row; bf16 scales and biases, k/64 per row).
 * Element i is code number i mod (32/bits) of word i / (32/bits), counted
 * from the least significant bits (the pages do not print the order inside
 * a word; lowest first is this reading). Value code * scale + bias, with
 * scale and bias of group i / 64: the product is exact in f32 (an 8-bit bf16
 * significand times a code of at most 8 bits), the addition rounds once. */
float oracle_affine_elem(int bits, const uint32_t *words, const uint16_t *scales,
                         const uint16_t *biases, int64_t i)
{
    int per = 32 / bits;
    uint32_t mask = (bits == 8) ? 0xffu : 0x0fu;
    uint32_t w = words[i / per];
    uint32_t q = (w >> (bits * (int)(i % per))) & mask;
    float sc = oracle_bf16_to_f32(scales[i / 64]);
    float bi = oracle_bf16_to_f32(biases[i / 64]);
    return (float)q * sc + bi;
}

/* y, s of the forward product for the listed rows (as oracle_gemv_rows), W
 * given as words [n][k*bits/32], scales and biases [n][k/64]. bits is 4 or 8
 * and k a multiple of 64. Returns 0, -1 on bad arguments, -2 if out of
 * memory. */
int oracle_affine_gemv_rows(int bits, const uint32_t *words, const uint16_t *scales,
                            const uint16_t *biases, const float *x, int64_t k, int64_t n,
                            int64_t m, const int64_t *rows, int64_t nrows, double *y, double *s)
{
    if ((bits != 4 && bits != 8) || k < 0 || k % 64 != 0 || n < 0 || m < 0 || nrows < 0)
        return -1;
    int64_t wpr = k * bits / 32, gpr = k / 64;
    float *w = (float *)malloc((size_t)(k > 0 ? k : 1) * sizeof(float));
    if (!w)
        return -2;
    for (int64_t r = 0; r < nrows; r++) {
        int64_t j = rows[r];
        if (j < 0 || j >= n) {
            free(w);
            return -1;
        }
        for (int64_t i = 0; i < k; i++)
            w[i] = oracle_affine_elem(bits, words + j * wpr, scales + j * gpr, biases + j * gpr, i);
        for (int64_t t = 0; t < m; t++) {
            double sum = 0.0, bound = 0.0;
            for (int64_t e = 0; e < k; e++) {
                double prod = (double)x[t * k + e] * (double)w[e];
                sum += prod;
                bound += fabs(prod);
            }
            y[t * nrows + r] = sum;
            if (s)
                s[t * nrows + r] = bound;
        }
    }
    free(w);
    return 0;
}
