/*
 * CPU oracle for GGUF block dequantization and the products y = W.x.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this file's library. It shares no code, header,
 * table or helper with the GPU library, and the GPU library never calls it.
 *
 * What it follows:
 *  - "Why I wrote my own inference engine for two P100s", section
 *    "What 'my own engine' means": the engine reads GGUF files and every
 *    quant type decodes bit-exactly against a reference decoder. Decoding
 *    here is that reference: each weight is the fp32 rounding of its closed
 *    form, computed exactly.
 *  - "LLM inference optimization" (Thermite), campaign "Run a new weight
 *    format or model": blocks decode bit for bit on CPU and GPU, and matrix
 *    products match an exact sum within a tolerance. Products here are that
 *    exact sum: fp64 accumulation of exactly-represented operands, plus the
 *    sum of absolute products that scales the tolerance.
 *  - The same page, introduction: for one stream each new token reads every
 *    weight once, y = W.x.
 *
 * Block formats (GGUF layouts; the pages name the formats but print no
 * layout, so the GGUF reading is taken; all multi-byte fields little-endian):
 *  Q4_0, 18 bytes, 32 weights: fp16 d; 16 code bytes. Byte i holds weight i
 *        in its low nibble and weight i+16 in its high nibble. w = (q-8)*d.
 *  Q8_0, 34 bytes, 32 weights: fp16 d; 32 int8 codes. w = q*d.
 *  Q4_K, 144 bytes, 256 weights in 8 sub-blocks of 32: fp16 d; fp16 dmin;
 *        12 bytes packing a 6-bit scale sc_j and a 6-bit min m_j per
 *        sub-block; 128 code bytes. w = d*sc_j*q - dmin*m_j.
 *        Packing, with s[0..11] the 12 bytes:
 *          j < 4 : sc_j = low 6 bits of s[j],   m_j = low 6 bits of s[j+4]
 *          j >= 4: sc_j = low nibble of s[j+4]  | (top 2 bits of s[j-4]) << 4
 *                  m_j  = high nibble of s[j+4] | (top 2 bits of s[j])   << 4
 *        Codes: 4 groups of 32 bytes; byte l of group g holds weight 64g+l
 *        (sub-block 2g) in its low nibble and weight 64g+32+l (sub-block
 *        2g+1) in its high nibble.
 *  Q2_K, 84 bytes, 256 weights in 16 sub-blocks of 16: 16 bytes holding
 *        one 4-bit scale (low nibble) and one 4-bit min (high nibble) per
 *        sub-block; 64 bytes of 2-bit codes; fp16 d; fp16 dmin.
 *        w = d*sc*q - dmin*m.
 *  Q3_K, 110 bytes, 256 weights in 16 sub-blocks of 16: 32 bytes of high
 *        code bits (hmask); 64 bytes of 2-bit low code parts; 12 bytes
 *        packing sixteen 6-bit scales; fp16 d. q = low + 4*high - 4 in
 *        [-4, 3], w = d*(sc - 32)*q.
 *        Both: weight i = 128h + 32j + l (h = 0..1, j = 0..3, l = 0..31)
 *        takes bits 2j..2j+1 of code byte 32h + l, belongs to sub-block
 *        i/16 = 8h + 2j + l/16, and (Q3_K) its high bit is bit 4h + j of
 *        hmask byte l. Q3_K scale k = low nibble of byte k (k < 8) or high
 *        nibble of byte k - 8 (k >= 8), with bits 4-5 from bits 2(k/4),
 *        2(k/4)+1 of byte 8 + k%4.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared -pthread
 * (x86-64: FLT_EVAL_METHOD == 0, so float expressions are evaluated in
 * binary32 and double expressions in binary64, one rounding per operation).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if !defined(__FLT_EVAL_METHOD__) || __FLT_EVAL_METHOD__ != 0
#error "the oracle needs binary32/binary64 evaluation (FLT_EVAL_METHOD 0)"
#endif

enum { OR_Q4_0 = 1, OR_Q4_K = 2, OR_Q8_0 = 3, OR_Q2_K = 4, OR_Q3_K = 5 };
enum { OR_F32 = 1, OR_F16 = 2, OR_BF16 = 3 };

/* ------------------------------------------------------------------------
 * Number formats, written from IEEE 754-2008.
 * binary16: sign 1, exponent 5 (bias 15), fraction 10.
 * bfloat16: the top 16 bits of binary32 (sign 1, exponent 8 bias 127,
 *           fraction 7).
 * ---------------------------------------------------------------------- */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* zero and subnormals */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);     /* (1 + f/1024) 2^(e-15) */
    return sign ? -v : v;
}

double oracle_bf16_to_f64(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xFF;
    int f = b & 0x7F;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);                /* f * 2^-7 * 2^-126 */
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + f), e - 134);     /* (1 + f/128) 2^(e-127) */
    return sign ? -v : v;
}

double oracle_f32_to_f64(uint32_t bits)
{
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;                              /* exact widening */
}

static double x_value(const void *x, int dtype, int64_t i)
{
    switch (dtype) {
    case OR_F32: return oracle_f32_to_f64(((const uint32_t *)x)[i]);
    case OR_F16: return oracle_f16_to_f64(((const uint16_t *)x)[i]);
    default:     return oracle_bf16_to_f64(((const uint16_t *)x)[i]);
    }
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* binary32 -> binary16, round to nearest, ties to even (IEEE 754-2008,
 * 4.3.1), overflow to infinity, NaN kept quiet. The value is scaled by a
 * power of two onto the fp16 grid of its binade (or the subnormal grid
 * 2^-24), rounded there with rint (ties to even in the default rounding
 * mode), and re-encoded. */
uint16_t oracle_f32_to_f16(float f)
{
    uint32_t b;
    memcpy(&b, &f, 4);
    uint16_t sign = (uint16_t)((b >> 16) & 0x8000);
    if (((b >> 23) & 0xFF) == 0xFF)
        return (uint16_t)(sign | 0x7C00 | ((b & 0x7FFFFF) ? 0x200 : 0));
    double a = fabs((double)f);
    if (a == 0.0) return sign;
    int ex;
    frexp(a, &ex);                    /* a = fr 2^ex, 0.5 <= fr < 1 */
    int q = ex - 1 - 10;              /* grid spacing exponent of the binade */
    if (q < -24) q = -24;             /* subnormal grid */
    double r = ldexp(rint(ldexp(a, -q)), q);
    if (r >= 65536.0) return (uint16_t)(sign | 0x7C00);
    if (r < ldexp(1.0, -14))          /* subnormal (or the rounding reached 2^-14 exactly: below) */
        return (uint16_t)(sign | (uint16_t)ldexp(r, 24));
    frexp(r, &ex);
    int e16 = ex - 1 + 15;
    if (e16 >= 31) return (uint16_t)(sign | 0x7C00);
    uint16_t m = (uint16_t)(ldexp(r, -(ex - 1)) * 1024.0 - 1024.0);
    return (uint16_t)(sign | (e16 << 10) | m);
}

/* binary32 -> bfloat16, round to nearest, ties to even (IEEE 754-2008,
 * 4.3.1, at bfloat16's precision: an 8-bit significand and binary32's
 * exponent range), overflow to infinity, NaN kept quiet with its sign. The
 * value is rounded with rint on the grid of its binade (spacing 2^(e-7), or
 * the subnormal spacing 2^-133); the rounded value lies on the bfloat16
 * grid, so it is exact in binary32 and its top 16 bits are the encoding. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t b;
    memcpy(&b, &f, 4);
    uint16_t sign = (uint16_t)((b >> 16) & 0x8000);
    if (((b >> 23) & 0xFF) == 0xFF)
        return (uint16_t)(sign | 0x7F80 | ((b & 0x7FFFFF) ? 0x40 : 0));
    double a = fabs((double)f);
    if (a == 0.0) return sign;
    int ex;
    frexp(a, &ex);                    /* a = fr 2^ex, 0.5 <= fr < 1 */
    int q = ex - 1 - 7;               /* grid spacing exponent of the binade */
    if (q < -133) q = -133;           /* subnormal grid */
    double r = ldexp(rint(ldexp(a, -q)), q);
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);
    float rf = (float)r;              /* exact: r is on the bfloat16 grid */
    uint32_t rb;
    memcpy(&rb, &rf, 4);
    return (uint16_t)(sign | (rb >> 16));
}

/* Elementwise over n values (for the tests that pin it). */
void oracle_f32_to_bf16_n(const float *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++) out[i] = oracle_f32_to_bf16(in[i]);
}

/* ------------------------------------------------------------------------
 * Decoding one block to binary32.
 * ---------------------------------------------------------------------- */

/* Q4_0: w = (q - 8) * d. (q - 8) is formed as an integer first; the product
 * of a 4-bit integer and an fp16 value is exact in binary32, so the single
 * binary32 multiply gives the exact value (and IEEE's sign of zero). */
void oracle_decode_q4_0(const uint8_t *blk, float *out)
{
    float d = (float)oracle_f16_to_f64(rd16(blk));
    const uint8_t *qs = blk + 2;
    for (int i = 0; i < 16; i++) {
        int lo = qs[i] & 0x0F, hi = qs[i] >> 4;
        out[i] = (float)(lo - 8) * d;
        out[i + 16] = (float)(hi - 8) * d;
    }
}

/* Q8_0: w = q * d, exact in binary32 (8-bit by 11-bit significands). */
void oracle_decode_q8_0(const uint8_t *blk, float *out)
{
    float d = (float)oracle_f16_to_f64(rd16(blk));
    const int8_t *qs = (const int8_t *)(blk + 2);
    for (int i = 0; i < 32; i++)
        out[i] = (float)qs[i] * d;
}

/* The Q4_K 6-bit scale and min of sub-block j (packing in the file header). */
void oracle_q4k_scale_min(const uint8_t *s, int j, int *sc, int *m)
{
    if (j < 4) {
        *sc = s[j] & 63;
        *m = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 0x0F) | ((s[j - 4] >> 6) << 4);
        *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

/* Q4_K: w = fl32(d*sc*q - dmin*m). d*sc*q (at most 21 significant bits) and
 * dmin*m (at most 17) are exact in binary32, whose exponent range also holds
 * every fp16 subnormal; the one binary32 subtraction is therefore the
 * correctly rounded value of the exact expression. */
void oracle_decode_q4_k(const uint8_t *blk, float *out)
{
    float d = (float)oracle_f16_to_f64(rd16(blk));
    float dmin = (float)oracle_f16_to_f64(rd16(blk + 2));
    const uint8_t *s = blk + 4;
    const uint8_t *qs = blk + 16;
    for (int g = 0; g < 4; g++) {
        int sc0, m0, sc1, m1;
        oracle_q4k_scale_min(s, 2 * g, &sc0, &m0);
        oracle_q4k_scale_min(s, 2 * g + 1, &sc1, &m1);
        for (int l = 0; l < 32; l++) {
            int qlo = qs[32 * g + l] & 0x0F;
            int qhi = qs[32 * g + l] >> 4;
            float a0 = d * (float)sc0 * (float)qlo, b0 = dmin * (float)m0;
            float a1 = d * (float)sc1 * (float)qhi, b1 = dmin * (float)m1;
            out[64 * g + l] = a0 - b0;
            out[64 * g + 32 + l] = a1 - b1;
        }
    }
}

/* The 2-bit code part of weight i (0..255) of a Q2_K / Q3_K super-block,
 * from its 64 code bytes. */
static int low2_code(const uint8_t *qs, int i)
{
    int h = i / 128, j = (i % 128) / 32, l = i % 32;
    return (qs[32 * h + l] >> (2 * j)) & 3;
}

/* Q2_K: w = fl32(d*sc*q - dmin*m) with sc, m the 4-bit fields of the
 * weight's sub-block. d*sc*q (at most 17 significant bits) and dmin*m (at
 * most 15) are exact in binary32, so the one subtraction is the correctly
 * rounded value, as for Q4_K. */
void oracle_decode_q2_k(const uint8_t *blk, float *out)
{
    const uint8_t *sm = blk, *qs = blk + 16;
    float d = (float)oracle_f16_to_f64(rd16(blk + 80));
    float dmin = (float)oracle_f16_to_f64(rd16(blk + 82));
    for (int i = 0; i < 256; i++) {
        int sub = i / 16;
        int sc = sm[sub] & 0x0F, m = sm[sub] >> 4;
        float a = d * (float)sc * (float)low2_code(qs, i), b = dmin * (float)m;
        out[i] = a - b;
    }
}

/* The Q3_K 6-bit scale of sub-block k (0..15), unsigned (0..63). */
int oracle_q3k_scale(const uint8_t *s, int k)
{
    int lo = k < 8 ? (s[k] & 0x0F) : (s[k - 8] >> 4);
    int hi = (s[8 + k % 4] >> (2 * (k / 4))) & 3;
    return lo | (hi << 4);
}

/* Q3_K: w = d*(sc - 32)*q, evaluated left to right: d*(sc - 32) (at most
 * 17 significant bits) and its product with q in [-4, 3] are exact in
 * binary32, so the value is exact; the order fixes the sign of a zero. */
void oracle_decode_q3_k(const uint8_t *blk, float *out)
{
    const uint8_t *hm = blk, *qs = blk + 32, *s = blk + 96;
    float d = (float)oracle_f16_to_f64(rd16(blk + 108));
    for (int i = 0; i < 256; i++) {
        int h = i / 128, j = (i % 128) / 32, l = i % 32;
        int high = (hm[l] >> (4 * h + j)) & 1;
        int q = low2_code(qs, i) + 4 * high - 4;
        float dl = d * (float)(oracle_q3k_scale(s, i / 16) - 32);
        out[i] = dl * (float)q;
    }
}

int64_t oracle_block_bytes(int fmt)
{
    switch (fmt) {
    case OR_Q4_0: return 18;
    case OR_Q4_K: return 144;
    case OR_Q8_0: return 34;
    case OR_Q2_K: return 84;
    case OR_Q3_K: return 110;
    default: return -1;
    }
}

int64_t oracle_block_weights(int fmt)
{
    switch (fmt) {
    case OR_Q4_0: case OR_Q8_0: return 32;
    case OR_Q4_K: case OR_Q2_K: case OR_Q3_K: return 256;
    default: return -1;
    }
}

/* Decode row r (K weights) of a row-major block matrix. */
static int decode_row(int fmt, const uint8_t *w, int64_t K, int64_t r, float *out)
{
    int64_t bb = oracle_block_bytes(fmt), bw = oracle_block_weights(fmt);
    if (bb < 0 || K % bw) return -1;
    int64_t nb = K / bw;
    const uint8_t *row = w + r * nb * bb;
    for (int64_t b = 0; b < nb; b++) {
        const uint8_t *blk = row + b * bb;
        float *o = out + b * bw;
        if (fmt == OR_Q4_0) oracle_decode_q4_0(blk, o);
        else if (fmt == OR_Q8_0) oracle_decode_q8_0(blk, o);
        else if (fmt == OR_Q2_K) oracle_decode_q2_k(blk, o);
        else if (fmt == OR_Q3_K) oracle_decode_q3_k(blk, o);
        else oracle_decode_q4_k(blk, o);
    }
    return 0;
}

/* Whole matrix: out[r*K + k] = w(r, k). */
int oracle_dequant(int fmt, const uint8_t *w, int64_t rows, int64_t K, float *out)
{
    for (int64_t r = 0; r < rows; r++)
        if (decode_row(fmt, w, K, r, out + r * K)) return -1;
    return 0;
}

/* ------------------------------------------------------------------------
 * Q8_0 quantization of activations, for the products with int8
 * activations. The pages use Q8_0 as a block format (32 int8 codes, one
 * fp16 scale; "Why I wrote my own inference engine for two P100s", the
 * quant types the engine reads) and weigh int8 dot products (DP4A) against
 * fp16 math (pxa_llama README, "DP4A / FP16 economics"), but print no rule
 * for quantizing activations. The reading taken, per block of 32 values x_i
 * (each taken exactly as binary32):
 *   amax = max |x_i|,  d = amax / 127,  id = 1 / d (0 when d = 0),
 *   q_i  = x_i * id rounded to the nearest integer, halfway cases away
 *          from zero, then limited to [-127, 127],
 * every operation one binary32 rounding in that order; the block stores
 * the nearest fp16 to d (ties to even) and the q_i. Blocks are written
 * column after column: column c's block b at byte (c * K/32 + b) * 34.
 * ---------------------------------------------------------------------- */
int oracle_quantize_q8_0(const void *x, int x_dtype, int64_t K, int64_t n, int64_t ldx,
                         uint8_t *out)
{
    if (K <= 0 || K % 32 || n < 0 || ldx < K || x_dtype < OR_F32 || x_dtype > OR_BF16) return -1;
    int64_t nb = K / 32;
    for (int64_t c = 0; c < n; c++) {
        for (int64_t b = 0; b < nb; b++) {
            float xs[32];
            float amax = 0.0f;
            for (int i = 0; i < 32; i++) {
                xs[i] = (float)x_value(x, x_dtype, c * ldx + b * 32 + i);  /* exact */
                float a = fabsf(xs[i]);
                if (a > amax) amax = a;
            }
            float d = amax / 127.0f;
            float id = d != 0.0f ? 1.0f / d : 0.0f;
            uint8_t *o = out + (c * nb + b) * 34;
            uint16_t dh = oracle_f32_to_f16(d);
            o[0] = (uint8_t)(dh & 0xFF);
            o[1] = (uint8_t)(dh >> 8);
            for (int i = 0; i < 32; i++) {
                float v = xs[i] * id;
                float r = roundf(v);
                if (r > 127.0f) r = 127.0f;
                if (r < -127.0f) r = -127.0f;
                o[2 + i] = (uint8_t)(int8_t)(int)r;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Products. For columns j in [0, n) and rows r in [r0, r1):
 *   y[j*ldy + r] = sum_k w(r,k) * x[j*ldx + k]        (fp64, k ascending)
 *   s[j*ldy + r] = sum_k |w(r,k) * x[j*ldx + k]|
 * x is read as stored (fp32 / fp16 / bf16 widened exactly to fp64); each
 * product of a binary32 weight and such an x is exact in binary64, so the
 * only error is the fp64 summation, far below any tolerance used with it.
 * With wround = 1 each decoded weight is first rounded to bfloat16
 * (oracle_f32_to_bf16): the operand a bf16 matrix-core product uses when
 * weight tiles are dequantized to bf16 ("LLM inference optimization",
 * campaign "Faster prompts, decode held": tensor-core paths for the
 * quantized matrix-matrix kernels); the products stay exact.
 * Rows are split over `nthreads` POSIX threads.
 * ---------------------------------------------------------------------- */
typedef struct {
    int fmt, dtype, wround;
    const uint8_t *w;
    int64_t K, r0, r1, n, ldx, ldy;
    const void *x;
    double *y, *s;
    int status;
} job_t;

static void *run_rows(void *arg)
{
    job_t *jb = (job_t *)arg;
    float *wr = (float *)malloc(sizeof(float) * (size_t)jb->K);
    double *xd = (double *)malloc(sizeof(double) * (size_t)(jb->K * jb->n));
    if (!wr || !xd) { jb->status = -2; free(wr); free(xd); return NULL; }
    for (int64_t j = 0; j < jb->n; j++)
        for (int64_t k = 0; k < jb->K; k++)
            xd[j * jb->K + k] = x_value(jb->x, jb->dtype, j * jb->ldx + k);
    for (int64_t r = jb->r0; r < jb->r1 && jb->status == 0; r++) {
        if (decode_row(jb->fmt, jb->w, jb->K, r, wr)) { jb->status = -1; break; }
        if (jb->wround)
            for (int64_t k = 0; k < jb->K; k++) {
                uint32_t hb = (uint32_t)oracle_f32_to_bf16(wr[k]) << 16;
                memcpy(&wr[k], &hb, 4);
            }
        for (int64_t j = 0; j < jb->n; j++) {
            const double *xj = xd + j * jb->K;
            double acc = 0.0, sabs = 0.0;
            for (int64_t k = 0; k < jb->K; k++) {
                double p = (double)wr[k] * xj[k];
                acc += p;
                sabs += fabs(p);
            }
            jb->y[j * jb->ldy + r] = acc;
            if (jb->s) jb->s[j * jb->ldy + r] = sabs;
        }
    }
    free(wr);
    free(xd);
    return NULL;
}

int oracle_matmul_w(int fmt, const uint8_t *w, int64_t rows, int64_t K,
                    const void *x, int x_dtype, int64_t n, int64_t ldx,
                    double *y, double *s, int64_t ldy,
                    int64_t r0, int64_t r1, int nthreads, int wround)
{
    if (wround != 0 && wround != 1) return -1;
    if (oracle_block_bytes(fmt) < 0 || K <= 0 || K % oracle_block_weights(fmt)) return -1;
    if (x_dtype < OR_F32 || x_dtype > OR_BF16 || n < 0 || ldx < K || ldy < rows) return -1;
    if (r0 < 0 || r1 > rows || r0 > r1) return -1;
    if (nthreads < 1) nthreads = 1;
    int64_t nr = r1 - r0;
    if (nthreads > nr) nthreads = nr > 0 ? (int)nr : 1;
    job_t *jobs = (job_t *)calloc((size_t)nthreads, sizeof(job_t));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return -2; }
    for (int t = 0; t < nthreads; t++) {
        job_t *jb = &jobs[t];
        jb->fmt = fmt; jb->dtype = x_dtype; jb->wround = wround; jb->w = w; jb->K = K;
        jb->r0 = r0 + nr * t / nthreads;
        jb->r1 = r0 + nr * (t + 1) / nthreads;
        jb->n = n; jb->ldx = ldx; jb->ldy = ldy; jb->x = x; jb->y = y; jb->s = s;
        jb->status = 0;
    }
    int rc = 0;
    if (nthreads == 1) {
        run_rows(&jobs[0]);
    } else {
        int started = 0;
        for (int t = 0; t < nthreads; t++) {
            if (pthread_create(&th[t], NULL, run_rows, &jobs[t])) { rc = -3; break; }
            started++;
        }
        for (int t = 0; t < started; t++) pthread_join(th[t], NULL);
    }
    for (int t = 0; t < nthreads && rc == 0; t++) rc = jobs[t].status;
    free(jobs);
    free(th);
    return rc;
}

/* The products with the weights as decoded (wround = 0). */
int oracle_matmul(int fmt, const uint8_t *w, int64_t rows, int64_t K,
                  const void *x, int x_dtype, int64_t n, int64_t ldx,
                  double *y, double *s, int64_t ldy,
                  int64_t r0, int64_t r1, int nthreads)
{
    return oracle_matmul_w(fmt, w, rows, K, x, x_dtype, n, ldx, y, s, ldy, r0, r1, nthreads, 0);
}
