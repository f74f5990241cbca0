/*
 * oracle.c -- plain, slow CPU oracle for the Hadamard-rotated W4A4 Q4_0 matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may load, link or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no source, header, table or constant
 * generator with the HIP library; it is built by gcc with
 * -ffp-contract=off so every floating-point operation below is one IEEE
 * operation in the order written.
 *
 * What it follows (1bit-MONSTER engine documentation, page "The lean option:
 * ROCmFP4, ROCmI4 and Hadamard Q4_0", section "Hadamard-rotated Q4_0: W4A4
 * prompt processing"):
 *   - weights are plain Q4_0 blocks of 32, one fp16 scale, and a code q
 *     stands for q - 8;
 *   - the weights are rotated once by a 32-point Walsh-Hadamard transform per
 *     32-element block along K, and the activations are rotated by the same
 *     transform at run time, so x.w = (Hx).(Hw) in exact arithmetic;
 *   - at run time it is the activations that get rounded to 4 bits (the
 *     weights are 4-bit already); the 4-bit weight codes and 4-bit
 *     activation codes are multiplied as integers.
 * Section "MoE: W4A4 on the experts" of the same page: the expert matmuls
 * (MUL_MAT_ID) take the same path.
 *
 * Readings of points the page leaves open (each is also listed in the design
 * notes of the repository):
 *   R1  H is the Sylvester-ordered Hadamard matrix H[i][j] = (-1)^popcount(i&j);
 *       the normalised transform is H/sqrt(32).
 *   R2  Weight rotation (offline): w'_t = fp32( (sum_j H[t][j] w_j) * c64 ),
 *       the sum taken in fp64 in ascending j, c64 = fp64(1/sqrt(32)).
 *   R3  Q4_0 quantisation of the rotated weights: the usual rule -- mx is the
 *       element of largest magnitude (first on ties, sign kept), d = mx/-8,
 *       id = 1/d (0 if d == 0), q = min(15, trunc(w*id + 8.5)), d stored
 *       as fp16 rounded to nearest even.  All fp32.
 *   R4  Activation rotation: unnormalised fast Walsh-Hadamard butterflies in
 *       fp32, stages h = 1, 2, 4, 8, 16, (a, b) -> (a + b, a - b).
 *   R5  Activation quantisation: symmetric int4 in [-7, 7] per block,
 *       d = amax/7, id = 1/d, q = clamp(round_half_away(v*id), -7, 7),
 *       stored scale s = d * c32 (the 1/sqrt(32) normalisation folded into
 *       the scale), c32 = fp32(1/sqrt(32)).  A block whose d is below
 *       FLT_MIN (zero or subnormal) gets codes 0 and s = 0.
 *   R6  Output: y[m][n] = sum_b dw[n][b] * s[m][b] * S[m][n][b], where
 *       S = sum_t (qw - 8) * qa is an exact integer; every term is formed and
 *       summed in fp64 and the total is rounded once to fp32.
 *   R7  MUL_MAT_ID: output row (t, j) uses expert ids[t][j] and activation
 *       row t (one activation row per token) or t*top_k + j (one per slot);
 *       an id outside [0, n_expert) gives a row of zeros.
 *   R8  W4A8-H32, the page's exact int8 path for a rotated file (section
 *       "Hadamard-rotated Q4_0: W4A4 prompt processing": the rotated file
 *       can run on the exact int8 path instead of W4A4): the activations are
 *       rotated as in R4 and rounded to 8 bits per block, d = amax/127,
 *       id = 1/d, q = clamp(round_half_away(v*id), -127, 127), s = d * c32,
 *       zero blocks as in R5; the output is R6 with these codes.  Codes are
 *       stored one signed byte per element, [m][k].
 *   R9  Unrotated W4A4, the ablation of section "MoE: W4A4 on the experts"
 *       (the same W4A4 without the rotation costs about twice the accuracy):
 *       the weights are plain Q4_0 of the unrotated weights (R3 applied to w
 *       itself), the activations are quantised per block as in R5 but with
 *       no rotation and no normalisation: v = x, d = amax/7, id = 1/d,
 *       q = clamp(round_half_away(v*id), -7, 7), s = d, zero blocks as in
 *       R5; the output is R6 with these codes and scales.
 *   R10 Rotated W4A16, the page's route where the rotated file runs with the
 *       activations rotated but not rounded to 4 bits (section
 *       "Hadamard-rotated Q4_0: W4A4 prompt processing"; no rule printed):
 *       activations x16_t = fp16( fl(v_t * c32) ) with v the R4 butterflies
 *       of the block (fp16 round to nearest even); weights dequantised as
 *       w16_t = fp16( fl(dw * (q_t - 8)) ) with dw = fp32(fp16 d) (the fp32
 *       product is exact; one rounding to fp16); output y[m][n] = sum over k
 *       of (double)w16 * (double)x16 in fp64, rounded once to fp32.
 *
 * Byte layouts:
 *   Q4_0 block (18 bytes): fp16 d (little endian), then 16 bytes; byte j holds
 *   element j in its low nibble and element j+16 in its high nibble, as codes
 *   0..15.  Rows of a weight matrix [n][k] are n consecutive runs of k/32
 *   blocks.
 *   Activation codes: [m][k/2] bytes in the same nibble order, each nibble a
 *   two's-complement int4.  Activation scales: [m][k/32] fp32.
 */
#include <math.h>
#include <float.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define QK 32

/* Run fn(ctx, r0, r1) over [0, n) split into contiguous row ranges, one per
 * thread.  Rows are independent, so the split changes no arithmetic. */
typedef void (*row_range_fn)(void *ctx, int64_t r0, int64_t r1);
typedef struct {
    row_range_fn fn;
    void *ctx;
    int64_t r0, r1;
} row_range_job;

static void *row_range_worker(void *p)
{
    row_range_job *j = (row_range_job *)p;
    j->fn(j->ctx, j->r0, j->r1);
    return NULL;
}

static void parallel_rows(int64_t n, int nthreads, row_range_fn fn, void *ctx)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > n)
        nthreads = (int)(n > 0 ? n : 1);
    if (nthreads == 1) {
        fn(ctx, 0, n);
        return;
    }
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    row_range_job *jobs = (row_range_job *)calloc((size_t)nthreads, sizeof(row_range_job));
    for (int t = 0; t < nthreads; t++) {
        jobs[t] = (row_range_job){fn, ctx, n * t / nthreads, n * (t + 1) / nthreads};
        pthread_create(&th[t], NULL, row_range_worker, &jobs[t]);
    }
    for (int t = 0; t < nthreads; t++)
        pthread_join(th[t], NULL);
    free(th);
    free(jobs);
}

/* ------------------------------------------------------------------ */
/* Hadamard matrix (R1)                                                */
/* ------------------------------------------------------------------ */

static int parity_of(unsigned v)
{
    int p = 0;
    while (v) {
        p ^= (int)(v & 1u);
        v >>= 1;
    }
    return p;
}

/* H[i*32 + j] = (-1)^popcount(i & j). */
void oracle_h32(int32_t *H)
{
    for (int i = 0; i < QK; i++)
        for (int j = 0; j < QK; j++)
            H[i * QK + j] = parity_of((unsigned)(i & j)) ? -1 : 1;
}

/* The two normalisation constants, correctly rounded. */
double oracle_c64(void) { return sqrt(2.0) / 8.0; } /* = 1/sqrt(32), one rounding */
float oracle_c32(void) { return (float)(sqrt(2.0) / 8.0); }

/* ------------------------------------------------------------------ */
/* fp16 <-> fp32 conversion, written out from the IEEE binary16 layout */
/* ------------------------------------------------------------------ */

float oracle_half_to_float(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int exp = (h >> 10) & 0x1f;
    int man = h & 0x3ff;
    float v;
    if (exp == 0)
        v = ldexpf((float)man, -24); /* zero or subnormal: man * 2^-24 */
    else if (exp == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexpf((float)(man + 1024), exp - 25); /* 1.man * 2^(exp-15) */
    return sign ? -v : v;
}

/* Round an fp32 value to binary16, ties to even. */
uint16_t oracle_float_to_half(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    float a = fabsf(f);
    if (isnan(f))
        return sign | 0x7e00u;
    if (a >= 65520.0f) /* rounds to infinity */
        return sign | 0x7c00u;
    if (a < ldexpf(1.0f, -14)) {
        /* subnormal range: value = n * 2^-24, n = round_even(a * 2^24) */
        float scaled = a * 16777216.0f; /* exact: power-of-two scaling */
        float n = nearbyintf(scaled);   /* default rounding mode: ties to even */
        return sign | (uint16_t)n;      /* n == 1024 becomes the smallest normal */
    }
    int e;
    float fr = frexpf(a, &e);          /* a = fr * 2^e, fr in [0.5, 1) */
    float sig = ldexpf(fr, 11);         /* in [1024, 2048) */
    float n = nearbyintf(sig);          /* ties to even */
    int exp_field = e - 1 + 15;
    if (n == 2048.0f) {
        n = 1024.0f;
        exp_field += 1;
    }
    if (exp_field >= 31)
        return sign | 0x7c00u;
    return sign | (uint16_t)(exp_field << 10) | (uint16_t)((int)n - 1024);
}

/* ------------------------------------------------------------------ */
/* Offline weight preparation (R2, R3)                                 */
/* ------------------------------------------------------------------ */

/* wr[r][32b + t] = fp32( (sum_j H[t][j] * w[r][32b + j]) * c64 ), sum in fp64. */
typedef struct {
    const float *w;
    int64_t k;
    float *wr;
} rotate_ctx;

static void rotate_rows(void *p, int64_t r0, int64_t r1)
{
    rotate_ctx *c = (rotate_ctx *)p;
    int32_t H[QK * QK];
    oracle_h32(H);
    const double c64 = oracle_c64();
    for (int64_t r = r0; r < r1; r++) {
        for (int64_t b = 0; b < c->k / QK; b++) {
            const float *src = c->w + r * c->k + b * QK;
            float *dst = c->wr + r * c->k + b * QK;
            for (int t = 0; t < QK; t++) {
                double u = 0.0;
                for (int j = 0; j < QK; j++)
                    u += (double)H[t * QK + j] * (double)src[j];
                dst[t] = (float)(u * c64);
            }
        }
    }
}

void oracle_rotate_weights(const float *w, int64_t n, int64_t k, float *wr, int nthreads)
{
    rotate_ctx c = {w, k, wr};
    parallel_rows(n, nthreads, rotate_rows, &c);
}

/* Q4_0-quantise rows of fp32 values (R3).  q4 gets n * (k/32) blocks of 18 B. */
typedef struct {
    const float *wr;
    int64_t k;
    uint8_t *q4;
} q4_ctx;

static void q4_rows(void *p, int64_t r0, int64_t r1)
{
    q4_ctx *c = (q4_ctx *)p;
    const float *wr = c->wr;
    const int64_t k = c->k;
    uint8_t *q4 = c->q4;
    for (int64_t r = r0; r < r1; r++) {
        for (int64_t b = 0; b < k / QK; b++) {
            const float *x = wr + r * k + b * QK;
            uint8_t *blk = q4 + (r * (k / QK) + b) * 18;
            float amax = 0.0f, mx = 0.0f;
            for (int t = 0; t < QK; t++) {
                if (fabsf(x[t]) > amax) {
                    amax = fabsf(x[t]);
                    mx = x[t];
                }
            }
            float d = mx / -8.0f;
            float id = (d != 0.0f) ? 1.0f / d : 0.0f;
            uint16_t dh = oracle_float_to_half(d);
            blk[0] = (uint8_t)(dh & 0xff);
            blk[1] = (uint8_t)(dh >> 8);
            for (int j = 0; j < QK / 2; j++) {
                float x0 = x[j] * id;
                float x1 = x[j + 16] * id;
                int q0 = (int)(x0 + 8.5f); /* non-negative: truncation is floor */
                int q1 = (int)(x1 + 8.5f);
                if (q0 > 15) q0 = 15;
                if (q1 > 15) q1 = 15;
                blk[2 + j] = (uint8_t)(q0 | (q1 << 4));
            }
        }
    }
}

void oracle_q4_0_quantize(const float *wr, int64_t n, int64_t k, uint8_t *q4, int nthreads)
{
    q4_ctx c = {wr, k, q4};
    parallel_rows(n, nthreads, q4_rows, &c);
}

/* Code t (0..15) of a Q4_0 block, and its value d * (q - 8). */
static int q4_code(const uint8_t *blk, int t)
{
    uint8_t byte = blk[2 + (t & 15)];
    return t < 16 ? (byte & 0x0f) : (byte >> 4);
}

static float q4_scale(const uint8_t *blk)
{
    return oracle_half_to_float((uint16_t)(blk[0] | (blk[1] << 8)));
}

/* Dequantise Q4_0 rows: out = d * (q - 8). */
void oracle_q4_0_dequantize(const uint8_t *q4, int64_t n, int64_t k, float *out)
{
    for (int64_t r = 0; r < n; r++)
        for (int64_t b = 0; b < k / QK; b++) {
            const uint8_t *blk = q4 + (r * (k / QK) + b) * 18;
            float d = q4_scale(blk);
            for (int t = 0; t < QK; t++)
                out[r * k + b * QK + t] = d * (float)(q4_code(blk, t) - 8);
        }
}

/* ------------------------------------------------------------------ */
/* Activation rotation and quantisation (R4, R5)                       */
/* ------------------------------------------------------------------ */

/* In-place unnormalised FWHT of 32 fp32 values, stages h = 1, 2, 4, 8, 16. */
void oracle_fwht32_f32(float *v)
{
    for (int h = 1; h < QK; h <<= 1) {
        for (int i = 0; i < QK; i++) {
            if (i & h)
                continue;
            float a = v[i], b = v[i + h];
            v[i] = a + b;
            v[i + h] = a - b;
        }
    }
}

/* round half away from zero, written out */
static float round_half_away(float x)
{
    float t = truncf(x);
    float frac = fabsf(x - t); /* exact for |x| < 2^23 */
    if (frac >= 0.5f)
        t += (x < 0.0f) ? -1.0f : 1.0f;
    return t;
}

/* Quantise one rotated block to codes q[32] in [-qmax, qmax] (qmax = 7 for
 * R5, 127 for R8); returns the stored scale. */
static float quantize_block(const float *v, int8_t *q, int qmax)
{
    float amax = 0.0f;
    for (int t = 0; t < QK; t++)
        if (fabsf(v[t]) > amax)
            amax = fabsf(v[t]);
    const float fq = (float)qmax;
    float d = amax / fq;
    if (!(d >= FLT_MIN)) {
        for (int t = 0; t < QK; t++)
            q[t] = 0;
        return 0.0f;
    }
    float id = 1.0f / d;
    for (int t = 0; t < QK; t++) {
        float r = round_half_away(v[t] * id);
        if (r > fq) r = fq;
        if (r < -fq) r = -fq;
        q[t] = (int8_t)r;
    }
    return d * oracle_c32();
}

/* Block b of row r of x, as fp32. */
static void load_block(const void *x, int dtype, int64_t ldx, int64_t r, int64_t b, float *v)
{
    for (int t = 0; t < QK; t++) {
        int64_t idx = r * ldx + b * QK + t;
        v[t] = dtype == 0 ? ((const float *)x)[idx] : oracle_half_to_float(((const uint16_t *)x)[idx]);
    }
}

typedef struct {
    const void *x;
    int dtype;
    int64_t k, ldx;
    uint8_t *codes;
    float *scales;
} act_ctx;

static void act_rows(void *p, int64_t r0, int64_t r1)
{
    act_ctx *c = (act_ctx *)p;
    const int64_t k = c->k, nb = k / QK;
    for (int64_t r = r0; r < r1; r++) {
        for (int64_t b = 0; b < nb; b++) {
            float v[QK];
            load_block(c->x, c->dtype, c->ldx, r, b, v);
            oracle_fwht32_f32(v);
            int8_t q[QK];
            c->scales[r * nb + b] = quantize_block(v, q, 7);
            uint8_t *dst = c->codes + r * (k / 2) + b * 16;
            for (int j = 0; j < 16; j++)
                dst[j] = (uint8_t)(((uint8_t)q[j] & 0x0f) | (((uint8_t)q[j + 16] & 0x0f) << 4));
        }
    }
}

/*
 * x: [m][ldx] elements, fp32 (dtype 0) or fp16 bits (dtype 1).
 * codes: [m][k/2] bytes, scales: [m][k/32].
 */
void oracle_rotate_quantize_act(const void *x, int dtype, int64_t m, int64_t k, int64_t ldx,
                                uint8_t *codes, float *scales, int nthreads)
{
    act_ctx c = {x, dtype, k, ldx, codes, scales};
    parallel_rows(m, nthreads, act_rows, &c);
}

/* R9: one unrotated block to codes q[32] in [-7, 7]; returns s = d. */
static float quantize_block_plain(const float *v, int8_t *q)
{
    float amax = 0.0f;
    for (int t = 0; t < QK; t++)
        if (fabsf(v[t]) > amax)
            amax = fabsf(v[t]);
    float d = amax / 7.0f;
    if (!(d >= FLT_MIN)) {
        for (int t = 0; t < QK; t++)
            q[t] = 0;
        return 0.0f;
    }
    float id = 1.0f / d;
    for (int t = 0; t < QK; t++) {
        float r = round_half_away(v[t] * id);
        if (r > 7.0f) r = 7.0f;
        if (r < -7.0f) r = -7.0f;
        q[t] = (int8_t)r;
    }
    return d;
}

static void act_plain_rows(void *p, int64_t r0, int64_t r1)
{
    act_ctx *c = (act_ctx *)p;
    const int64_t k = c->k, nb = k / QK;
    for (int64_t r = r0; r < r1; r++) {
        for (int64_t b = 0; b < nb; b++) {
            float v[QK];
            load_block(c->x, c->dtype, c->ldx, r, b, v);
            int8_t q[QK];
            c->scales[r * nb + b] = quantize_block_plain(v, q);
            uint8_t *dst = c->codes + r * (k / 2) + b * 16;
            for (int j = 0; j < 16; j++)
                dst[j] = (uint8_t)(((uint8_t)q[j] & 0x0f) | (((uint8_t)q[j + 16] & 0x0f) << 4));
        }
    }
}

/* R9 activations: as oracle_rotate_quantize_act without the rotation. */
void oracle_quantize_act_plain(const void *x, int dtype, int64_t m, int64_t k, int64_t ldx,
                               uint8_t *codes, float *scales, int nthreads)
{
    act_ctx c = {x, dtype, k, ldx, codes, scales};
    parallel_rows(m, nthreads, act_plain_rows, &c);
}

/* R10 activations: x fp32/fp16 [m][ldx] -> rotated fp16 bits [m][k]. */
typedef struct {
    const void *x;
    int dtype;
    int64_t k, ldx;
    uint16_t *xr;
} rot16_ctx;

static void rot16_rows(void *p, int64_t r0, int64_t r1)
{
    rot16_ctx *c = (rot16_ctx *)p;
    const int64_t k = c->k, nb = k / QK;
    const float cc = oracle_c32();
    for (int64_t r = r0; r < r1; r++) {
        for (int64_t b = 0; b < nb; b++) {
            float v[QK];
            load_block(c->x, c->dtype, c->ldx, r, b, v);
            oracle_fwht32_f32(v);
            for (int t = 0; t < QK; t++)
                c->xr[r * k + b * QK + t] = oracle_float_to_half(v[t] * cc);
        }
    }
}

void oracle_rotate_act16(const void *x, int dtype, int64_t m, int64_t k, int64_t ldx, uint16_t *xr,
                         int nthreads)
{
    rot16_ctx c = {x, dtype, k, ldx, xr};
    parallel_rows(m, nthreads, rot16_rows, &c);
}

/* R10 weights: Q4_0 [n][k/32][18] -> dequantised fp16 bits [n][k]. */
void oracle_dequantize_w16(const uint8_t *q4, int64_t n, int64_t k, uint16_t *w16)
{
    const int64_t nb = k / QK;
    for (int64_t r = 0; r < n; r++)
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *blk = q4 + (r * nb + b) * 18;
            const float d = q4_scale(blk);
            for (int t = 0; t < QK; t++)
                w16[r * k + b * QK + t] = oracle_float_to_half(d * (float)(q4_code(blk, t) - 8));
        }
}

/* R10 output: y[m][n] = fp32( sum_k (double)w16 * (double)x16 ), fp64 sums. */
typedef struct {
    const uint16_t *w16, *x16;
    int64_t n, k;
    float *y;
    int64_t ldy;
} gemm16_ctx;

static void gemm16_rows(void *p, int64_t r0, int64_t r1)
{
    gemm16_ctx *c = (gemm16_ctx *)p;
    for (int64_t r = r0; r < r1; r++)
        for (int64_t j = 0; j < c->n; j++) {
            double acc = 0.0;
            for (int64_t t = 0; t < c->k; t++)
                acc += (double)oracle_half_to_float(c->w16[j * c->k + t]) *
                       (double)oracle_half_to_float(c->x16[r * c->k + t]);
            c->y[r * c->ldy + j] = (float)acc;
        }
}

void oracle_gemm_w16(const uint16_t *w16, const uint16_t *x16, int64_t m, int64_t n, int64_t k, float *y,
                     int64_t ldy, int nthreads)
{
    gemm16_ctx c = {w16, x16, n, k, y, ldy};
    parallel_rows(m, nthreads, gemm16_rows, &c);
}

static void act8_rows(void *p, int64_t r0, int64_t r1)
{
    act_ctx *c = (act_ctx *)p;
    const int64_t k = c->k, nb = k / QK;
    for (int64_t r = r0; r < r1; r++)
        for (int64_t b = 0; b < nb; b++) {
            float v[QK];
            load_block(c->x, c->dtype, c->ldx, r, b, v);
            oracle_fwht32_f32(v);
            c->scales[r * nb + b] = quantize_block(v, (int8_t *)(c->codes + r * k + b * QK), 127);
        }
}

/* R8: codes [m][k] signed bytes, scales [m][k/32]. */
void oracle_rotate_quantize_act8(const void *x, int dtype, int64_t m, int64_t k, int64_t ldx,
                                 int8_t *codes, float *scales, int nthreads)
{
    act_ctx c = {x, dtype, k, ldx, (uint8_t *)codes, scales};
    parallel_rows(m, nthreads, act8_rows, &c);
}

/* Signed int4 code t (-8..7) of an activation block. */
static int act_code(const uint8_t *blk16, int t)
{
    uint8_t byte = blk16[t & 15];
    int nib = t < 16 ? (byte & 0x0f) : (byte >> 4);
    return nib >= 8 ? nib - 16 : nib;
}

/* ------------------------------------------------------------------ */
/* Integer block dots and the fp64 output (R6)                         */
/* ------------------------------------------------------------------ */

/* S[(i*n + j)*nb + b] = sum_t (qw - 8) * qa, exact int32. */
void oracle_block_sums(const uint8_t *q4, const uint8_t *codes, int64_t m, int64_t n, int64_t k,
                       int32_t *S)
{
    const int64_t nb = k / QK;
    for (int64_t i = 0; i < m; i++)
        for (int64_t j = 0; j < n; j++)
            for (int64_t b = 0; b < nb; b++) {
                const uint8_t *wb = q4 + (j * nb + b) * 18;
                const uint8_t *ab = codes + i * (k / 2) + b * 16;
                int32_t s = 0;
                for (int t = 0; t < QK; t++)
                    s += (q4_code(wb, t) - 8) * act_code(ab, t);
                S[(i * n + j) * nb + b] = s;
            }
}

/* R8 block dots: S[(i*n + j)*nb + b] = sum_t (qw - 8) * qa with int8 codes. */
void oracle_block_sums_a8(const uint8_t *q4, const int8_t *codes, int64_t m, int64_t n, int64_t k,
                          int32_t *S)
{
    const int64_t nb = k / QK;
    for (int64_t i = 0; i < m; i++)
        for (int64_t j = 0; j < n; j++)
            for (int64_t b = 0; b < nb; b++) {
                const uint8_t *wb = q4 + (j * nb + b) * 18;
                const int8_t *ab = codes + i * k + b * QK;
                int32_t s = 0;
                for (int t = 0; t < QK; t++)
                    s += (q4_code(wb, t) - 8) * ab[t];
                S[(i * n + j) * nb + b] = s;
            }
}

/* One output element: fp64 sum of exact per-block terms, rounded once. */
static float gemm_elem(const uint8_t *wrow, const uint8_t *arow, const float *srow, int64_t nb)
{
    double acc = 0.0;
    for (int64_t b = 0; b < nb; b++) {
        const uint8_t *wb = wrow + b * 18;
        const uint8_t *ab = arow + b * 16;
        int32_t s = 0;
        for (int t = 0; t < QK; t++)
            s += (q4_code(wb, t) - 8) * act_code(ab, t);
        acc += (double)q4_scale(wb) * (double)srow[b] * (double)s;
    }
    return (float)acc;
}

typedef struct {
    const uint8_t *q4;
    const uint8_t *codes;
    const float *scales;
    int64_t m, n, k;
    float *y;
    int64_t ldy;
    int64_t row_begin, row_end;
} gemm_job;

static void *gemm_worker(void *p)
{
    gemm_job *g = (gemm_job *)p;
    const int64_t nb = g->k / QK;
    for (int64_t i = g->row_begin; i < g->row_end; i++)
        for (int64_t j = 0; j < g->n; j++)
            g->y[i * g->ldy + j] =
                gemm_elem(g->q4 + j * nb * 18, g->codes + i * (g->k / 2), g->scales + i * nb, nb);
    return NULL;
}

/* y[m][ldy] = W4A4 product of activation codes/scales with Q4_0 weights [n][k]. */
void oracle_gemm(const uint8_t *q4, const uint8_t *codes, const float *scales, int64_t m,
                 int64_t n, int64_t k, float *y, int64_t ldy, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > m)
        nthreads = (int)(m > 0 ? m : 1);
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    gemm_job *jobs = (gemm_job *)calloc((size_t)nthreads, sizeof(gemm_job));
    for (int t = 0; t < nthreads; t++) {
        jobs[t] = (gemm_job){q4, codes, scales, m, n, k, y, ldy,
                             m * t / nthreads, m * (t + 1) / nthreads};
        pthread_create(&th[t], NULL, gemm_worker, &jobs[t]);
    }
    for (int t = 0; t < nthreads; t++)
        pthread_join(th[t], NULL);
    free(th);
    free(jobs);
}

/* R8 output: as oracle_gemm with int8 codes [m][k]. */
typedef struct {
    const uint8_t *q4;
    const int8_t *codes;
    const float *scales;
    int64_t n, k;
    float *y;
    int64_t ldy;
} gemm8_ctx;

static void gemm8_rows(void *p, int64_t r0, int64_t r1)
{
    gemm8_ctx *g = (gemm8_ctx *)p;
    const int64_t nb = g->k / QK;
    for (int64_t i = r0; i < r1; i++)
        for (int64_t j = 0; j < g->n; j++) {
            double acc = 0.0;
            for (int64_t b = 0; b < nb; b++) {
                const uint8_t *wb = g->q4 + (j * nb + b) * 18;
                const int8_t *ab = g->codes + i * g->k + b * QK;
                int32_t s = 0;
                for (int t = 0; t < QK; t++)
                    s += (q4_code(wb, t) - 8) * ab[t];
                acc += (double)q4_scale(wb) * (double)g->scales[i * nb + b] * (double)s;
            }
            g->y[i * g->ldy + j] = (float)acc;
        }
}

void oracle_gemm_a8(const uint8_t *q4, const int8_t *codes, const float *scales, int64_t m,
                    int64_t n, int64_t k, float *y, int64_t ldy, int nthreads)
{
    gemm8_ctx c = {q4, codes, scales, n, k, y, ldy};
    parallel_rows(m, nthreads, gemm8_rows, &c);
}

/* ------------------------------------------------------------------ */
/* MUL_MAT_ID (R7)                                                     */
/* ------------------------------------------------------------------ */

typedef struct {
    const uint8_t *q4;
    int64_t n_expert;
    const uint8_t *codes;
    const float *scales;
    int64_t act_rows_per_token;
    const int32_t *ids;
    int64_t n_tokens, top_k, n, k;
    float *y;
    int64_t tok_begin, tok_end;
} gemm_id_job;

static void *gemm_id_worker(void *p)
{
    gemm_id_job *g = (gemm_id_job *)p;
    const int64_t nb = g->k / QK;
    const int64_t expert_blocks = g->n * nb;
    for (int64_t t = g->tok_begin; t < g->tok_end; t++)
        for (int64_t s = 0; s < g->top_k; s++) {
            int32_t e = g->ids[t * g->top_k + s];
            float *yrow = g->y + (t * g->top_k + s) * g->n;
            if (e < 0 || e >= g->n_expert) {
                for (int64_t j = 0; j < g->n; j++)
                    yrow[j] = 0.0f;
                continue;
            }
            int64_t r = g->act_rows_per_token == 1 ? t : t * g->top_k + s;
            const uint8_t *w = g->q4 + (int64_t)e * expert_blocks * 18;
            for (int64_t j = 0; j < g->n; j++)
                yrow[j] = gemm_elem(w + j * nb * 18, g->codes + r * (g->k / 2),
                                    g->scales + r * nb, nb);
        }
    return NULL;
}

void oracle_gemm_id(const uint8_t *q4, int64_t n_expert, const uint8_t *codes,
                    const float *scales, int64_t act_rows_per_token, const int32_t *ids,
                    int64_t n_tokens, int64_t top_k, int64_t n, int64_t k, float *y,
                    int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > n_tokens)
        nthreads = (int)(n_tokens > 0 ? n_tokens : 1);
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    gemm_id_job *jobs = (gemm_id_job *)calloc((size_t)nthreads, sizeof(gemm_id_job));
    for (int t = 0; t < nthreads; t++) {
        jobs[t] = (gemm_id_job){q4, n_expert, codes, scales, act_rows_per_token, ids,
                                n_tokens, top_k, n, k, y,
                                n_tokens * t / nthreads, n_tokens * (t + 1) / nthreads};
        pthread_create(&th[t], NULL, gemm_id_worker, &jobs[t]);
    }
    for (int t = 0; t < nthreads; t++)
        pthread_join(th[t], NULL);
    free(th);
    free(jobs);
}
