/*
 * Plain scalar CPU oracle for the block-quantized matrix-vector product.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the bench's CPU
 * baseline leg use it.  It shares no code, header, table or constant with the
 * HIP library; the two meet only through the raw block bytes produced by the
 * seeded input generator.
 *
 * What it computes (the plain definition the fast path must reach):
 *   y[t][i] = sum_j Wdeq[i][j] * x[t][j]
 *   S[t][i] = sum_j |Wdeq[i][j] * x[t][j]|     (the per-element error scale)
 * with W stored one row per output ("A neuron is a dot product", section 1 of
 * "Running an LLM, then forgetting it"; the matmul of section 8.7.1.4 "Five
 * small functions" of dasLLAMA-00), every row decoded once and reused for all
 * tokens (the batched matmul of section 11 "Prefill and decode", same blog).
 * Arithmetic is IEEE binary64, summed in plain increasing column order.
 *
 * Block decoders, one per format:
 *   Q8_0  -- section 10 "Loading weights" of the llmoxide blog: 34 bytes,
 *            f16 scale d at offset 0, then 32 signed bytes; weight = d*q.
 *   Q4_0  -- the Go "llm" package README, Design points (18-byte blocks),
 *            with w = (q-8)*d for unsigned 4-bit q.  Field order (f16 d then
 *            16 code bytes) and nibble order (low nibble of byte l is column
 *            l, high nibble is column l+16) are readings, not printed facts.
 *   Q4_K  -- "Building llamini.cpp", section "What I reimplemented": 256
 *            weights, eight 32-element sub-blocks whose 6-bit (scale, min)
 *            pairs are packed in 12 bytes and unpacked by get_scale_min_k4;
 *            4.5 bits per weight (section 10 of the llmoxide blog) = 144 B.
 *            Reading: d, dmin (f16), scales[12], qs[128]; w = d*sc*q - dmin*m;
 *            qs[32c+l] holds sub-block 2c in its low nibble and 2c+1 in its
 *            high nibble.
 *   Q6_K  -- section 10 "Loading weights" of the llmoxide blog: a k-quant of
 *            256-weight super-blocks with their own scales at about 6.6 bits
 *            per weight; "Building llamini.cpp" (section "What I
 *            reimplemented") names it the second super-block format of a
 *            Q4_K_M file.  Reading (the GGUF layout of those files, not
 *            printed on the pages): 210 bytes = ql[128], qh[64], scales[16]
 *            (int8, one per 16 columns), d (f16); the 6-bit code of column
 *            c = 128h + 32j + l (h < 2, j < 4, l < 32) takes its low four bits
 *            from ql[64h + 32(j mod 2) + l] (low nibble for j < 2, high nibble
 *            for j >= 2) and its top two bits from bits 2j, 2j+1 of
 *            qh[32h + l]; w = d * scales[c / 16] * (q - 32).
 *   I8ROW -- minillm-cpp README, Quantization paragraph: symmetric per-channel
 *            int8 with one scale per output row; w = s_row * q.
 *
 * SwiGLU (section 2 of the llmoxide blog; section 8.7.1.6.3 of dasLLAMA-00):
 *   g = Wg x, u = Wu x, h_j = g_j / (1 + exp(-g_j)) * u_j, out = Wd h.
 *
 * RMSNorm (section 4 "Keeping the numbers in range" of the llmoxide blog; the
 * rmsnorm of dasLLAMA-00's "Five small functions"): the mean of the squares
 * over the row, scale = 1 / sqrt(mean + eps), out_j = x_j * scale * gamma_j.
 * The FFN block of the residual stream (section 7 "The block, and the
 * residual stream", same blog): out = x + FFN(rmsnorm(x) * gamma).
 *
 * Greedy sampling (dasLLAMA-00's most_likely; the Go "llm" package's Argmax,
 * first index on ties): start from index 0 and move to a later index only
 * when its logit is strictly greater.
 *
 * Q8_0 activations (the Go "llm" package's ExactGGML mode: activations are
 * quantised to Q8_0 before every quantised matrix product).  Reading: per
 * 32-element block, d = max|x| / 127, q = round(x * (1/d)) with halves away
 * from zero (q = 0 when d = 0), all in binary32; the block stores d rounded
 * to binary16 (nearest even, the package's F32ToF16), so the product sees
 * x replaced by f16(d) * q.  The oracle's product is then the plain one on
 * that representation, in binary64.
 *
 * Parity pins for every function live in tests/test_oracle_*.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_ERR_SHAPE -2
#define OR_ERR_FORMAT -4
#define OR_ERR_NOMEM -8

enum { OR_Q4_0 = 0, OR_Q8_0 = 1, OR_Q4_K = 2, OR_I8ROW = 3, OR_Q6_K = 4 };

/* IEEE 754 binary16 -> binary64, exact (the Go "llm" package documents its
 * F16ToF32 as exact).  Sign, 5-bit exponent biased by 15, 10-bit fraction;
 * exponent 0 is zero/subnormal (m * 2^-24), exponent 31 is Inf/NaN. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return sign ? -v : v;
}

static uint16_t rd_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* binary32 -> binary16 bits, round to nearest even (the Go "llm" package's
 * F32ToF16).  The magnitude is divided, exactly, by the binary16 spacing of
 * its binade (2^-24 below 2^-14) and rounded by nearbyint in the default
 * nearest-even mode; past the largest finite value (65504) it is infinite. */
uint16_t oracle_f32_to_f16(float f)
{
    const uint16_t sign = signbit(f) ? 0x8000 : 0;
    if (isnan(f))
        return sign | 0x7E00;
    double a = fabs((double)f);
    if (isinf(f))
        return sign | 0x7C00;
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);   /* a in [2^(e-1), 2^e) */
    int ue = e - 1;
    if (ue < -14)
        ue = -14;
    const double spacing = ldexp(1.0, ue - 10);
    const double r = nearbyint(a / spacing);
    const double v = r * spacing;
    if (v > 65504.0)
        return sign | 0x7C00;
    if (v < ldexp(1.0, -14))
        return sign | (uint16_t)r;   /* subnormal: v = r * 2^-24 */
    frexp(v, &e);
    ue = e - 1;
    const uint16_t frac = (uint16_t)(ldexp(v, 10 - ue) - 1024.0);
    return sign | (uint16_t)((ue + 15) << 10) | frac;
}

/* Q4_K scale/min unpack for sub-block j (0..7) from the 12-byte field q, as
 * the llamini.cpp post describes it: sub-blocks 0-3 keep their 6-bit scale and
 * min directly in bytes j and j+4; sub-blocks 4-7 take their low 4 bits from
 * byte j+4 and their top 2 bits from the spare high bits of bytes j-4 / j. */
void oracle_q4k_scale_min(int j, const uint8_t *q, int *sc, int *m)
{
    if (j < 4) {
        *sc = q[j] & 63;
        *m = q[j + 4] & 63;
    } else {
        *sc = (q[j + 4] & 0x0F) | ((q[j - 4] >> 6) << 4);
        *m = (q[j + 4] >> 4) | ((q[j] >> 6) << 4);
    }
}

/* Decode row `r` of a tensor into `out` (cols doubles, exact values). */
static void decode_row(int fmt, const uint8_t *raw, const float *row_scale, int64_t r, int64_t cols,
                       double *out)
{
    if (fmt == OR_Q8_0) {
        int64_t nb = cols / 32;
        const uint8_t *row = raw + r * nb * 34;
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *blk = row + b * 34;
            double d = oracle_f16_to_f64(rd_u16(blk));
            for (int l = 0; l < 32; l++) {
                int q = (int8_t)blk[2 + l];
                out[b * 32 + l] = d * (double)q;
            }
        }
    } else if (fmt == OR_Q4_0) {
        int64_t nb = cols / 32;
        const uint8_t *row = raw + r * nb * 18;
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *blk = row + b * 18;
            double d = oracle_f16_to_f64(rd_u16(blk));
            const uint8_t *qs = blk + 2;
            for (int l = 0; l < 16; l++) {
                int lo = qs[l] & 0x0F;
                int hi = qs[l] >> 4;
                out[b * 32 + l] = (double)(lo - 8) * d;
                out[b * 32 + 16 + l] = (double)(hi - 8) * d;
            }
        }
    } else if (fmt == OR_Q4_K) {
        int64_t nsb = cols / 256;
        const uint8_t *row = raw + r * nsb * 144;
        for (int64_t b = 0; b < nsb; b++) {
            const uint8_t *blk = row + b * 144;
            double d = oracle_f16_to_f64(rd_u16(blk));
            double dmin = oracle_f16_to_f64(rd_u16(blk + 2));
            const uint8_t *scales = blk + 4;
            const uint8_t *qs = blk + 16;
            for (int s = 0; s < 8; s++) {
                int sc, m;
                oracle_q4k_scale_min(s, scales, &sc, &m);
                const uint8_t *chunk = qs + 32 * (s / 2);
                for (int l = 0; l < 32; l++) {
                    int q = (s % 2 == 0) ? (chunk[l] & 0x0F) : (chunk[l] >> 4);
                    out[b * 256 + 32 * s + l] = d * (double)sc * (double)q - dmin * (double)m;
                }
            }
        }
    } else if (fmt == OR_Q6_K) {
        int64_t nsb = cols / 256;
        const uint8_t *row = raw + r * nsb * 210;
        for (int64_t b = 0; b < nsb; b++) {
            const uint8_t *blk = row + b * 210;
            const uint8_t *ql = blk;
            const uint8_t *qh = blk + 128;
            const int8_t *scales = (const int8_t *)(blk + 192);
            double d = oracle_f16_to_f64(rd_u16(blk + 208));
            for (int c = 0; c < 256; c++) {
                int half = c / 128, j = (c % 128) / 32, l = c % 32;
                int lo_byte = ql[64 * half + 32 * (j % 2) + l];
                int lo = (j < 2) ? (lo_byte & 0x0F) : (lo_byte >> 4);
                int hi = (qh[32 * half + l] >> (2 * j)) & 3;
                int q = lo | (hi << 4);
                out[b * 256 + c] = d * (double)scales[c / 16] * (double)(q - 32);
            }
        }
    } else { /* OR_I8ROW */
        const int8_t *row = (const int8_t *)raw + r * cols;
        double s = (double)row_scale[r];
        for (int64_t j = 0; j < cols; j++)
            out[j] = s * (double)row[j];
    }
}

static int check_shape(int fmt, int64_t rows, int64_t cols)
{
    if (fmt < OR_Q4_0 || fmt > OR_Q6_K)
        return OR_ERR_FORMAT;
    if (rows < 0 || cols < 0)
        return OR_ERR_SHAPE;
    if ((fmt == OR_Q4_0 || fmt == OR_Q8_0) && cols % 32)
        return OR_ERR_SHAPE;
    if ((fmt == OR_Q4_K || fmt == OR_Q6_K) && cols % 256)
        return OR_ERR_SHAPE;
    return OR_OK;
}

/* Dequantized weights rounded once (round-to-nearest-even) to binary32.
 * For Q8_0, Q4_0, Q4_K and Q6_K the binary64 value is exact and the cast is
 * the single rounding; for I8ROW likewise (s*q has at most 32 significant
 * bits). */
int oracle_dequant(int fmt, const void *raw, const float *row_scale, int64_t rows, int64_t cols,
                   float *w_out)
{
    int st = check_shape(fmt, rows, cols);
    if (st)
        return st;
    double *row = (double *)malloc(sizeof(double) * (size_t)(cols > 0 ? cols : 1));
    if (!row)
        return OR_ERR_NOMEM;
    for (int64_t r = 0; r < rows; r++) {
        decode_row(fmt, (const uint8_t *)raw, row_scale, r, cols, row);
        for (int64_t j = 0; j < cols; j++)
            w_out[r * cols + j] = (float)row[j];
    }
    free(row);
    return OR_OK;
}

/* y = Wdeq x for rows [row_begin, row_end), every token.
 * x is float [n_tok][cols]; y and S are double [n_tok][row_end - row_begin]. */
int oracle_gemv(int fmt, const void *raw, const float *row_scale, const float *x, int64_t rows,
                int64_t cols, int64_t n_tok, int64_t row_begin, int64_t row_end, double *y, double *S)
{
    int st = check_shape(fmt, rows, cols);
    if (st)
        return st;
    if (row_begin < 0 || row_end > rows || row_begin > row_end || n_tok < 0)
        return OR_ERR_SHAPE;
    int64_t nr = row_end - row_begin;
    double *row = (double *)malloc(sizeof(double) * (size_t)(cols > 0 ? cols : 1));
    if (!row)
        return OR_ERR_NOMEM;
    for (int64_t o = row_begin; o < row_end; o++) {
        decode_row(fmt, (const uint8_t *)raw, row_scale, o, cols, row); /* decode the row once */
        for (int64_t t = 0; t < n_tok; t++) {                          /* ...then every token */
            const float *xt = x + t * cols;
            double acc = 0.0, mag = 0.0;
            for (int64_t j = 0; j < cols; j++) {
                double p = row[j] * (double)xt[j];
                acc += p;
                mag += fabs(p);
            }
            y[t * nr + (o - row_begin)] = acc;
            S[t * nr + (o - row_begin)] = mag;
        }
    }
    free(row);
    return OR_OK;
}

/* Same product with a binary64 right-hand side (used for the FFN's down
 * projection applied to the oracle's own binary64 h). */
int oracle_gemv_f64x(int fmt, const void *raw, const float *row_scale, const double *x, int64_t rows,
                     int64_t cols, int64_t n_tok, double *y, double *S)
{
    int st = check_shape(fmt, rows, cols);
    if (st)
        return st;
    double *row = (double *)malloc(sizeof(double) * (size_t)(cols > 0 ? cols : 1));
    if (!row)
        return OR_ERR_NOMEM;
    for (int64_t o = 0; o < rows; o++) {
        decode_row(fmt, (const uint8_t *)raw, row_scale, o, cols, row);
        for (int64_t t = 0; t < n_tok; t++) {
            const double *xt = x + t * cols;
            double acc = 0.0, mag = 0.0;
            for (int64_t j = 0; j < cols; j++) {
                double p = row[j] * xt[j];
                acc += p;
                mag += fabs(p);
            }
            y[t * rows + o] = acc;
            S[t * rows + o] = mag;
        }
    }
    free(row);
    return OR_OK;
}

/* SiLU in the division form x / (1 + e^-x), binary64. */
double oracle_silu(double g) { return g / (1.0 + exp(-g)); }

/* SwiGLU FFN: gate and up are [ffn][d_model], down is [d_model][ffn].
 * Outputs (all binary64, token-major): g, u, h [n_tok][ffn]; out [n_tok][d_model];
 * Sg, Su [n_tok][ffn] and Sd [n_tok][d_model] are the sum|w*x| scales of the three
 * products (Sd is taken over the binary64 h).  No residual and no norm. */
int oracle_swiglu(int fmt, const void *wg, const float *sg, const void *wu, const float *su,
                  const void *wd, const float *sd, const float *x, int64_t d_model, int64_t ffn,
                  int64_t n_tok, double *g, double *u, double *h, double *out, double *Sg, double *Su,
                  double *Sd)
{
    int st = oracle_gemv(fmt, wg, sg, x, ffn, d_model, n_tok, 0, ffn, g, Sg);
    if (st)
        return st;
    st = oracle_gemv(fmt, wu, su, x, ffn, d_model, n_tok, 0, ffn, u, Su);
    if (st)
        return st;
    for (int64_t i = 0; i < n_tok * ffn; i++)
        h[i] = oracle_silu(g[i]) * u[i];
    return oracle_gemv_f64x(fmt, wd, sd, h, d_model, ffn, n_tok, out, Sd);
}

/* RMSNorm of each token row, binary64: scale[t] = 1/sqrt(sum_j x_j^2 / n + eps),
 * out[t][j] = x[t][j] * scale[t] * gamma[j].  x float [n_tok][n]. */
int oracle_rmsnorm(const float *x, const float *gamma, int64_t n, int64_t n_tok, double eps, double *out,
                   double *scale)
{
    if (n < 1 || n_tok < 0)
        return OR_ERR_SHAPE;
    for (int64_t t = 0; t < n_tok; t++) {
        const float *xt = x + t * n;
        double ss = 0.0;
        for (int64_t j = 0; j < n; j++)
            ss += (double)xt[j] * (double)xt[j];
        const double sc = 1.0 / sqrt(ss / (double)n + eps);
        scale[t] = sc;
        for (int64_t j = 0; j < n; j++)
            out[t * n + j] = (double)xt[j] * sc * (double)gamma[j];
    }
    return OR_OK;
}

/* The FFN block: xn = rmsnorm(x) * gamma; g = Wg xn, u = Wu xn, h = silu(g) u,
 * d = Wd h, out = x + d.  All outputs binary64, token-major; xn [n_tok][d_model],
 * g, u, h, Sg, Su [n_tok][ffn], d, out, Sd [n_tok][d_model]. */
int oracle_ffn_block(int fmt, const void *wg, const float *sg, const void *wu, const float *su,
                     const void *wd, const float *sd, const float *gamma, double eps, const float *x,
                     int64_t d_model, int64_t ffn, int64_t n_tok, double *xn, double *g, double *u,
                     double *h, double *d, double *out, double *Sg, double *Su, double *Sd)
{
    double *scale = (double *)malloc(sizeof(double) * (size_t)(n_tok > 0 ? n_tok : 1));
    if (!scale)
        return OR_ERR_NOMEM;
    int st = oracle_rmsnorm(x, gamma, d_model, n_tok, eps, xn, scale);
    free(scale);
    if (st)
        return st;
    st = oracle_gemv_f64x(fmt, wg, sg, xn, ffn, d_model, n_tok, g, Sg);
    if (st)
        return st;
    st = oracle_gemv_f64x(fmt, wu, su, xn, ffn, d_model, n_tok, u, Su);
    if (st)
        return st;
    for (int64_t i = 0; i < n_tok * ffn; i++)
        h[i] = oracle_silu(g[i]) * u[i];
    st = oracle_gemv_f64x(fmt, wd, sd, h, d_model, ffn, n_tok, d, Sd);
    if (st)
        return st;
    for (int64_t i = 0; i < n_tok * d_model; i++)
        out[i] = (double)x[i] + d[i];
    return OR_OK;
}

/* Q8_0 quantization of activation rows: n a multiple of 32, x [n_tok][n];
 * d_bits [n_tok][n/32] binary16 scales, q [n_tok][n] codes. */
int oracle_quantize_q8_0(const float *x, int64_t n, int64_t n_tok, uint16_t *d_bits, int8_t *q)
{
    if (n < 0 || n % 32 || n_tok < 0)
        return OR_ERR_SHAPE;
    for (int64_t b = 0; b < n_tok * (n / 32); b++) {
        const float *xb = x + 32 * b;
        float amax = 0.0f;
        for (int l = 0; l < 32; l++) {
            const float a = fabsf(xb[l]);
            if (a > amax)
                amax = a;
        }
        const float d = amax / 127.0f;
        const float id = d != 0.0f ? 1.0f / d : 0.0f;
        for (int l = 0; l < 32; l++)
            q[32 * b + l] = (int8_t)roundf(xb[l] * id);
        d_bits[b] = oracle_f32_to_f16(d);
    }
    return OR_OK;
}

/* y = Wdeq xq with xq the Q8_0 representation of x (f16(d) * q per block),
 * binary64; S = sum_j |w_ij * xq_tj|.  Q4_0 and Q8_0 weights (the formats of
 * the model the mode was written for). */
int oracle_gemv_q8act(int fmt, const void *raw, const float *x, int64_t rows, int64_t cols, int64_t n_tok,
                      double *y, double *S)
{
    if (fmt != OR_Q4_0 && fmt != OR_Q8_0)
        return OR_ERR_FORMAT;
    int st = check_shape(fmt, rows, cols);
    if (st)
        return st;
    if (n_tok < 0)
        return OR_ERR_SHAPE;
    const int64_t nx = n_tok * cols;
    uint16_t *d_bits = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(nx / 32 + 1));
    int8_t *q = (int8_t *)malloc((size_t)(nx + 1));
    double *xq = (double *)malloc(sizeof(double) * (size_t)(nx + 1));
    if (!d_bits || !q || !xq) {
        free(d_bits);
        free(q);
        free(xq);
        return OR_ERR_NOMEM;
    }
    oracle_quantize_q8_0(x, cols, n_tok, d_bits, q);
    for (int64_t j = 0; j < nx; j++)
        xq[j] = oracle_f16_to_f64(d_bits[j / 32]) * (double)q[j];
    st = oracle_gemv_f64x(fmt, raw, NULL, xq, rows, cols, n_tok, y, S);
    free(d_bits);
    free(q);
    free(xq);
    return st;
}

/* Index of the largest of v[0..n), scanning in order and replacing the best
 * only on a strictly greater value: the first index wins ties, -0 equals +0,
 * a NaN never replaces the best (and a NaN at index 0 is never replaced). */
int64_t oracle_argmax(const float *v, int64_t n)
{
    if (n < 1)
        return OR_ERR_SHAPE;
    int64_t best = 0;
    for (int64_t i = 1; i < n; i++)
        if (v[i] > v[best])
            best = i;
    return best;
}
