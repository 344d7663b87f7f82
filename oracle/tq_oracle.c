/*
 * tq_oracle.c -- plain, slow CPU oracle for the ternary GEMV hot path.
 *
 * TEST INFRASTRUCTURE ONLY (see tq_oracle.h).  Compiled by gcc with
 * -O2 -fno-fast-math -ffp-contract=off, so every float expression below is
 * evaluated as written, one IEEE fp32 (or fp64) rounding per operation.
 *
 * Every function is the plain definition written out: no blocking, no
 * fusion, no reordering.  Pages are cited by title; see tq_oracle.h.
 */
#include "tq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* bf16 is the upper 16 bits of an IEEE binary32; widening is exact. */
float tqo_bf16_to_f32(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/*
 * Packing.  [ISSUE] "Architecture": ternary weights are stored as uint8,
 * four values per byte; "Weight mapping (bitnet-b1.58-2B-4T)": a projection
 * [N,K] is held as a [N/4,K] uint8 array.  The assignment of rows to the
 * four 2-bit fields and the code of each value are not given on the page;
 * the reading used here (row j*N/4+i in bits 2j..2j+1, code = w+1) is the
 * plainest one that reproduces those shapes.
 */
int tqo_pack(const int8_t *w, int64_t N, int64_t K, uint8_t *packed)
{
    if (N < 0 || K < 0) return TQO_EARG;
    if (N % 4 != 0) return TQO_ESHAPE;
    if ((N > 0 && K > 0) && (!w || !packed)) return TQO_EARG;
    const int64_t n4 = N / 4;
    for (int64_t i = 0; i < n4; i++) {
        for (int64_t k = 0; k < K; k++) {
            unsigned byte = 0;
            for (int j = 0; j < 4; j++) {
                int v = w[(j * n4 + i) * K + k];
                if (v < -1 || v > 1) return TQO_ECODE;
                unsigned code = (unsigned)(v + 1);
                byte |= code << (2 * j);
            }
            packed[i * K + k] = (uint8_t)byte;
        }
    }
    return TQO_OK;
}

int tqo_unpack(const uint8_t *packed, int64_t N, int64_t K, int8_t *w)
{
    if (N < 0 || K < 0) return TQO_EARG;
    if (N % 4 != 0) return TQO_ESHAPE;
    if ((N > 0 && K > 0) && (!w || !packed)) return TQO_EARG;
    const int64_t n4 = N / 4;
    for (int64_t n = 0; n < N; n++) {
        int64_t j = n / n4;
        int64_t i = n % n4;
        for (int64_t k = 0; k < K; k++) {
            unsigned code = (packed[i * K + k] >> (2 * j)) & 3u;
            if (code == 3u) return TQO_ECODE;
            w[n * K + k] = (int8_t)((int)code - 1);
        }
    }
    return TQO_OK;
}

/*
 * Denser packing: five ternary weights per byte, 1.6 bits per weight (the
 * page "Feature request: BitNet 1.58-bit ternary inference on ROCm
 * (gfx1151)", section "Context", names the "TQ1_0" family only; no layout
 * is given).  Reading used here: the packed array is [N5, K] with
 * N5 = ceil(N/5); byte [i,k] holds rows j*N5 + i (j = 0..4) of column k as
 * the base-3 number v = sum_j c_j 3^j of their codes c = w + 1 (rows past N
 * are zero weights, c = 1), stored as the byte q = ceil(256 v / 243).  v is
 * recovered as floor(243 q / 256); bytes that are not the image of some v
 * (13 of the 256) are reserved.
 */
static int64_t n5_of(int64_t N) { return (N + 4) / 5; }

int tqo_pack3(const int8_t *w, int64_t N, int64_t K, uint8_t *packed)
{
    if (N < 0 || K < 0) return TQO_EARG;
    const int64_t n5 = n5_of(N);
    if ((n5 > 0 && K > 0) && (!w || !packed)) return TQO_EARG;
    for (int64_t i = 0; i < n5; i++) {
        for (int64_t k = 0; k < K; k++) {
            unsigned v = 0, p3 = 1;
            for (int j = 0; j < 5; j++) {
                int64_t n = j * n5 + i;
                int c = 1;                      /* padding row: weight 0 */
                if (n < N) {
                    int wv = w[n * K + k];
                    if (wv < -1 || wv > 1) return TQO_ECODE;
                    c = wv + 1;
                }
                v += (unsigned)c * p3;
                p3 *= 3;
            }
            packed[i * K + k] = (uint8_t)((v * 256 + 242) / 243);
        }
    }
    return TQO_OK;
}

int tqo_unpack3(const uint8_t *packed, int64_t N, int64_t K, int8_t *w)
{
    if (N < 0 || K < 0) return TQO_EARG;
    const int64_t n5 = n5_of(N);
    if ((n5 > 0 && K > 0) && (!w || !packed)) return TQO_EARG;
    for (int64_t i = 0; i < n5; i++) {
        for (int64_t k = 0; k < K; k++) {
            unsigned q = packed[i * K + k];
            unsigned v = (q * 243) >> 8;
            if ((v * 256 + 242) / 243 != q) return TQO_ECODE;   /* reserved */
            for (int j = 0; j < 5; j++) {
                int c = (int)(v % 3);
                v /= 3;
                int64_t n = j * n5 + i;
                if (n < N)
                    w[n * K + k] = (int8_t)(c - 1);
                else if (c != 1)
                    return TQO_ECODE;                        /* padding not zero */
            }
        }
    }
    return TQO_OK;
}

/*
 * Per-token absmax quantization to int8 of one row of K fp32 values.
 * Decision arithmetic is fp32, as in the kernel that takes the same decision.
 */
static void quant_row(const float *x, int64_t K, int8_t *q, float *s_x)
{
    float a = 0.0f;
    for (int64_t k = 0; k < K; k++) {
        float ax = fabsf(x[k]);
        if (ax > a) a = ax;
    }
    float ap = a > 1e-5f ? a : 1e-5f;      /* floor keeps 127/a' finite */
    float inv = 127.0f / ap;                /* one correctly rounded divide */
    for (int64_t k = 0; k < K; k++) {
        float t = x[k] * inv;               /* one fp32 rounding */
        float r = nearbyintf(t);            /* ties to even (default mode) */
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        q[k] = (int8_t)r;
    }
    *s_x = ap / 127.0f;
}

int tqo_act_quant_f32(const float *x, int64_t M, int64_t K,
                      int8_t *q, float *s_x)
{
    if (M < 0 || K < 0) return TQO_EARG;
    if (M > 0 && !s_x) return TQO_EARG;
    if (M > 0 && K > 0 && (!x || !q)) return TQO_EARG;
    for (int64_t m = 0; m < M; m++)
        quant_row(x + m * K, K, q + m * K, s_x + m);
    return TQO_OK;
}

int tqo_act_quant_bf16(const uint16_t *x, int64_t M, int64_t K,
                       int8_t *q, float *s_x)
{
    if (M < 0 || K < 0) return TQO_EARG;
    if (M > 0 && !s_x) return TQO_EARG;
    if (M > 0 && K > 0 && (!x || !q)) return TQO_EARG;
    /* Widen each row exactly to fp32, then quantize it as an fp32 row. */
    float *row = (float *)malloc((size_t)(K > 0 ? K : 1) * sizeof(float));
    if (!row) return TQO_EARG;
    for (int64_t m = 0; m < M; m++) {
        for (int64_t k = 0; k < K; k++)
            row[k] = tqo_bf16_to_f32(x[m * K + k]);
        quant_row(row, K, q + m * K, s_x + m);
    }
    free(row);
    return TQO_OK;
}

/*
 * Sub-layer RMSNorm folded into the quantization of one row ([ISSUE]
 * "Architecture": sub-layer norms before o_proj and down_proj; "Diagnose"
 * lists RMSNorm).  RMSNorm(x)_k = r * x_k * gamma_k with
 * r = 1/sqrt(mean_k(x_k^2) + eps).  Absmax quantization gives the same codes
 * for a row and for any positive multiple of it, so the codes are those of
 * u = x*gamma (fp32 products) and r goes into the scale:
 * s_x = (a'/127) * r, with a' the floored absmax of u.  mean(x^2) and r are
 * formed in fp64 (each x^2 is exact there) and r is rounded once to fp32.
 */
static void rms_quant_row(const float *x, const float *gamma, int64_t K,
                          float eps, int8_t *q, float *s_x, float *u)
{
    double ss = 0.0;
    for (int64_t k = 0; k < K; k++) {
        u[k] = x[k] * gamma[k];             /* one fp32 rounding */
        ss += (double)x[k] * (double)x[k];
    }
    float s_q;
    quant_row(u, K, q, &s_q);
    double r = 1.0 / sqrt(ss / (double)K + (double)eps);
    *s_x = s_q * (float)r;
}

int tqo_rmsnorm_act_quant_f32(const float *x, const float *gamma, float eps,
                              int64_t M, int64_t K, int8_t *q, float *s_x)
{
    if (M < 0 || K <= 0 || !(eps > 0.0f)) return TQO_EARG;
    if (M > 0 && (!x || !gamma || !q || !s_x)) return TQO_EARG;
    float *u = (float *)malloc((size_t)K * sizeof(float));
    if (!u) return TQO_EARG;
    for (int64_t m = 0; m < M; m++)
        rms_quant_row(x + m * K, gamma, K, eps, q + m * K, s_x + m, u);
    free(u);
    return TQO_OK;
}

int tqo_rmsnorm_act_quant_bf16(const uint16_t *x, const uint16_t *gamma,
                               float eps, int64_t M, int64_t K, int8_t *q,
                               float *s_x)
{
    if (M < 0 || K <= 0 || !(eps > 0.0f)) return TQO_EARG;
    if (M > 0 && (!x || !gamma || !q || !s_x)) return TQO_EARG;
    float *buf = (float *)malloc((size_t)K * 3 * sizeof(float));
    if (!buf) return TQO_EARG;
    float *row = buf, *g = buf + K, *u = buf + 2 * K;
    for (int64_t k = 0; k < K; k++) g[k] = tqo_bf16_to_f32(gamma[k]);
    for (int64_t m = 0; m < M; m++) {
        for (int64_t k = 0; k < K; k++) row[k] = tqo_bf16_to_f32(x[m * K + k]);
        rms_quant_row(row, g, K, eps, q + m * K, s_x + m, u);
    }
    free(buf);
    return TQO_OK;
}

/*
 * The ternary product as its definition: every weight is decoded to
 * {-1,0,+1} and multiplied into an exact int64 sum.  [DIGEST] first item:
 * with weights in {-1,0,1} each product is an add, a subtract or nothing.
 */
static int dot_row(const uint8_t *packed, const int8_t *qrow,
                   int64_t N, int64_t K, int64_t n, int32_t *out)
{
    const int64_t n4 = N / 4;
    const int64_t j = n / n4;
    const int64_t i = n % n4;
    int64_t sum = 0;
    for (int64_t k = 0; k < K; k++) {
        unsigned code = (packed[i * K + k] >> (2 * j)) & 3u;
        if (code == 3u) return TQO_ECODE;
        int64_t w = (int64_t)code - 1;
        sum += w * (int64_t)qrow[k];
    }
    if (sum > INT32_MAX || sum < INT32_MIN) return TQO_ERANGE;
    *out = (int32_t)sum;
    return TQO_OK;
}

int tqo_ternary_matmul(const uint8_t *packed, const int8_t *q,
                       int64_t M, int64_t N, int64_t K, int32_t *acc)
{
    if (M < 0 || N < 0 || K < 0) return TQO_EARG;
    if (N % 4 != 0) return TQO_ESHAPE;
    if (M > 0 && N > 0 && !acc) return TQO_EARG;
    if (M > 0 && N > 0 && K > 0 && (!packed || !q)) return TQO_EARG;
    for (int64_t m = 0; m < M; m++) {
        for (int64_t n = 0; n < N; n++) {
            int rc = dot_row(packed, q + m * K, N, K, n, &acc[m * N + n]);
            if (rc) return rc;
        }
    }
    return TQO_OK;
}

int tqo_ternary_matmul_rows(const uint8_t *packed, const int8_t *q,
                            int64_t M, int64_t N, int64_t K,
                            const int64_t *rows, int64_t R, int32_t *acc)
{
    if (M < 0 || N < 0 || K < 0 || R < 0) return TQO_EARG;
    if (N % 4 != 0) return TQO_ESHAPE;
    if (M > 0 && R > 0 && (!acc || !rows)) return TQO_EARG;
    if (M > 0 && R > 0 && K > 0 && (!packed || !q)) return TQO_EARG;
    for (int64_t m = 0; m < M; m++) {
        for (int64_t r = 0; r < R; r++) {
            if (rows[r] < 0 || rows[r] >= N) return TQO_EARG;
            int rc = dot_row(packed, q + m * K, N, K, rows[r], &acc[m * R + r]);
            if (rc) return rc;
        }
    }
    return TQO_OK;
}

/*
 * Rescale of the exact integer sum to fp32.  The combined scale is one fp32
 * product, then one fp32 product with the (exactly converted) sum; with no
 * additions there is nothing for a compiler to contract.
 */
int tqo_rescale_f32(const int32_t *acc, float s_w, const float *s_x,
                    int64_t M, int64_t N, float *y)
{
    if (M < 0 || N < 0) return TQO_EARG;
    if (M > 0 && N > 0 && (!acc || !s_x || !y)) return TQO_EARG;
    for (int64_t m = 0; m < M; m++) {
        float c = s_w * s_x[m];
        for (int64_t n = 0; n < N; n++)
            y[m * N + n] = (float)acc[m * N + n] * c;
    }
    return TQO_OK;
}

int tqo_rescale_f64(const int32_t *acc, float s_w, const float *s_x,
                    int64_t M, int64_t N, double *y)
{
    if (M < 0 || N < 0) return TQO_EARG;
    if (M > 0 && N > 0 && (!acc || !s_x || !y)) return TQO_EARG;
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++)
            y[m * N + n] = (double)acc[m * N + n] * (double)s_w * (double)s_x[m];
    return TQO_OK;
}

/* [ISSUE] "Architecture": the MLP uses a squared ReLU in place of SiLU. */
int tqo_relu2_f32(const float *g, const float *u, int64_t n, float *h)
{
    if (n < 0) return TQO_EARG;
    if (n > 0 && (!g || !u || !h)) return TQO_EARG;
    for (int64_t i = 0; i < n; i++) {
        float r = g[i] > 0.0f ? g[i] : 0.0f;
        h[i] = (r * r) * u[i];
    }
    return TQO_OK;
}

int tqo_relu2_f64(const double *g, const double *u, int64_t n, double *h)
{
    if (n < 0) return TQO_EARG;
    if (n > 0 && (!g || !u || !h)) return TQO_EARG;
    for (int64_t i = 0; i < n; i++) {
        double r = g[i] > 0.0 ? g[i] : 0.0;
        h[i] = (r * r) * u[i];
    }
    return TQO_OK;
}
