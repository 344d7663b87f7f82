/*
 * tq_oracle.h -- plain, slow CPU oracle for the BitNet b1.58 ternary
 * matrix-vector product at decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library and its Python binding) never calls, links or imports it, and
 * this file shares no code, header, table or constant with that path.
 *
 * Pages cited (by title):
 *   [ISSUE]  "Feature request: BitNet 1.58-bit ternary inference on ROCm
 *            (gfx1151)" -- sections "Architecture" and
 *            "Weight mapping (bitnet-b1.58-2B-4T)".
 *   [DIGEST] "BitNet" news-digest tag page -- first item (the C99 engine):
 *            weights in {-1,0,1} turn multiplies into adds and subtracts.
 *
 * Conventions fixed here (the pages leave them open; each is one reading):
 *   - code of a weight w in {-1,0,+1} is the unsigned 2-bit value w+1
 *     (0 -> -1, 1 -> 0, 2 -> +1, 3 is reserved and rejected);
 *   - packed byte [i,k] of a [N/4,K] array holds the codes of rows
 *     i, i+N/4, i+2N/4, i+3N/4 of column k, row j*N/4+i in bits 2j..2j+1;
 *   - activations: per row, a = max|x|, a' = max(a, 1e-5f),
 *     inv = 127/a' (fp32), q = clamp(round-half-even(x*inv), -127, 127),
 *     s_x = a'/127 (fp32);
 *   - sub-layer RMSNorm before quantizing: codes of u = x*gamma, and
 *     s_x = (a'/127) * r, r = 1/sqrt(mean(x^2) + eps) in fp64 rounded once;
 *   - rescale: y = (float)acc * (s_w * s_x), each product rounded to fp32;
 *   - relu^2 gate: r = g > 0 ? g : 0,  h = (r*r)*u, in fp32.
 * The fp64 variants give the exact value of the same definition.
 *
 * Return value of every int function: 0 on success, nonzero on bad input
 * (see TQO_E*).  No function allocates memory that outlives the call.
 */
#ifndef TQ_ORACLE_H
#define TQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    TQO_OK = 0,
    TQO_EARG = 1,     /* null pointer or negative size */
    TQO_ESHAPE = 2,   /* N not a multiple of 4 */
    TQO_ECODE = 3,    /* weight outside {-1,0,1}, or reserved code 3 */
    TQO_ERANGE = 4    /* accumulator does not fit int32 */
};

/* bf16 bit pattern -> fp32 (exact: bf16 is the top half of an fp32). */
float tqo_bf16_to_f32(uint16_t b);

/* Pack int8 weights w[N,K] (values in {-1,0,1}) into packed[N/4,K]. */
int tqo_pack(const int8_t *w, int64_t N, int64_t K, uint8_t *packed);

/* Inverse of tqo_pack: packed[N/4,K] -> w[N,K]. */
int tqo_unpack(const uint8_t *packed, int64_t N, int64_t K, int8_t *w);

/* Five weights per byte: w[N,K] -> packed[ceil(N/5),K]; byte [i,k] holds rows
 * j*ceil(N/5)+i as q = ceil(256 v/243), v = sum_j (w+1) 3^j (rows past N are
 * zero weights).  Unpack rejects reserved bytes and nonzero padding. */
int tqo_pack3(const int8_t *w, int64_t N, int64_t K, uint8_t *packed);
int tqo_unpack3(const uint8_t *packed, int64_t N, int64_t K, int8_t *w);

/* Per-row absmax int8 quantization of x[M,K] (fp32 or bf16 bit patterns). */
int tqo_act_quant_f32(const float *x, int64_t M, int64_t K,
                      int8_t *q, float *s_x);
int tqo_act_quant_bf16(const uint16_t *x, int64_t M, int64_t K,
                       int8_t *q, float *s_x);

/* RMSNorm(x) * gamma folded into the quantization of each row of x[M,K]:
 * q = codes of u = x*gamma (fp32), s_x = (a'/127) * r with
 * r = 1/sqrt(mean(x^2) + eps) (fp64, rounded once).  K > 0, eps > 0;
 * gamma[K] has the dtype of x. */
int tqo_rmsnorm_act_quant_f32(const float *x, const float *gamma, float eps,
                              int64_t M, int64_t K, int8_t *q, float *s_x);
int tqo_rmsnorm_act_quant_bf16(const uint16_t *x, const uint16_t *gamma,
                               float eps, int64_t M, int64_t K, int8_t *q,
                               float *s_x);

/* acc[m,n] = sum_k W[n,k] * q[m,k], W decoded from packed[N/4,K]. */
int tqo_ternary_matmul(const uint8_t *packed, const int8_t *q,
                       int64_t M, int64_t N, int64_t K, int32_t *acc);

/* Same, for a subset of output rows: acc[m, r] for n = rows[r]. */
int tqo_ternary_matmul_rows(const uint8_t *packed, const int8_t *q,
                            int64_t M, int64_t N, int64_t K,
                            const int64_t *rows, int64_t R, int32_t *acc);

/* y[m,n] = acc[m,n] * s_w * s_x[m]; fp32 in the fixed order, or exact fp64. */
int tqo_rescale_f32(const int32_t *acc, float s_w, const float *s_x,
                    int64_t M, int64_t N, float *y);
int tqo_rescale_f64(const int32_t *acc, float s_w, const float *s_x,
                    int64_t M, int64_t N, double *y);

/* h = relu(g)^2 * u, elementwise over n values. */
int tqo_relu2_f32(const float *g, const float *u, int64_t n, float *h);
int tqo_relu2_f64(const double *g, const double *u, int64_t n, double *h);

#ifdef __cplusplus
}
#endif

#endif /* TQ_ORACLE_H */
