/*
 * tq.h -- C ABI of the ternary GEMV library (libtq.so) for AMD MI355X
 * (gfx950 / CDNA4).
 *
 * The library computes the BitNet b1.58 ternary matrix-vector product at
 * decode and its small-batch and gated-MLP variants.  Pages cited by title:
 *   [ISSUE]  "Feature request: BitNet 1.58-bit ternary inference on ROCm
 *            (gfx1151)" -- section "Architecture" (ternary weights stored
 *            as uint8, four values per byte; squared-ReLU MLP) and section
 *            "Weight mapping (bitnet-b1.58-2B-4T)" (a projection [N,K] is
 *            held as a [N/4,K] uint8 array; per-tensor .weight_scale keys
 *            are named in "What We Need"); section "Context" names the
 *            TQ1_0 ternary format family.
 *   [ARC]    "the full arc: how the 1bit.systems ternary stack got from
 *            broken to 76.7 tok/s" -- TL;DR (a hand-tuned ternary GEMV
 *            near the memory-bandwidth peak is the decode hot loop).
 *   [DIGEST] "BitNet" news-digest tag page, first item: weights in {-1,0,1}
 *            replace multiplies with adds and subtracts.
 *   [README] "1bit.systems" project README -- sections "hardware" and
 *            "honest numbers".
 *   [BLOG]   "Blog · field notes" (1bit engine) -- posts "Qwen3.8-27B at
 *            45.7 tok/s" (decode is bandwidth bound, prompt processing
 *            matrix-unit bound) and "One GPU, many users" (several requests
 *            served by one GPU).
 *
 * Data conventions (shared by every call):
 *   - W is an [N,K] matrix of ternary weights w in {-1,0,+1}.  Packed form:
 *     uint8 [N/4,K], row-major (K contiguous).  Byte [i,k] holds, in bits
 *     2j..2j+1 (j = 0..3, least significant pair first), the code w+1 of
 *     row n = j*(N/4) + i, column k.  Code 3 is reserved.  (The page fixes
 *     the [N/4,K] uint8 shape; the code and the row-to-bit assignment are
 *     this library's reading.)
 *   - s_w: one fp32 weight scale per tensor, passed by value; the real
 *     weight is s_w * w.
 *   - Activations x: [M,K] row-major, bf16 or fp32.  Each row m is quantized
 *     to int8 by its absmax: a = max_k |x[m,k]|, a' = max(a, 1e-5),
 *     inv = 127/a' (fp32, correctly rounded), q = clamp(rne(x*inv), +-127)
 *     with rne = round half to even, and s_x[m] = a'/127 (fp32).
 *   - Products are exact: acc[m,n] = sum_k w[n,k]*q[m,k] in int32.
 *   - Rescale: y[m,n] = (float)acc[m,n] * (s_w * s_x[m]), each product
 *     rounded once to fp32, in that order.  Results are bit-reproducible.
 *
 * Memory and streams:
 *   - Every array argument is caller-owned DEVICE memory on the current HIP
 *     device.  The library allocates and frees nothing and keeps no state
 *     beyond a per-device cache of the compute-unit count (and the fixed
 *     device array of tq_attn_decode_noalloc, with its per-device address).
 *   - Every call enqueues its work on `stream` (NULL = the default stream)
 *     and returns without synchronizing.  Calls are thread-safe.
 *
 * Errors: a call returns a tq_status synchronously.  Host-detectable
 * problems (null pointer, bad shape, misalignment, bad dtype, no device) are
 * reported before anything is enqueued; nothing is launched then.
 * TQ_ERR_LAUNCH reports a failed kernel launch.  Faults during execution
 * surface at the caller's next synchronization, as in HIP.
 *
 * Shape rules: N % 4 == 0; K % 16 == 0; 0 <= K <= TQ_MAX_K;
 * 1 <= M <= TQ_MAX_M where M is an argument.  N == 0 or M == 0 is a no-op
 * returning TQ_OK.  K == 0 is allowed (empty sums: acc = 0).
 * Alignment: packed, xq, x and the int8 weights of tq_pack / tq_pack3 16-byte
 * aligned; y, acc, h, x_scale 4-byte.
 * Inputs must be finite; NaN/Inf activations are outside the contract.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exported entry points (the library is built with hidden visibility). */
#define TQ_API __attribute__((visibility("default")))

/* HIP's stream handle (identical to the typedef in hip_runtime_api.h). */
typedef struct ihipStream_t *hipStream_t;

typedef enum tq_status {
    TQ_OK = 0,
    TQ_ERR_NULL = 1,    /* a required pointer is NULL */
    TQ_ERR_SHAPE = 2,   /* size out of range or not a required multiple */
    TQ_ERR_ALIGN = 3,   /* pointer not aligned as required */
    TQ_ERR_DTYPE = 4,   /* unknown tq_dtype */
    TQ_ERR_DEVICE = 5,  /* no usable HIP device */
    TQ_ERR_LAUNCH = 6   /* the kernel launch failed */
} tq_status;

typedef enum tq_dtype {
    TQ_BF16 = 0,
    TQ_F32 = 1
} tq_dtype;

/* Largest K: 127*K stays below 2^24, so (float)acc is exact, and the int8
   activation row fits the kernels' LDS staging. */
#define TQ_MAX_K 131072
/* Largest activation batch of tq_gemm_small / tq_gate_up_relu2. */
#define TQ_MAX_M 64

/*
 * tq_pack -- pack ternary weights ([ISSUE] "Architecture": uint8, four
 * values per byte; "Weight mapping": [N,K] -> [N/4,K]).
 *   w       int8 [N,K], 16-byte aligned, values in {-1,0,1}; any other value
 *           is written as the reserved code 3 (outside the contract of every
 *           other call).
 *   packed  uint8 [N/4,K], output, 16-byte aligned.
 */
TQ_API tq_status tq_pack(const int8_t *w, int64_t N, int64_t K, uint8_t *packed,
                  hipStream_t stream);

/*
 * tq_pack3 -- the denser layout: five weights per byte, 1.6 bits per weight
 * ([ISSUE] section "Context" names the "TQ1_0" family of such formats
 * only; the layout is this library's reading).  packed [N5, K], N5 = ceil(N/5); byte [i,k]
 * holds rows j*N5 + i (j = 0..4) of column k as the base-3 number
 * v = sum_j (w+1) 3^j (rows past N count as zero weights), stored as
 * q = ceil(256 v / 243).  13 byte values encode no v and are reserved.
 *   w       int8 [N,K], values in {-1,0,1}, 16-B aligned; any other value
 *           makes its byte the reserved value 1 (outside the contract of
 *           tq_gemv3).
 *   packed  uint8 [ceil(N/5), K], output, 16-byte aligned.
 * K % 16 == 0; any N >= 0.
 */
TQ_API tq_status tq_pack3(const int8_t *w, int64_t N, int64_t K, uint8_t *packed,
                          hipStream_t stream);

/*
 * tq_gemv3 -- tq_gemv on the tq_pack3 layout: the same exact sums and the
 * same fp32 outputs, bit for bit, reading 20% fewer weight bytes.
 *   packed   uint8 [ceil(N/5), K] from tq_pack3 (16-B aligned), w_scale = s_w.
 *   xq, x_scale, y, acc  as tq_gemv.
 * 16 <= K <= 32768, K % 16 == 0; N >= 0 (N = 0: nothing is written).
 */
TQ_API tq_status tq_gemv3(const uint8_t *packed, float w_scale, const int8_t *xq,
                          const float *x_scale, int64_t N, int64_t K, float *y,
                          int32_t *acc, hipStream_t stream);

/*
 * tq_act_quant -- per-token absmax int8 quantization of activations
 * (the conventions above).
 *   x        [M,K] bf16 (xt = TQ_BF16) or fp32 (xt = TQ_F32), 16-B aligned.
 *   xq       int8 [M,K], output, 16-B aligned.
 *   x_scale  fp32 [M], output: s_x[m] = a'/127.
 *   M        1..TQ_MAX_M.
 */
TQ_API tq_status tq_act_quant(const void *x, tq_dtype xt, int64_t M, int64_t K,
                       int8_t *xq, float *x_scale, hipStream_t stream);

/*
 * tq_gemv -- the ternary matrix-vector product at M = 1 ([ARC] TL;DR:
 * the decode hot loop; [DIGEST]: add/subtract/skip per weight).
 *   packed   uint8 [N/4,K] (16-B aligned), w_scale = s_w.
 *   xq       int8 [K] (16-B aligned), x_scale fp32 [1] (device).
 *   y        fp32 [N], output: y[n] = (float)acc[n] * (s_w * x_scale[0]).
 *   acc      int32 [N], optional output of the exact sums (NULL = skip).
 */
TQ_API tq_status tq_gemv(const uint8_t *packed, float w_scale, const int8_t *xq,
                  const float *x_scale, int64_t N, int64_t K, float *y,
                  int32_t *acc, hipStream_t stream);

/*
 * tq_gemm_small -- the same product for a small batch of activation rows
 * (batched decode / short prefill; [BLOG] "One GPU, many users"), on the
 * int8 matrix cores (M = 2 with K <= 16384 on the vector ALU instead: the
 * GEMV's structure with both rows in registers, which measured faster
 * there).  Every row equals the M = 1 GEMV of that row bit for bit.
 *   xq       int8 [M,K] (16-B aligned), x_scale fp32 [M].
 *   y        fp32 [M,N], output: y[m,n] = (float)acc[m,n]*(s_w*x_scale[m]).
 *   acc      int32 [M,N], optional (NULL = skip).
 *   M        1..TQ_MAX_M.
 */
TQ_API tq_status tq_gemm_small(const uint8_t *packed, float w_scale, const int8_t *xq,
                        const float *x_scale, int64_t M, int64_t N, int64_t K,
                        float *y, int32_t *acc, hipStream_t stream);

/*
 * tq_gate_up_relu2 -- fused gate and up projections with the squared-ReLU
 * gate ([ISSUE] "Architecture": relu_squared in place of SiLU):
 *   g = gemm(packed_gate, s_gate), u = gemm(packed_up, s_up) on the same xq,
 *   h[m,n] = (r*r) * u[m,n] with r = g[m,n] > 0 ? g[m,n] : 0 (fp32).
 *   packed_gate, packed_up  uint8 [N/4,K] each (16-B aligned).
 *   xq int8 [M,K], x_scale fp32 [M]; h fp32 [M,N] output.
 *   acc_gate, acc_up  int32 [M,N], optional exact sums (NULL = skip).
 *   M  1..TQ_MAX_M (M = 1 uses the GEMV kernels, M > 1 the matrix cores).
 */
TQ_API tq_status tq_gate_up_relu2(const uint8_t *packed_gate, float s_gate,
                           const uint8_t *packed_up, float s_up,
                           const int8_t *xq, const float *x_scale, int64_t M,
                           int64_t N, int64_t K, float *h, int32_t *acc_gate,
                           int32_t *acc_up, hipStream_t stream);

/*
 * tq_quant_gemv -- tq_act_quant followed by tq_gemv at M = 1 in one launch
 * (the per-token quantization runs in the GEMV prologue; every block
 * recomputes the row's absmax, then quantizes into LDS).  Results are bit-
 * identical to the two calls.
 *   x        [K] bf16 (xt = TQ_BF16) or fp32 (xt = TQ_F32), 16-B aligned.
 *   packed   uint8 [N/4,K] (16-B aligned), w_scale = s_w.
 *   y        fp32 [N], output: y[n] = (float)acc[n] * (s_w * s), where s is
 *            *y_scale when y_scale is non-NULL, else the row's own s_x.
 *   acc      int32 [N], optional exact sums (NULL = skip).
 *   xq       int8 [K], output: the quantized row (16-B aligned, required).
 *   x_scale  fp32 [1], output: s_x (required).
 *   y_scale  fp32 [1] device pointer or NULL: an activation scale to use in
 *            the rescale instead of s_x (a caller that treats its input as
 *            already normalized passes 1/127 here).
 * With N == 0 only xq and x_scale are produced.  K == 0 or K > 32768 take
 * two launches internally (same results).
 */
TQ_API tq_status tq_quant_gemv(const void *x, tq_dtype xt,
                               const uint8_t *packed, float w_scale, int64_t N,
                               int64_t K, float *y, int32_t *acc, int8_t *xq,
                               float *x_scale, const float *y_scale,
                               hipStream_t stream);

/*
 * tq_rmsnorm_act_quant -- the sub-layer RMSNorm folded into the per-token
 * quantization ([ISSUE] "Architecture": norms before o_proj and down_proj;
 * RMSNorm(x)_k = x_k * gamma_k / sqrt(mean(x^2) + eps)).  Absmax
 * quantization gives the same codes for any positive multiple of a row, so
 * the codes are those of u = x * gamma (fp32 products) and the RMS factor
 * goes into the scale:
 *   xq[m,:]    = the tq_act_quant codes of u[m,:]
 *   x_scale[m] = (a'/127) * r,  r = 1/sqrt(mean_k x[m,k]^2 + eps), the mean
 *                and r formed in fp64 and r rounded once to fp32.
 * xq * x_scale approximates RMSNorm(x) * gamma.  The codes are exact
 * decisions; x_scale depends on the order in which the squares are summed
 * only in its last bit, rarely.
 *   x, xq, x_scale, M  as tq_act_quant.
 *   gamma    [K], the dtype of x, 16-B aligned (device).
 *   eps      > 0 and finite.
 *   K        > 0 (an empty row has no mean).
 */
TQ_API tq_status tq_rmsnorm_act_quant(const void *x, tq_dtype xt, const void *gamma,
                                      float eps, int64_t M, int64_t K, int8_t *xq,
                                      float *x_scale, hipStream_t stream);

/*
 * tq_rmsnorm_quant_gemv -- tq_rmsnorm_act_quant followed by tq_gemv at
 * M = 1 in one launch: the RMSNorm and the quantization run in the GEMV
 * prologue (every block recomputes the row's absmax and sum of squares in
 * the same order).  Arguments as tq_quant_gemv (no y_scale: y uses the
 * row's own x_scale) plus gamma and eps as tq_rmsnorm_act_quant.  Codes and
 * acc equal those of the two calls exactly; x_scale and y may differ from
 * theirs in the last bit, rarely (the squares are summed in another order).
 * K > 32768 takes two launches internally.
 */
TQ_API tq_status tq_rmsnorm_quant_gemv(const void *x, tq_dtype xt, const void *gamma,
                                       float eps, const uint8_t *packed, float w_scale,
                                       int64_t N, int64_t K, float *y, int32_t *acc,
                                       int8_t *xq, float *x_scale, hipStream_t stream);

/*
 * tq_quant_gate_up_relu2 -- tq_act_quant followed by tq_gate_up_relu2 at
 * M = 1 in one launch; arguments as tq_quant_gemv and tq_gate_up_relu2.
 */
TQ_API tq_status tq_quant_gate_up_relu2(const void *x, tq_dtype xt,
                                        const uint8_t *packed_gate,
                                        float s_gate, const uint8_t *packed_up,
                                        float s_up, int64_t N, int64_t K,
                                        float *h, int32_t *acc_gate,
                                        int32_t *acc_up, int8_t *xq,
                                        float *x_scale, const float *y_scale,
                                        hipStream_t stream);

/*
 * tq_quant_gemv_group -- `count` ternary GEMVs that read the same raw
 * activation row, in one launch: tq_quant_gemv for each matrix, with one
 * shared quantization (the q, k and v projections of an attention layer,
 * whose inputs are the same normalized hidden state; [ISSUE] "Weight
 * mapping": q_proj [2560,2560], k_proj and v_proj [640,2560]).
 *   count    1..4.
 *   packed, w_scale, N, y, acc: HOST arrays of `count` entries (the one
 *            exception to the device-memory rule): matrix i is packed[i]
 *            (uint8 [N[i]/4,K], device, 16-B aligned) with scale w_scale[i],
 *            writing y[i] (fp32 [N[i]], device) and, when acc is non-NULL
 *            and acc[i] non-NULL, acc[i] (int32 [N[i]], device).
 *   x, xt, K, xq, x_scale, y_scale: as tq_quant_gemv (all matrices share K
 *            and the activation scale).
 * Every y[i] is bit-identical to tq_quant_gemv on matrix i alone.  Matrices
 * with N[i] == 0 are skipped.  The host arrays are read before the call
 * returns and may be reused at once.
 */
TQ_API tq_status tq_quant_gemv_group(const void *x, tq_dtype xt, int32_t count,
                                     const uint8_t *const *packed,
                                     const float *w_scale, const int64_t *N,
                                     int64_t K, float *const *y,
                                     int32_t *const *acc, int8_t *xq,
                                     float *x_scale, const float *y_scale,
                                     hipStream_t stream);

/*
 * tq_ternarize -- bf16 weights -> packed ternary codes and the weight scale,
 * by the absmean rule (the step before the GEMV for checkpoints that come as
 * pre-dequantized bf16: [ISSUE] "Architecture"; absmean quantization is
 * named on the "1bit.systems" README, "read more").  The pages give no
 * formula; this library's reading:
 *   s' = max(RN32(mean_{n,k} |w[n,k]|), 1e-5)  -- the sum is exact, rounded
 *        once, so the result does not depend on summation order;
 *   c  = clamp(rne(RN32(w * RN32(1/s'))), -1, 1), packed as tq_pack does.
 *   w          bf16 [N,K] device, 16-B aligned; finite values.
 *   packed     uint8 [N/4,K] device output, 16-B aligned.
 *   w_scale    fp32 [1] device output: s' (pass it by value to the GEMV calls
 *              after reading it back once).
 *   workspace  device scratch of at least TQ_TERNARIZE_WORKSPACE_BYTES bytes,
 *              8-B aligned, any contents; the call clears what it uses.  Calls
 *              that overlap in time must not share one workspace.
 * N % 4 == 0, K % 16 == 0, N*K <= 2^31 - 1.  With N*K == 0 only w_scale is
 * written (1e-5).  Four launches (clear, exact |w| histogram, final
 * rounding, quantize + pack).
 */
#define TQ_TERNARIZE_WORKSPACE_BYTES 4096
TQ_API tq_status tq_ternarize(const void *w, int64_t N, int64_t K,
                              uint8_t *packed, float *w_scale, void *workspace,
                              hipStream_t stream);

/*
 * tq_attn_decode -- attention of one query token over a KV cache, split
 * over the cache (flash-decoding; [README] "honest numbers" names split-KV
 * Flash-Decoding at L = 2048; [ISSUE] "Weight mapping": 20 query heads,
 * 5 KV heads, head_dim 128).  The pages give no formula; this library's:
 *   s[h,t] = scale * sum_d q[h,d] k[t,g,d],   g = h / (H/Hkv)
 *   out[h,:] = sum_t softmax_t(s[h,:]) v[t,g,:]
 * Scores, weights and the sums over a chunk of tokens are fp32 (the bf16
 * inputs widen exactly); the chunks are merged in fp64 and the result is
 * rounded once to fp32.  Summation orders are fixed, so identical calls give
 * identical bits.
 *   q          fp32 [H, D] device, 16-B aligned.
 *   k_cache, v_cache  bf16 [L, Hkv, D] device (token-major), 16-B aligned.
 *   out        fp32 [H, D] device output.
 *   workspace  device memory of workspace_bytes >=
 *              TQ_ATTN_WORKSPACE_BYTES(H, D, L) bytes, 16-B aligned, any
 *              contents (per-chunk partial results).  Calls that overlap in
 *              time must not share one workspace.
 * H % Hkv == 0 with H/Hkv in {1, 2, 4, 8}; D in {64, 128};
 * 1 <= L <= TQ_ATTN_MAX_L; a workspace below the size is TQ_ERR_SHAPE.  Two
 * launches (chunk pass, combine); one when L fits in one chunk.
 */
#define TQ_ATTN_MAX_L 131072
#define TQ_ATTN_WORKSPACE_BYTES(H, D, L) \
  ((size_t)(H) * (((size_t)(L) + 63u) / 64u) * ((size_t)(D) + 4u) * 4u)
TQ_API tq_status tq_attn_decode(const float *q, const void *k_cache,
                                const void *v_cache, int64_t H, int64_t Hkv,
                                int64_t D, int64_t L, float scale, float *out,
                                void *workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * tq_attn_decode_noalloc -- tq_attn_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): no workspace argument, and the call
 * allocates nothing.  The per-chunk partials live in a fixed device array
 * of TQ_ATTN_NOALLOC_SCRATCH_BYTES inside the library (one copy per GPU,
 * held until the process ends; its address is looked up once per device on
 * the first call there).  Same kernels, so the output is bit-identical to
 * tq_attn_decode's.
 *   q, k_cache, v_cache, H, Hkv, D, L, scale, out: as tq_attn_decode.
 *   H  1..TQ_ATTN_NOALLOC_MAX_H (larger H: TQ_ERR_SHAPE, nothing launched).
 * Every call on one GPU shares that GPU's array: calls that may overlap in
 * time on one GPU (different streams, other threads) race and must not be
 * issued; calls in order on one stream are safe.
 */
#define TQ_ATTN_NOALLOC_MAX_H 64
#define TQ_ATTN_NOALLOC_SCRATCH_BYTES \
  ((size_t)TQ_ATTN_NOALLOC_MAX_H * 64u * (128u + 4u) * 4u)
TQ_API tq_status tq_attn_decode_noalloc(const float *q, const void *k_cache,
                                        const void *v_cache, int64_t H,
                                        int64_t Hkv, int64_t D, int64_t L,
                                        float scale, float *out,
                                        hipStream_t stream);

/*
 * tq_stream_read -- measurement helper: the practical HBM read ceiling that
 * the GEMV's weight stream is compared with ([ARC] TL;DR and [README]
 * "hardware": a GEMV is judged by the fraction of memory bandwidth it
 * reaches).  Reads `bytes` of `buf` with the GEMV's access (16-byte
 * non-temporal loads, consecutive lanes on consecutive pieces) and does
 * nothing else.
 *   buf         device, 16-B aligned; bytes % 16 == 0 (bytes == 0: no-op).
 *   sink        device, 16-B aligned, `sink_words` 16-byte words.  Block b
 *               writes word b: the XOR of the 16-byte words it read, so the
 *               XOR of the written words equals the XOR of every 16-byte
 *               word of buf; at most min(sink_words, 8 x CUs) words are
 *               written, the rest are left as they were.
 * Errors: TQ_ERR_SHAPE (bytes < 0, bytes % 16, sink_words < 1), TQ_ERR_NULL,
 * TQ_ERR_ALIGN, TQ_ERR_DEVICE, TQ_ERR_LAUNCH.
 */
TQ_API tq_status tq_stream_read(const void *buf, int64_t bytes, void *sink,
                                int64_t sink_words, hipStream_t stream);

/* Static, human-readable text for a status code. */
TQ_API const char *tq_status_string(tq_status status);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
