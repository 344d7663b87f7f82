// tq_act_quant.hip -- tq_act_quant: per-token absmax int8 quantization.
//
// Per row m: a = max|x|, a' = max(a, 1e-5), inv = 127/a' (fp32, correctly
// rounded), q = clamp(rne(x*inv), -127, 127), s_x = a'/127.  The pages do
// not describe activation quantization; this is the library's convention
// (one correctly rounded divide per row, round half to even, symmetric
// clamp), applied identically wherever an fp32 value decides an int8 code.
// The clamp never binds (quant4 in tq_device.h gives the bound).
//
// tq_rmsnorm_act_quant: the same with the sub-layer RMSNorm folded in (page
// "Feature request: BitNet 1.58-bit ternary inference on ROCm (gfx1151)",
// section "Architecture": norms before o_proj and down_proj).  The codes are
// those of u = x * gamma (fp32 products) and s_x = (a'/127) * r with
// r = 1/sqrt(mean(x^2) + eps), formed in fp64 and rounded once: absmax
// quantization gives the same codes for any positive multiple of a row, so
// the RMS factor is carried in the scale.
#include "tq_device.h"
#include "tq_host.h"

namespace tq {
namespace {

constexpr int kAqThreads = 512;

struct RmsArgs {
  const void *gamma;  // [K], dtype of x (kRms only)
  float eps;
};

// Block-wide fp64 sum in a fixed order (waves in order), same in every thread.
template <int kThreads>
__device__ __forceinline__ double block_sum_f64(double v, double *lds) {
  v = wave_sum_f64(v);
  if ((threadIdx.x & (kWave - 1)) == 0) lds[threadIdx.x / kWave] = v;
  __syncthreads();
  double t = lds[0];
#pragma unroll
  for (int w = 1; w < kThreads / kWave; ++w) t += lds[w];
  return t;
}

// Two passes (absmax, then quantize) for rows longer than the register
// kernel holds; one block per activation row.
template <bool kBf16, bool kRms>
__global__ __launch_bounds__(kAqThreads) void act_quant_kernel(
    const void *__restrict__ x, int64_t K, int8_t *__restrict__ q,
    float *__restrict__ s_x, RmsArgs rms) {
  __shared__ float wave_max_lds[kAqThreads / kWave];
  __shared__ double ss_lds[kAqThreads / kWave];
  constexpr bool kQBf16 = kRms ? false : kBf16;  // form of the quantized values
  const int64_t m = blockIdx.x;
  const int64_t kp = K / 16;
  const size_t elem = kBf16 ? 2 : 4;
  const void *xr = reinterpret_cast<const char *>(x) + (size_t)(m * K) * elem;
  auto values = [&](int64_t p, double &ss) {
    if constexpr (kRms)
      return scale_piece<kBf16>(load_piece<kBf16>(xr, p), load_piece<kBf16>(rms.gamma, p), ss);
    else
      return load_piece<kBf16>(xr, p);
  };

  uint32_t mb = 0;
  double ss = 0.0;
  for (int64_t p = threadIdx.x; p < kp; p += kAqThreads)
    mb = absmax_bits<kQBf16>(values(p, ss), mb);
  float a = wave_max(absmax_value<kQBf16>(mb));
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) wave_max_lds[wave] = a;
  float r = 1.0f;
  if constexpr (kRms) r = rms_factor(block_sum_f64<kAqThreads>(ss, ss_lds), K, rms.eps);
  __syncthreads();
  a = wave_max_lds[0];
#pragma unroll
  for (int w = 1; w < kAqThreads / kWave; ++w) a = fmaxf(a, wave_max_lds[w]);

  const float ap = a > 1e-5f ? a : 1e-5f;
  const float inv = 127.0f / ap;  // correctly rounded fp32 division

  u32x4 *qr = reinterpret_cast<u32x4 *>(q + m * K);
  double unused = 0.0;
  for (int64_t p = threadIdx.x; p < kp; p += kAqThreads)
    qr[p] = quant_piece<kQBf16>(values(p, unused), inv);
  if (threadIdx.x == 0) s_x[m] = kRms ? (ap / 127.0f) * r : ap / 127.0f;
}

// Single pass for K <= 32768: each thread keeps its PPT pieces (16 values
// each) in registers between the absmax reduction and the quantization, so
// the row is read once.
constexpr int kAqRegThreads = 1024;

template <bool kBf16, bool kRms, int PPT>
__global__ __launch_bounds__(kAqRegThreads) void act_quant_reg_kernel(
    const void *__restrict__ x, int64_t K, int8_t *__restrict__ q,
    float *__restrict__ s_x, RmsArgs rms) {
  __shared__ float wave_max_lds[kAqRegThreads / kWave];
  __shared__ double ss_lds[kAqRegThreads / kWave];
  constexpr bool kQBf16 = kRms ? false : kBf16;
  const int64_t m = blockIdx.x;
  const int kp = (int)(K / 16);
  const size_t elem = kBf16 ? 2 : 4;
  const void *xr = reinterpret_cast<const char *>(x) + (size_t)(m * K) * elem;
  RawPiece<kQBf16> v[PPT];
  uint32_t mb = 0;
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int p = threadIdx.x + i * kAqRegThreads;
    if (p < kp) {
      if constexpr (kRms)
        v[i] = scale_piece<kBf16>(load_piece<kBf16>(xr, p), load_piece<kBf16>(rms.gamma, p), ss);
      else
        v[i] = load_piece<kBf16>(xr, p);
      mb = absmax_bits<kQBf16>(v[i], mb);
    }
  }
  float a = wave_max(absmax_value<kQBf16>(mb));
  if ((threadIdx.x & (kWave - 1)) == 0) wave_max_lds[threadIdx.x / kWave] = a;
  float r = 1.0f;
  if constexpr (kRms) r = rms_factor(block_sum_f64<kAqRegThreads>(ss, ss_lds), K, rms.eps);
  __syncthreads();
  a = wave_max_lds[0];
#pragma unroll
  for (int w = 1; w < kAqRegThreads / kWave; ++w) a = fmaxf(a, wave_max_lds[w]);

  const float ap = a > 1e-5f ? a : 1e-5f;
  const float inv = 127.0f / ap;  // correctly rounded fp32 division
  u32x4 *qr = reinterpret_cast<u32x4 *>(q + m * K);
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int p = threadIdx.x + i * kAqRegThreads;
    if (p < kp) qr[p] = quant_piece<kQBf16>(v[i], inv);
  }
  if (threadIdx.x == 0) s_x[m] = kRms ? (ap / 127.0f) * r : ap / 127.0f;
}

template <bool kBf16, bool kRms>
tq_status launch_act_quant(const void *x, int64_t M, int64_t K, int8_t *xq,
                           float *x_scale, RmsArgs rms, hipStream_t stream) {
  const int64_t kp = K / 16;
  const dim3 grid((unsigned)M);
  if (kp <= kAqRegThreads)
    return launch(act_quant_reg_kernel<kBf16, kRms, 1>, grid, dim3(kAqRegThreads), 0,
                  stream, x, K, xq, x_scale, rms);
  if (kp <= 2 * kAqRegThreads)
    return launch(act_quant_reg_kernel<kBf16, kRms, 2>, grid, dim3(kAqRegThreads), 0,
                  stream, x, K, xq, x_scale, rms);
  return launch(act_quant_kernel<kBf16, kRms>, grid, dim3(kAqThreads), 0, stream, x,
                K, xq, x_scale, rms);
}

tq_status check_act_quant(const void *x, tq_dtype xt, int64_t M, int64_t K,
                          const int8_t *xq, const float *x_scale) {
  if (xt != TQ_BF16 && xt != TQ_F32) return TQ_ERR_DTYPE;
  if (check_m(M) != TQ_OK || K < 0 || K % 16 != 0 || K > TQ_MAX_K)
    return TQ_ERR_SHAPE;
  if (M == 0) return TQ_OK;
  if (!x_scale || (K > 0 && (!x || !xq))) return TQ_ERR_NULL;
  if (!aligned(x_scale, 4) || !aligned(x, 16) || !aligned(xq, 16))
    return TQ_ERR_ALIGN;
  return TQ_OK;
}

}  // namespace

// Shared with the GEMV entry points' fallbacks (K > 32768).
tq_status rmsnorm_act_quant(const void *x, tq_dtype xt, const void *gamma, float eps,
                            int64_t M, int64_t K, int8_t *xq, float *x_scale,
                            hipStream_t stream) {
  DeviceInfo dev;
  if (tq_status s = current_device(&dev)) return s;
  const RmsArgs rms{gamma, eps};
  return xt == TQ_BF16
             ? launch_act_quant<true, true>(x, M, K, xq, x_scale, rms, stream)
             : launch_act_quant<false, true>(x, M, K, xq, x_scale, rms, stream);
}

// RMSNorm arguments: gamma [K] of the dtype of x, eps > 0 and finite, K > 0.
tq_status check_rms(const void *gamma, float eps, int64_t K) {
  if (K <= 0 || !(eps > 0.0f) || !(eps <= 3.4e38f)) return TQ_ERR_SHAPE;
  if (!gamma) return TQ_ERR_NULL;
  if (!aligned(gamma, 16)) return TQ_ERR_ALIGN;
  return TQ_OK;
}

}  // namespace tq

extern "C" tq_status tq_act_quant(const void *x, tq_dtype xt, int64_t M,
                                  int64_t K, int8_t *xq, float *x_scale,
                                  hipStream_t stream) {
  using namespace tq;
  if (tq_status s = check_act_quant(x, xt, M, K, xq, x_scale)) return s;
  if (M == 0) return TQ_OK;
  DeviceInfo dev;
  if (tq_status s = current_device(&dev)) return s;
  const RmsArgs none{nullptr, 0.0f};
  return xt == TQ_BF16
             ? launch_act_quant<true, false>(x, M, K, xq, x_scale, none, stream)
             : launch_act_quant<false, false>(x, M, K, xq, x_scale, none, stream);
}

extern "C" tq_status tq_rmsnorm_act_quant(const void *x, tq_dtype xt,
                                          const void *gamma, float eps,
                                          int64_t M, int64_t K, int8_t *xq,
                                          float *x_scale, hipStream_t stream) {
  using namespace tq;
  if (tq_status s = check_act_quant(x, xt, M, K, xq, x_scale)) return s;
  if (tq_status s = check_rms(gamma, eps, K)) return s;
  if (M == 0) return TQ_OK;
  return rmsnorm_act_quant(x, xt, gamma, eps, M, K, xq, x_scale, stream);
}
