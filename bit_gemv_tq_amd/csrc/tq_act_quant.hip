// tq_act_quant.hip -- tq_act_quant: per-token absmax int8 quantization.
//
// Per row m: a = max|x|, a' = max(a, 1e-5), inv = 127/a' (fp32, correctly
// rounded), q = clamp(rne(x*inv), -127, 127), s_x = a'/127.  The pages do
// not describe activation quantization; this is the library's convention
// (one correctly rounded divide per row, round half to even, symmetric
// clamp), applied identically wherever an fp32 value decides an int8 code.
// The clamp never binds (quant4 in tq_device.h gives the bound).
#include "tq_device.h"
#include "tq_host.h"

namespace tq {
namespace {

constexpr int kAqThreads = 512;

// Two passes (absmax, then quantize) for rows longer than the register
// kernel holds; one block per activation row.
template <bool kBf16>
__global__ __launch_bounds__(kAqThreads) void act_quant_kernel(
    const void *__restrict__ x, int64_t K, int8_t *__restrict__ q,
    float *__restrict__ s_x) {
  __shared__ float wave_max_lds[kAqThreads / kWave];
  const int64_t m = blockIdx.x;
  const int64_t kp = K / 16;
  const size_t elem = kBf16 ? 2 : 4;
  const void *xr = reinterpret_cast<const char *>(x) + (size_t)(m * K) * elem;

  uint32_t mb = 0;
  for (int64_t p = threadIdx.x; p < kp; p += kAqThreads)
    mb = absmax_bits<kBf16>(load_piece<kBf16>(xr, p), mb);
  float a = wave_max(absmax_value<kBf16>(mb));
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) wave_max_lds[wave] = a;
  __syncthreads();
  a = wave_max_lds[0];
#pragma unroll
  for (int w = 1; w < kAqThreads / kWave; ++w) a = fmaxf(a, wave_max_lds[w]);

  const float ap = a > 1e-5f ? a : 1e-5f;
  const float inv = 127.0f / ap;  // correctly rounded fp32 division

  u32x4 *qr = reinterpret_cast<u32x4 *>(q + m * K);
  for (int64_t p = threadIdx.x; p < kp; p += kAqThreads)
    qr[p] = quant_piece<kBf16>(load_piece<kBf16>(xr, p), inv);
  if (threadIdx.x == 0) s_x[m] = ap / 127.0f;
}

// Single pass for K <= 32768: each thread keeps its PPT pieces (16 values
// each) in registers between the absmax reduction and the quantization, so
// the row is read once.
constexpr int kAqRegThreads = 1024;

template <bool kBf16, int PPT>
__global__ __launch_bounds__(kAqRegThreads) void act_quant_reg_kernel(
    const void *__restrict__ x, int64_t K, int8_t *__restrict__ q,
    float *__restrict__ s_x) {
  __shared__ float wave_max_lds[kAqRegThreads / kWave];
  const int64_t m = blockIdx.x;
  const int kp = (int)(K / 16);
  const size_t elem = kBf16 ? 2 : 4;
  const void *xr = reinterpret_cast<const char *>(x) + (size_t)(m * K) * elem;
  RawPiece<kBf16> v[PPT];
  uint32_t mb = 0;
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int p = threadIdx.x + i * kAqRegThreads;
    if (p < kp) {
      v[i] = load_piece<kBf16>(xr, p);
      mb = absmax_bits<kBf16>(v[i], mb);
    }
  }
  float a = wave_max(absmax_value<kBf16>(mb));
  if ((threadIdx.x & (kWave - 1)) == 0) wave_max_lds[threadIdx.x / kWave] = a;
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
    if (p < kp) qr[p] = quant_piece<kBf16>(v[i], inv);
  }
  if (threadIdx.x == 0) s_x[m] = ap / 127.0f;
}

template <bool kBf16>
tq_status launch_act_quant(const void *x, int64_t M, int64_t K, int8_t *xq,
                           float *x_scale, hipStream_t stream) {
  const int64_t kp = K / 16;
  const dim3 grid((unsigned)M);
  if (kp <= kAqRegThreads)
    return launch(act_quant_reg_kernel<kBf16, 1>, grid, dim3(kAqRegThreads), 0,
                  stream, x, K, xq, x_scale);
  if (kp <= 2 * kAqRegThreads)
    return launch(act_quant_reg_kernel<kBf16, 2>, grid, dim3(kAqRegThreads), 0,
                  stream, x, K, xq, x_scale);
  return launch(act_quant_kernel<kBf16>, grid, dim3(kAqThreads), 0, stream, x,
                K, xq, x_scale);
}

}  // namespace
}  // namespace tq

extern "C" tq_status tq_act_quant(const void *x, tq_dtype xt, int64_t M,
                                  int64_t K, int8_t *xq, float *x_scale,
                                  hipStream_t stream) {
  using namespace tq;
  if (xt != TQ_BF16 && xt != TQ_F32) return TQ_ERR_DTYPE;
  if (check_m(M) != TQ_OK || K < 0 || K % 16 != 0 || K > TQ_MAX_K)
    return TQ_ERR_SHAPE;
  if (M == 0) return TQ_OK;
  if (!x_scale || (K > 0 && (!x || !xq))) return TQ_ERR_NULL;
  if (!aligned(x_scale, 4) || !aligned(x, 16) || !aligned(xq, 16))
    return TQ_ERR_ALIGN;
  DeviceInfo dev;
  if (tq_status s = current_device(&dev)) return s;
  return xt == TQ_BF16
             ? launch_act_quant<true>(x, M, K, xq, x_scale, stream)
             : launch_act_quant<false>(x, M, K, xq, x_scale, stream);
}
