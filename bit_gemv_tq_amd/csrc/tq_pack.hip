// tq_pack.hip -- tq_pack: int8 ternary weights [N,K] -> packed uint8 [N/4,K].
//
// Page "Feature request: BitNet 1.58-bit ternary inference on ROCm
// (gfx1151)", section "Architecture": ternary weights are stored as uint8
// with four values per byte; section "Weight mapping (bitnet-b1.58-2B-4T)":
// a [N,K] projection is held as [N/4,K] uint8.  Code w+1 of row j*(N/4)+i
// goes to bits 2j..2j+1 of byte [i,k] (this library's reading).
#include "tq_device.h"
#include "tq_host.h"

namespace tq {
namespace {

__device__ __forceinline__ uint32_t code_of(uint32_t byte) {
  // int8 -1, 0, +1 -> 0, 1, 2; anything else -> reserved code 3.
  const int v = (int)(int8_t)(byte & 0xffu);
  return (v >= -1 && v <= 1) ? (uint32_t)(v + 1) : 3u;
}

__device__ __forceinline__ uint32_t pack_dword(uint32_t r0, uint32_t r1,
                                               uint32_t r2, uint32_t r3) {
  uint32_t out = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int s = 8 * b;
    const uint32_t byte = code_of(r0 >> s) | (code_of(r1 >> s) << 2) |
                          (code_of(r2 >> s) << 4) | (code_of(r3 >> s) << 6);
    out |= byte << s;
  }
  return out;
}

// One thread per 16-byte piece of the packed array.
__global__ __launch_bounds__(256) void pack_kernel(const uint4 *__restrict__ w,
                                                   int64_t n4, int64_t kp,
                                                   uint4 *__restrict__ packed) {
  const int64_t total = n4 * kp;
  const int64_t plane_stride = n4 * kp;  // pieces between rows i and i + N/4
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const uint4 a = w[t];
    const uint4 b = w[t + plane_stride];
    const uint4 c = w[t + 2 * plane_stride];
    const uint4 d = w[t + 3 * plane_stride];
    uint4 o;
    o.x = pack_dword(a.x, b.x, c.x, d.x);
    o.y = pack_dword(a.y, b.y, c.y, d.y);
    o.z = pack_dword(a.z, b.z, c.z, d.z);
    o.w = pack_dword(a.w, b.w, c.w, d.w);
    packed[t] = o;
  }
}

}  // namespace
}  // namespace tq

extern "C" tq_status tq_pack(const int8_t *w, int64_t N, int64_t K,
                             uint8_t *packed, hipStream_t stream) {
  using namespace tq;
  if (N < 0 || K < 0 || N % 4 != 0 || K % 16 != 0) return TQ_ERR_SHAPE;
  if (N == 0 || K == 0) return TQ_OK;
  if (!w || !packed) return TQ_ERR_NULL;
  if (!aligned(w, 16) || !aligned(packed, 16)) return TQ_ERR_ALIGN;
  DeviceInfo dev;
  if (tq_status s = current_device(&dev)) return s;
  const int64_t n4 = N / 4, kp = K / 16;
  const int64_t total = n4 * kp;
  int64_t blocks = (total + 255) / 256;
  const int64_t cap = (int64_t)dev.num_cus * 16;
  if (blocks > cap) blocks = cap;
  return launch(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                reinterpret_cast<const uint4 *>(w), n4, kp,
                reinterpret_cast<uint4 *>(packed));
}
