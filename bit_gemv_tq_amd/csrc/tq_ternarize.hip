// tq_ternarize.hip -- tq_ternarize: bf16 weights [N,K] -> packed ternary
// codes [N/4,K] and the per-tensor weight scale, by the absmean rule.
//
// Page "1bit.systems" project README, section "read more": the project's
// training runs use absmean quantization-aware training.  Page "Feature
// request: BitNet 1.58-bit ternary inference on ROCm (gfx1151)", section
// "Architecture": checkpoints come as packed uint8 or as pre-dequantized
// bf16; the latter need this step before the GEMV.  The pages give no
// formula; this library's reading, with every decision exact:
//   s   = RN32(mean |w|)  (the sum over all N*K weights is exact, then one
//         rounding: the result does not depend on summation order)
//   s'  = max(s, 1e-5)    (the weight scale written out)
//   inv = RN32(1 / s')
//   c   = clamp(rne(RN32(w * inv)), -1, 1), packed as tq_pack does.
//
// Exact sum: |w| = M * 2^(max(e,1) - 134) for the 8-bit exponent field e
// and the significand M (hidden bit included for e >= 1).  Integer sums per
// exponent (so any order gives the same totals) are built per block, in
// registers for the common exponents and in LDS for the rest, and merged
// with 64-bit global atomics; a tree of 384-bit integers then combines them
// and one thread divides by N*K and rounds once.
#include "tq_device.h"
#include "tq_host.h"

namespace tq {
namespace {

constexpr int kWsInvOffset = 2048;  // workspace: u64 bucket[256], then inv
constexpr int kWindow = 24;         // binades below a block's top exponent
                                    // summed in per-thread registers

__global__ __launch_bounds__(256) void ws_clear_kernel(unsigned long long *ws) {
  ws[threadIdx.x] = 0ull;  // 256 buckets (and the 2 KB that follow are
                           // written before they are read)
}

// bucket[e] receives integers B with sum|w| = sum_e B[e] * 2^(max(e,1)-134).
// Weights with exponent field e in [R - kWindow, R] (R: the largest exponent
// among the block's first loads) are summed exactly in a 64-bit register as
// M << (e - (R - kWindow)) and enter bucket[R - kWindow] once per thread
// (M < 2^8, shift <= 24: a term is < 2^32, so a thread's sum and any
// bucket over <= 2^31 weights stay < 2^63).  The rest (rare for real
// weights) go to an LDS histogram of significand sums.
__global__ __launch_bounds__(256) void absmean_hist_kernel(
    const u32x4 *__restrict__ w, int64_t pieces, unsigned long long *bucket) {
  __shared__ unsigned long long h64[256];
  __shared__ unsigned h32[256];
  __shared__ unsigned top_lds[256 / kWave];
  h64[threadIdx.x] = 0ull;
  h32[threadIdx.x] = 0u;
  const int64_t first = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  unsigned emax = 0;
  if (first < pieces) {
    const u32x4 v = w[first];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const unsigned e0 = (v[d] >> 7) & 0xffu, e1 = (v[d] >> 23) & 0xffu;
      emax = max(emax, max(e0, e1));
    }
  }
  for (int off = 32; off >= 1; off >>= 1) emax = max(emax, (unsigned)__shfl_xor((int)emax, off, kWave));
  if ((threadIdx.x & (kWave - 1)) == 0) top_lds[threadIdx.x / kWave] = emax;
  __syncthreads();
  unsigned R = top_lds[0];
#pragma unroll
  for (int i = 1; i < 256 / kWave; ++i) R = max(R, top_lds[i]);
  // Window only over normal exponents (R - kWindow >= 1 keeps the scaling
  // of bucket[R - kWindow] the plain 2^(e-134)).
  const unsigned lo = R > kWindow ? R - kWindow : 256u;  // 256: no window
  unsigned long long acc = 0ull;
  auto add_piece = [&](const u32x4 &v) {  // 8 bf16
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t b = (v[d] >> (16 * h)) & 0xffffu;
        const uint32_t e = (b >> 7) & 0xffu;
        const uint32_t m = (b & 0x7fu) | (e ? 0x80u : 0u);
        if (e >= lo && e <= R) {
          acc += (unsigned long long)m << (e - lo);
        } else if (m) {
          atomicAdd(&h32[e], m);  // < 2^32: at most 2^24 weights per block
        }
      }
  };
  for (int64_t p = first; p < pieces; p += stride) add_piece(w[p]);
  if (acc) atomicAdd(&h64[lo], acc);
  __syncthreads();
  const unsigned long long total = h64[threadIdx.x] + h32[threadIdx.x];
  if (total) atomicAdd(&bucket[threadIdx.x], total);
}

constexpr int kLimbs = 12;  // 384-bit integers

// Final rounding.  T' = sum_e bucket[e] * 2^(max(e,1) - 1 + 64), so that
// sum|w| = T' * 2^-197; bucket < 2^63 and the shift <= 317 give T' < 2^381.
// Every thread turns one bucket into a 12-limb integer, a tree in LDS sums
// them, and thread 0 divides by the count and rounds once.
__global__ __launch_bounds__(256) void absmean_final_kernel(
    const unsigned long long *bucket, uint32_t count, float *w_scale,
    float *inv_out) {
  __shared__ uint32_t limbs[256][kLimbs + 1];  // +1: bank spread
  {
    uint32_t *t = limbs[threadIdx.x];
#pragma unroll
    for (int i = 0; i < kLimbs; ++i) t[i] = 0u;
    const int e = threadIdx.x;
    const uint64_t b = e < 255 ? bucket[e] : 0ull;  // 255: Inf/NaN, outside
    if (b) {
      const int sh = (e > 0 ? e : 1) - 1 + 64;
      const int limb = sh >> 5, bit = sh & 31;
      // b << bit spans three limbs (b < 2^63, bit < 32).
      const uint64_t lo = (uint64_t)(uint32_t)b << bit;
      const uint64_t hi = (uint64_t)(uint32_t)(b >> 32) << bit;
      const uint64_t mid = (lo >> 32) + (hi & 0xffffffffull);
      t[limb] = (uint32_t)lo;
      t[limb + 1] = (uint32_t)mid;
      t[limb + 2] = (uint32_t)((hi >> 32) + (mid >> 32));
    }
  }
  __syncthreads();
  for (int half = 128; half >= 1; half >>= 1) {
    if ((int)threadIdx.x < half) {
      uint32_t *a = limbs[threadIdx.x];
      const uint32_t *c = limbs[threadIdx.x + half];
      uint64_t carry = 0;
#pragma unroll
      for (int i = 0; i < kLimbs; ++i) {
        const uint64_t s = (uint64_t)a[i] + c[i] + carry;
        a[i] = (uint32_t)s;
        carry = s >> 32;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x != 0) return;
  const uint32_t *t = limbs[0];
  float s = 0.0f;
  if (count > 0) {
    // q = floor(T' / count), rem = T' mod count.
    uint32_t q[kLimbs];
    uint64_t rem = 0;
#pragma unroll
    for (int i = kLimbs - 1; i >= 0; --i) {
      const uint64_t cur = (rem << 32) | t[i];
      q[i] = (uint32_t)(cur / count);
      rem = cur % count;
    }
    int top_limb = kLimbs - 1;
    while (top_limb >= 0 && q[top_limb] == 0u) --top_limb;
    if (top_limb >= 0) {
      // q >= 2^64 / 2^31 whenever T' > 0, so it has >= 34 significant bits.
      const int nbits = 32 * top_limb + (32 - __builtin_clz(q[top_limb]));
      int e2 = nbits - 1 - 197;  // mean in [2^e2, 2^(e2+1))
      if (e2 >= -126) {          // below that the 1e-5 floor applies anyway
        auto bit_at = [&](int pos) { return (q[pos >> 5] >> (pos & 31)) & 1u; };
        const int shift = nbits - 24;
        uint32_t top = 0;
        for (int k = 23; k >= 0; --k) top = (top << 1) | bit_at(shift + k);
        const uint32_t round = bit_at(shift - 1);
        // sticky: any set bit below position shift - 1, or a remainder
        bool sticky = rem != 0;
        const int below = shift - 1;  // bits [0, below) of q
        for (int i = 0; i < kLimbs && 32 * i < below; ++i) {
          const int nb = below - 32 * i;
          const uint32_t mask = nb >= 32 ? 0xffffffffu : ((1u << nb) - 1u);
          sticky |= (q[i] & mask) != 0u;
        }
        if (round && (sticky || (top & 1u))) ++top;
        if (top == (1u << 24)) {
          top >>= 1;
          ++e2;
        }
        s = ldexpf((float)top, e2 - 23);  // exact: top < 2^24, normal range
      }
    }
  }
  const float sp = s > 1e-5f ? s : 1e-5f;
  w_scale[0] = sp;
  inv_out[0] = 1.0f / sp;  // correctly rounded fp32 division
}

// Ternary code + 1 (0, 1, 2) of one bf16 weight: rne(y) >= 1 exactly when
// y > 0.5 (0.5 itself is a tie that rounds to 0), and <= -1 when y < -0.5.
__device__ __forceinline__ uint32_t ternary_code(uint32_t bf16, float inv) {
  const float y = __uint_as_float(bf16 << 16) * inv;
  return 1u + (y > 0.5f ? 1u : 0u) - (y < -0.5f ? 1u : 0u);
}

// One thread per 16-byte packed piece: 16 k of the 4 rows i + j*N/4.
__global__ __launch_bounds__(256) void ternary_pack_kernel(
    const u32x4 *__restrict__ w, int64_t n4, int64_t kp,
    const float *__restrict__ inv_p, u32x4 *__restrict__ packed) {
  const float inv = inv_p[0];
  const int64_t total = n4 * kp;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t base = 2 * (t + j * total);  // 16-B units of bf16 rows
      const u32x4 r[2] = {w[base], w[base + 1]};
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const uint32_t b = (r[k / 8][(k % 8) / 2] >> (16 * (k % 2))) & 0xffffu;
        out[k / 4] |= ternary_code(b, inv) << (8 * (k % 4) + 2 * j);
      }
    }
    packed[t] = u32x4{out[0], out[1], out[2], out[3]};
  }
}

}  // namespace
}  // namespace tq

extern "C" tq_status tq_ternarize(const void *w, int64_t N, int64_t K,
                                  uint8_t *packed, float *w_scale,
                                  void *workspace, hipStream_t stream) {
  using namespace tq;
  if (N < 0 || K < 0 || N % 4 != 0 || K % 16 != 0) return TQ_ERR_SHAPE;
  if (K > 0 && N > (int64_t)INT32_MAX / K) return TQ_ERR_SHAPE;
  const int64_t count = N * K;
  if (!w_scale || !workspace || (count > 0 && (!w || !packed))) return TQ_ERR_NULL;
  if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(w_scale, 4) ||
      !aligned(workspace, 8))
    return TQ_ERR_ALIGN;
  DeviceInfo dev;
  if (tq_status s = current_device(&dev)) return s;
  auto *ws = static_cast<unsigned long long *>(workspace);
  auto *inv = reinterpret_cast<float *>(static_cast<char *>(workspace) + kWsInvOffset);
  if (tq_status s = launch(ws_clear_kernel, dim3(1), dim3(256), 0, stream, ws)) return s;
  if (count > 0) {
    const int64_t pieces = count / 8;
    // >= pieces / 2^21 blocks keeps every block at <= 2^24 elements.
    int64_t blocks = (pieces + 255) / 256;
    const int64_t cap = (int64_t)dev.num_cus * 8;
    const int64_t need = (pieces + (1 << 21) - 1) >> 21;
    if (blocks > cap) blocks = cap > need ? cap : need;
    if (tq_status s = launch(absmean_hist_kernel, dim3((unsigned)blocks), dim3(256), 0,
                             stream, static_cast<const u32x4 *>(w), pieces, ws))
      return s;
  }
  if (tq_status s = launch(absmean_final_kernel, dim3(1), dim3(256), 0, stream,
                           static_cast<const unsigned long long *>(ws),
                           (uint32_t)count, w_scale, inv))
    return s;
  if (count == 0) return TQ_OK;
  const int64_t n4 = N / 4, kp = K / 16;
  int64_t blocks = (n4 * kp + 255) / 256;
  const int64_t cap = (int64_t)dev.num_cus * 16;
  if (blocks > cap) blocks = cap;
  return launch(ternary_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                static_cast<const u32x4 *>(w), n4, kp, static_cast<const float *>(inv),
                reinterpret_cast<u32x4 *>(packed));
}
