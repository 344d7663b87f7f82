// tq_attn.hip -- tq_attn_decode: split-KV (flash-decoding) attention for one
// query token over a bf16 KV cache, grouped-query heads.
//
// Page "1bit.systems" project README, section "honest numbers": split-KV
// Flash-Decoding attention at L = 2048.  Page "Feature request: BitNet 1.58-
// bit ternary inference on ROCm (gfx1151)", section "Weight mapping": 20
// query heads, 5 KV heads, head_dim 128.  The pages give no formula or
// precision; this library computes
//   s[h,t] = scale * sum_d q[h,d] k[t,g,d],  g = h / (H/Hkv)
//   o[h,:] = sum_t softmax_t(s[h,:]) v[t,g,:]
// in fp32 (bf16 inputs widen exactly; fp32 FMAs, expf) within each split,
// and merges the splits in fp64.  Every summation order is fixed (no
// atomics), so identical calls give identical bits.  The op streams the KV
// cache once: HBM bound at long contexts.
//
// Split pass: block (g, c) handles the G query heads of KV head g over the
// token chunk c.  A token row of one KV head (D bf16 = 2D bytes) is read by
// LPT = D/8 consecutive lanes, 16 bytes each; a lane slot takes kT tokens per
// step, so each lane has kT row loads in flight.  The kT*G partial dots of a
// slot are summed by a reduce-scatter butterfly over its LPT lanes.  Scores,
// then weights, live in LDS; the chunk's max, exp-sum and unnormalized
// output per head go to the workspace.  Combine pass: one block per query
// head merges the chunks in order.
#include <math.h>

#include "tq_device.h"
#include "tq_host.h"

namespace tq {
namespace {

constexpr int kAttnThreads = 256;
constexpr int kAttnMaxSplits = 64;
constexpr int kAttnMaxChunk = 2048;

// Workspace layout (fp64): for split c of head h: m, l, then D values of o.
__host__ __device__ inline size_t ws_index(int h, int c, int D) {
  return ((size_t)h * kAttnMaxSplits + c) * (size_t)(D + 2);
}

__device__ __forceinline__ void widen8(const u32x4 &r, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(r[i] << 16);
    x[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
  }
}

// One halving step of the reduce-scatter (and the steps after it), with
// compile-time offsets and widths so every register index is a constant:
// lanes whose bit OFF is set keep the upper half of their first W values,
// the others the lower half, each adding its partner's copy of that half.
template <int OFF, int W, int N>
__device__ __forceinline__ void reduce_scatter(float (&val)[N], int lt) {
  if constexpr (OFF >= 1) {
    const bool upper = (lt & OFF) != 0;
#pragma unroll
    for (int k = 0; k < W / 2; ++k) {
      const float send = upper ? val[k] : val[k + W / 2];
      const float keep = upper ? val[k + W / 2] : val[k];
      val[k] = keep + __shfl_xor(send, OFF, kWave);
    }
    reduce_scatter<OFF / 2, W / 2>(val, lt);
  }
}

template <int G, int D>
__global__ __launch_bounds__(kAttnThreads) void attn_split_kernel(
    const float *__restrict__ q, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, int Hkv, int L, int chunk, float scale,
    double *__restrict__ ws) {
  constexpr int LPT = D / 8;             // lanes per token row
  constexpr int TPW = kWave / LPT;       // token slots per wave
  constexpr int NW = kAttnThreads / kWave;
  constexpr int TPB = NW * TPW;          // token slots per block
  // kT tokens per slot per step: at least LPT/G (every lane ends with a
  // complete sum), 8 otherwise, at most 32/G partial dots (registers).
  constexpr int kTcap = 32 / G < 8 ? 32 / G : 8;
  constexpr int kT = LPT / G > kTcap ? LPT / G : kTcap;
  constexpr int NV = kT * G;             // partial dots per lane
  constexpr int VPL = NV / LPT;          // complete sums per lane at the end
  static_assert(NV % LPT == 0 && VPL >= 1, "butterfly shape");
  // Dynamic LDS: [G][chunk] scores, then weights; after the P.V loop the
  // same space holds the per-wave outputs [NW][G][D].
  extern __shared__ float s_lds[];
  __shared__ float red[NW][G];

  const int g = blockIdx.x, c = blockIdx.y;
  const int t0 = c * chunk, t1 = min(t0 + chunk, L);
  const int n = t1 - t0;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int lt = lane % LPT;            // piece of the row (8 dims)
  const int tw = lane / LPT;            // token slot within the wave

  float qd[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float4 *qp = reinterpret_cast<const float4 *>(q + (size_t)(g * G + j) * D + lt * 8);
    const float4 a = qp[0], b = qp[1];
    qd[j][0] = a.x; qd[j][1] = a.y; qd[j][2] = a.z; qd[j][3] = a.w;
    qd[j][4] = b.x; qd[j][5] = b.y; qd[j][6] = b.z; qd[j][7] = b.w;
  }
  auto row = [&](const uint16_t *base, int t) {
    return *reinterpret_cast<const u32x4 *>(base + ((size_t)t * Hkv + g) * D + lt * 8);
  };

  // 1. scores: token i = it + u*TPW + tw for u < kT (it advancing by TPB*kT)
  for (int it = wave * TPW * kT; it < n; it += TPB * kT) {
    u32x4 r[kT];
#pragma unroll
    for (int u = 0; u < kT; ++u) {
      const int i = it + u * TPW + tw;
      r[u] = row(kc, t0 + (i < n ? i : 0));  // past the chunk: an in-chunk row
    }
    float val[NV];
#pragma unroll
    for (int u = 0; u < kT; ++u) {
      float x[8];
      widen8(r[u], x);
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float dsum = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) dsum = fmaf(qd[j][e], x[e], dsum);
        val[u * G + j] = dsum;
      }
    }
    // reduce-scatter: after the step with offset `off` a lane keeps the half
    // of its values selected by its bit `off`; lane lt ends with the complete
    // sums of values v = VPL*lt + b (v = u*G + j)
    reduce_scatter<LPT / 2, NV>(val, lt);
#pragma unroll
    for (int b = 0; b < VPL; ++b) {
      const int v = VPL * lt + b;
      const int u = v / G, j = v % G;
      const int i = it + u * TPW + tw;
      if (i < n) s_lds[j * chunk + i] = val[b] * scale;
    }
  }
  __syncthreads();

  // 2. per-head max and exp-sum over the chunk (fixed reduction order)
  float mx[G], sum[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float m = -INFINITY;
    for (int i = threadIdx.x; i < n; i += kAttnThreads) m = fmaxf(m, s_lds[j * chunk + i]);
    for (int off = kWave / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    if (lane == 0) red[wave][j] = m;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < G; ++j) {
    mx[j] = red[0][j];
#pragma unroll
    for (int w = 1; w < NW; ++w) mx[j] = fmaxf(mx[j], red[w][j]);
  }
  __syncthreads();  // red is reused below
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float sacc = 0.0f;
    for (int i = threadIdx.x; i < n; i += kAttnThreads) {
      const float p = expf(s_lds[j * chunk + i] - mx[j]);
      s_lds[j * chunk + i] = p;
      sacc += p;
    }
    for (int off = kWave / 2; off >= 1; off >>= 1) sacc += __shfl_xor(sacc, off, kWave);
    if (lane == 0) red[wave][j] = sacc;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < G; ++j) {
    sum[j] = red[0][j];
#pragma unroll
    for (int w = 1; w < NW; ++w) sum[j] += red[w][j];
  }

  // 3. unnormalized output sum_t p[t] v[t] over the chunk, kT rows in flight
  float acc[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.0f;
  for (int it = wave * TPW * kT; it < n; it += TPB * kT) {
    u32x4 r[kT];
#pragma unroll
    for (int u = 0; u < kT; ++u) {
      const int i = it + u * TPW + tw;
      r[u] = row(vc, t0 + (i < n ? i : 0));
    }
#pragma unroll
    for (int u = 0; u < kT; ++u) {
      const int i = it + u * TPW + tw;
      if (i < n) {
        float x[8];
        widen8(r[u], x);
#pragma unroll
        for (int j = 0; j < G; ++j) {
          const float p = s_lds[j * chunk + i];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[j][e] = fmaf(p, x[e], acc[j][e]);
        }
      }
    }
  }
  // token slots of a wave (lanes LPT apart), then the waves, in order
#pragma unroll
  for (int off = LPT; off < kWave; off <<= 1)
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] += __shfl_xor(acc[j][e], off, kWave);
  __syncthreads();  // every wave is done reading the weights
  float *o_red = s_lds;  // [NW][G][D]
  if (tw == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) o_red[(wave * G + j) * D + lt * 8 + e] = acc[j][e];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += kAttnThreads) {
    const int j = idx / D, d = idx % D;
    float o = o_red[j * D + d];
#pragma unroll
    for (int w = 1; w < NW; ++w) o += o_red[(w * G + j) * D + d];
    ws[ws_index(g * G + j, c, D) + 2 + d] = (double)o;
  }
  if (threadIdx.x < G) {
    const int j = threadIdx.x;
    ws[ws_index(g * G + j, c, D)] = (double)mx[j];
    ws[ws_index(g * G + j, c, D) + 1] = (double)sum[j];
  }
}

// One block per query head: merge the splits in order, round once.  The
// per-split maxima and weights are loaded in parallel and staged in LDS; the
// output sums keep 8 loads in flight per thread.
constexpr int kCombineThreads = 128;

__global__ __launch_bounds__(kCombineThreads) void attn_combine_kernel(
    const double *__restrict__ ws, int splits, int D, float *__restrict__ out) {
  __shared__ double f[kAttnMaxSplits];   // exp(m_c - M)
  __shared__ double ls[kAttnMaxSplits];  // l_c
  __shared__ double wmax[kCombineThreads / kWave];
  __shared__ double den_s;
  const int h = blockIdx.x;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int c = threadIdx.x;
  const double m = c < splits ? ws[ws_index(h, c, D)] : -INFINITY;
  const double l = c < splits ? ws[ws_index(h, c, D) + 1] : 0.0;
  double M = m;
  for (int off = kWave / 2; off >= 1; off >>= 1) M = fmax(M, __shfl_xor(M, off, kWave));
  if (lane == 0) wmax[wave] = M;
  __syncthreads();
  M = wmax[0];
#pragma unroll
  for (int w = 1; w < kCombineThreads / kWave; ++w) M = fmax(M, wmax[w]);
  if (c < kAttnMaxSplits) {  // splits past the end weigh exactly 0
    f[c] = c < splits ? exp(m - M) : 0.0;
    ls[c] = l;
  }
  __syncthreads();
  if (c == 0) {  // fixed order
    double den = 0.0;
    for (int i = 0; i < splits; ++i) den = fma(f[i], ls[i], den);
    den_s = den;
  }
  __syncthreads();
  const double den = den_s;
  for (int d = threadIdx.x; d < D; d += kCombineThreads) {
    // splits summed in order, kUnroll loads issued per round
    constexpr int kUnroll = 8;  // loads in flight per thread
    double num = 0.0;
    for (int i0 = 0; i0 < splits; i0 += kUnroll) {
      double o[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)  // past the end: weight 0, valid row
        o[u] = ws[ws_index(h, min(i0 + u, splits - 1), D) + 2 + d];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        num = fma(i0 + u < kAttnMaxSplits ? f[i0 + u] : 0.0, o[u], num);
    }
    out[(size_t)h * D + d] = (float)(num / den);
  }
}

template <int G, int D>
tq_status launch_attn(const float *q, const void *k, const void *v, int H,
                      int Hkv, int L, float scale, float *out, double *ws,
                      hipStream_t s) {
  // Chunks: about kAttnMaxSplits per KV head (enough blocks to spread the
  // cache over every CU), a multiple of the tokens a block steps by.
  constexpr int TPB = (kAttnThreads / kWave) * (kWave / (D / 8));
  int chunk = (L + kAttnMaxSplits - 1) / kAttnMaxSplits;
  chunk = (chunk + TPB - 1) / TPB * TPB;  // whole block steps
  if (chunk > kAttnMaxChunk) return TQ_ERR_SHAPE;  // excluded by the caller
  const int splits = (L + chunk - 1) / chunk;
  constexpr int kOutFloats = (kAttnThreads / kWave) * G * D;
  const size_t lds = (size_t)(G * chunk > kOutFloats ? G * chunk : kOutFloats) *
                     sizeof(float);
  if (tq_status st = allow_dynamic_lds((const void *)attn_split_kernel<G, D>, (int)lds))
    return st;
  if (tq_status st = launch(attn_split_kernel<G, D>, dim3(Hkv, splits),
                            dim3(kAttnThreads), lds, s, q,
                            static_cast<const uint16_t *>(k),
                            static_cast<const uint16_t *>(v), Hkv, L, chunk,
                            scale, ws))
    return st;
  return launch(attn_combine_kernel, dim3(H), dim3(kCombineThreads), 0, s,
                static_cast<const double *>(ws), splits, D, out);
}

template <int D>
tq_status launch_attn_d(int G, const float *q, const void *k, const void *v,
                        int H, int Hkv, int L, float scale, float *out,
                        double *ws, hipStream_t s) {
  switch (G) {
    case 1: return launch_attn<1, D>(q, k, v, H, Hkv, L, scale, out, ws, s);
    case 2: return launch_attn<2, D>(q, k, v, H, Hkv, L, scale, out, ws, s);
    case 4: return launch_attn<4, D>(q, k, v, H, Hkv, L, scale, out, ws, s);
    case 8: return launch_attn<8, D>(q, k, v, H, Hkv, L, scale, out, ws, s);
  }
  return TQ_ERR_SHAPE;
}

}  // namespace
}  // namespace tq

extern "C" tq_status tq_attn_decode(const float *q, const void *k_cache,
                                    const void *v_cache, int64_t H, int64_t Hkv,
                                    int64_t D, int64_t L, float scale,
                                    float *out, void *workspace,
                                    hipStream_t stream) {
  using namespace tq;
  if (H < 1 || Hkv < 1 || H % Hkv != 0 || H > 256) return TQ_ERR_SHAPE;
  const int64_t G = H / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return TQ_ERR_SHAPE;
  if (D != 64 && D != 128) return TQ_ERR_SHAPE;
  if (L < 1 || L > (int64_t)kAttnMaxSplits * kAttnMaxChunk) return TQ_ERR_SHAPE;
  if (!q || !k_cache || !v_cache || !out || !workspace) return TQ_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(out, 4) || !aligned(workspace, 8))
    return TQ_ERR_ALIGN;
  DeviceInfo dev;
  if (tq_status s = current_device(&dev)) return s;
  auto *ws = static_cast<double *>(workspace);
  return D == 128 ? launch_attn_d<128>((int)G, q, k_cache, v_cache, (int)H, (int)Hkv,
                                       (int)L, scale, out, ws, stream)
                  : launch_attn_d<64>((int)G, q, k_cache, v_cache, (int)H, (int)Hkv,
                                      (int)L, scale, out, ws, stream);
}
