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
// in fp32 (bf16 inputs widen exactly; fp32 FMAs, expf) within each chunk of
// tokens, and merges the chunks in fp64.  Every summation order is fixed (no
// atomics), so identical calls give identical bits.  The op streams the KV
// cache once: HBM bound at long contexts.
//
// Chunk pass: block (g, c) of 4 or 8 waves handles the G query heads of KV
// head g over the tokens of chunk c (at most kAttnMaxSplits chunks per KV
// head, fewer where that keeps every CU to one block; plan in
// launch_attn_g), in steps of STEP tokens.  A token row of one KV head (D bf16 = 2D bytes) is read by
// LPT = D/8 consecutive lanes, 16 bytes each; a lane slot takes kT tokens per
// step, and the next step's rows are loaded during this step's arithmetic.  The kT*G partial dots of a
// slot are summed by a reduce-scatter butterfly over its LPT lanes.  Scores,
// then weights, live in LDS token-major (the G heads of a token adjacent, so
// the P.V loop reads them with one vector load per token); the first step's
// V rows are loaded while the
// softmax statistics are formed.  The chunk's max m, exp-sum l and
// unnormalized output o go to the workspace (fp32: they are fp32 sums).  A
// single chunk writes the output itself.
//
// Combine pass: block (h, slice) merges the chunks of query head h for 16
// dims in fp64, all of its loads issued at once (one memory round trip).
// A second launch, not a last-arriving block: a device-wide handoff inside
// one launch costs a store acknowledgement, an atomic and a load, about
// three memory round trips on this chip, against one launch gap here.
#include <math.h>

#include <mutex>

#include "tq_device.h"
#include "tq_host.h"

namespace tq {
namespace {

constexpr int kAttnThreads = 256;
constexpr int kAttnNW = kAttnThreads / kWave;
constexpr int kAttnMinChunk = 64;    // smallest step of any (G, D, kT)
constexpr int kAttnMaxSplits = 64;   // chunks per KV head
constexpr int kCombineDims = 16;     // dims per combine block
constexpr int kCombineSubs = kAttnThreads / kCombineDims;  // row subranges
constexpr int kCombineBatch =  // rows per thread
    (kAttnMaxSplits + kCombineSubs - 1) / kCombineSubs;

// Per (G, D, kT): lanes per token row, token slots, tokens per block step.
// kT (tokens per lane slot and step) is at least LPT/G so that every lane
// ends the butterfly with a complete sum.
template <int G, int D, int KT, int NW>
struct AttnShape {
  static constexpr int LPT = D / 8;          // lanes per token row
  static constexpr int TPW = kWave / LPT;    // token slots per wave
  static constexpr int TPB = NW * TPW;       // token slots per block
  static constexpr int kT = KT;
  static constexpr int CH = TPB * kT;         // tokens per block step
  static constexpr int NV = kT * G;           // partial dots per lane
  static constexpr int VPL = NV / LPT;        // complete sums per lane
  static_assert(NV % LPT == 0 && VPL >= 1, "butterfly shape");
  static_assert(CH >= kAttnMinChunk, "workspace sized for 64-token steps");
};
// Tokens per lane slot and step: 4, or LPT/G where that is more (every lane
// must end the butterfly with a complete sum).  Measured on MI355X: 8 per
// slot at long contexts (larger steps, fewer of them) was slower with both
// block sizes.
template <int G, int D>
constexpr int kt_of() {
  return D / 8 / G > 4 ? D / 8 / G : 4;
}

struct AttnArgs {
  const float *q;         // [H, D]
  const uint16_t *k, *v;  // [L, Hkv, D] bf16
  int Hkv, L;
  int chunk;              // tokens per chunk (whole steps)
  int S;                  // chunks per KV head
  float scale;
  float *part;            // [H][S][D + 4]: o[D], m, l, 2 unused
  float *out;             // [H, D]
};

__device__ __forceinline__ void widen8(const u32x4 &r, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(r[i] << 16);
    x[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
  }
}

// The partner of a halving step at bit OFF, read through DPP (no LDS round
// trip): within aligned groups of 2*OFF lanes, lane i takes lane 2*OFF-1-i
// for OFF = 8 and 4 (row mirror, half-row mirror) and lane i ^ OFF for
// OFF = 2 and 1 (quad permutations).  Each partner differs from i in bit
// OFF and agrees with it in the bits above, which is all a step needs: both
// then hold sums over the same lanes, of opposite halves.
template <int OFF>
__device__ __forceinline__ float butterfly_partner(float v) {
  static_assert(OFF == 8 || OFF == 4 || OFF == 2 || OFF == 1, "step");
  constexpr int ctrl = OFF == 8 ? 0x140 : (OFF == 4 ? 0x141 : (OFF == 2 ? 0x4e : 0xb1));
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xf, 0xf, false));
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
      val[k] = keep + butterfly_partner<OFF>(send);
    }
    reduce_scatter<OFF / 2, W / 2>(val, lt);
  }
}

// Wave reductions by DPP that end in the last lane (row shifts within each
// 16-lane row, then the two row broadcasts).  For the maximum a lane with no
// source keeps its own value; for the sum it adds zero.
template <int Ctrl, int RowMask>
__device__ __forceinline__ float dpp_keep(float v) {
  const int x = __float_as_int(v);
  return __int_as_float(__builtin_amdgcn_update_dpp(x, x, Ctrl, RowMask, 0xf, false));
}

template <int Ctrl, int RowMask>
__device__ __forceinline__ float dpp_zero(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), Ctrl, RowMask, 0xf, false));
}

template <int Ctrl, int RowMask>
__device__ __forceinline__ double dpp_zero(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)b, Ctrl, RowMask, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)(b >> 32), Ctrl, RowMask, 0xf, false);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

__device__ __forceinline__ float wave_max_last(float v) {
  v = fmaxf(v, dpp_keep<0x111, 0xf>(v));
  v = fmaxf(v, dpp_keep<0x112, 0xf>(v));
  v = fmaxf(v, dpp_keep<0x114, 0xf>(v));
  v = fmaxf(v, dpp_keep<0x118, 0xf>(v));
  v = fmaxf(v, dpp_keep<0x142, 0xa>(v));
  return fmaxf(v, dpp_keep<0x143, 0xc>(v));
}

__device__ __forceinline__ float wave_sum_last(float v) {
  v += dpp_zero<0x111, 0xf>(v);
  v += dpp_zero<0x112, 0xf>(v);
  v += dpp_zero<0x114, 0xf>(v);
  v += dpp_zero<0x118, 0xf>(v);
  v += dpp_zero<0x142, 0xa>(v);
  return v + dpp_zero<0x143, 0xc>(v);
}

__device__ __forceinline__ double wave_sum_last(double v) {
  v += dpp_zero<0x111, 0xf>(v);
  v += dpp_zero<0x112, 0xf>(v);
  v += dpp_zero<0x114, 0xf>(v);
  v += dpp_zero<0x118, 0xf>(v);
  v += dpp_zero<0x142, 0xa>(v);
  return v + dpp_zero<0x143, 0xc>(v);
}

// v plus its value in lane (lane ^ OFF), OFF = 8, 16 or 32, without an LDS
// round trip: a DPP rotate by 8 within each 16-lane row (which is lane ^ 8),
// or the row-swap instructions of gfx950 (v_permlane16_swap /
// v_permlane32_swap: called with one value as both operands, the two
// results hold the two partners of every pair).  Both lanes of a pair get
// the same sum, bit for bit, as from a shuffle (addition commutes).
template <int OFF>
__device__ __forceinline__ float add_lane_xor(float v) {
  static_assert(OFF == 8 || OFF == 16 || OFF == 32, "lane offset");
  if constexpr (OFF == 8) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false));
  } else if constexpr (OFF == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
  } else {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
}

template <int G, int D, int KT, int NW>
__global__ __launch_bounds__(NW *kWave) void attn_chunk_kernel(AttnArgs a) {
  using Sh = AttnShape<G, D, KT, NW>;
  constexpr int LPT = Sh::LPT, TPW = Sh::TPW, kT = Sh::kT, STEP = Sh::CH;
  constexpr int NV = Sh::NV, VPL = Sh::VPL, NT = NW * kWave;
  // Dynamic LDS: scores [chunk][G], then weights; after the P.V loop the
  // per-wave outputs [NW][G][D].
  extern __shared__ __align__(16) float s_lds[];
  __shared__ float red_m[NW][G], red_s[NW][G];

  const int chunk = a.chunk;
  const int g = blockIdx.x, c = blockIdx.y;
  const int t0 = c * chunk;
  const int n = min(chunk, a.L - t0);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int lt = lane % LPT;       // piece of the row (8 dims)
  const int tw = lane / LPT;       // token slot within the wave
  const int i0 = wave * TPW * kT;  // this wave's first token of a step

  // token of slot step u in the step starting at `it` (wave-uniform `it`)
  auto row = [&](const uint16_t *base, int i) {
    const int t = t0 + (i < n ? i : 0);  // past the chunk: an in-chunk row
    return *reinterpret_cast<const u32x4 *>(base + ((size_t)t * a.Hkv + g) * D + lt * 8);
  };

  float qd[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float4 *qp = reinterpret_cast<const float4 *>(a.q + (size_t)(g * G + j) * D + lt * 8);
    const float4 x0 = qp[0], x1 = qp[1];
    qd[j][0] = x0.x; qd[j][1] = x0.y; qd[j][2] = x0.z; qd[j][3] = x0.w;
    qd[j][4] = x1.x; qd[j][5] = x1.y; qd[j][6] = x1.z; qd[j][7] = x1.w;
  }

  // 1. scores, one step at a time, the next step's K rows in flight during
  // this step's arithmetic: after the reduce-scatter lane lt holds the
  // complete sums of values v = VPL*lt + b (v = u*G + j)
  // (Loads are unconditional, past the chunk they re-read an in-chunk row,
  // so the compiler's wait counts cover exactly the rows a step needs.)
  u32x4 rk[kT];
#pragma unroll
  for (int u = 0; u < kT; ++u) rk[u] = row(a.k, i0 + u * TPW + tw);
  for (int it = i0; it < n; it += STEP) {
    u32x4 rkn[kT];
#pragma unroll
    for (int u = 0; u < kT; ++u) rkn[u] = row(a.k, it + STEP + u * TPW + tw);
    float val[NV];
#pragma unroll
    for (int u = 0; u < kT; ++u) {
      float x[8];
      widen8(rk[u], x);
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float dsum = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) dsum = fmaf(qd[j][e], x[e], dsum);
        val[u * G + j] = dsum;
      }
    }
    reduce_scatter<LPT / 2, NV>(val, lt);
#pragma unroll
    for (int b = 0; b < VPL; ++b) {
      const int v = VPL * lt + b;
      const int i = it + (v / G) * TPW + tw;
      if (i < n) s_lds[i * G + v % G] = val[b] * a.scale;
    }
#pragma unroll
    for (int u = 0; u < kT; ++u) rk[u] = rkn[u];
  }
  // the first P.V step's V rows, in flight during the softmax statistics
  u32x4 rv[kT];
#pragma unroll
  for (int u = 0; u < kT; ++u) rv[u] = row(a.v, i0 + u * TPW + tw);
  __syncthreads();

  // 2. per-head max and exp-sum over the chunk (fixed reduction order): per
  // thread, then a DPP tree per wave ending in its last lane, then the
  // waves in order.  The G heads go through one loop and their trees
  // interleave (one head after another, each tree a chain of dependent LDS
  // shuffles, took about 2.5 us per block whatever the chunk length).
  float mx[G], sum[G];
  {
    float m[G];
#pragma unroll
    for (int j = 0; j < G; ++j) m[j] = -INFINITY;
    for (int i = threadIdx.x; i < n; i += NT)
#pragma unroll
      for (int j = 0; j < G; ++j) m[j] = fmaxf(m[j], s_lds[i * G + j]);
#pragma unroll
    for (int j = 0; j < G; ++j) m[j] = wave_max_last(m[j]);
    if (lane == kWave - 1) {
#pragma unroll
      for (int j = 0; j < G; ++j) red_m[wave][j] = m[j];
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < G; ++j) {
    mx[j] = red_m[0][j];
#pragma unroll
    for (int w = 1; w < NW; ++w) mx[j] = fmaxf(mx[j], red_m[w][j]);
  }
  {
    float sacc[G];
#pragma unroll
    for (int j = 0; j < G; ++j) sacc[j] = 0.0f;
    for (int i = threadIdx.x; i < n; i += NT)
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float p = expf(s_lds[i * G + j] - mx[j]);
        s_lds[i * G + j] = p;
        sacc[j] += p;
      }
#pragma unroll
    for (int j = 0; j < G; ++j) sacc[j] = wave_sum_last(sacc[j]);
    if (lane == kWave - 1) {
#pragma unroll
      for (int j = 0; j < G; ++j) red_s[wave][j] = sacc[j];
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < G; ++j) {
    sum[j] = red_s[0][j];
#pragma unroll
    for (int w = 1; w < NW; ++w) sum[j] += red_s[w][j];
  }

  // 3. unnormalized output sum_t p[t] v[t] over the chunk
  float acc[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.0f;
  auto pv_step = [&](const u32x4 (&r)[kT], int it) {
#pragma unroll
    for (int u = 0; u < kT; ++u) {
      // past the chunk: weight 0 on a re-read in-chunk row (adds +-0 exactly;
      // no branch, so the next step's loads stay in flight)
      const int i = it + u * TPW + tw;
      const int ic = i < n ? i : n - 1;
      const float keep = i < n ? 1.0f : 0.0f;
      float x[8];
      widen8(r[u], x);
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float p = s_lds[ic * G + j] * keep;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = fmaf(p, x[e], acc[j][e]);
      }
    }
  };
  auto load_v = [&](u32x4 (&r)[kT], int it) {
#pragma unroll
    for (int u = 0; u < kT; ++u) r[u] = row(a.v, it + u * TPW + tw);
  };
  // two steps per trip through two register sets (no copies between them,
  // so one set's loads stay in flight while the other is consumed)
  for (int it = i0; it < n; it += 2 * STEP) {
    u32x4 rv2[kT];
    load_v(rv2, it + STEP);
    pv_step(rv, it);
    if (it + STEP >= n) break;  // wave-uniform
    load_v(rv, it + 2 * STEP);
    pv_step(rv2, it + STEP);
  }
  // token slots of a wave (lanes LPT apart), then the waves, in order
  static_assert(LPT == 8 || LPT == 16, "lanes per token row");
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float t = acc[j][e];
      if constexpr (LPT == 8) t = add_lane_xor<8>(t);
      t = add_lane_xor<16>(t);
      acc[j][e] = add_lane_xor<32>(t);
    }
  __syncthreads();  // every wave is done reading the weights
  float *o_red = s_lds;  // [NW][G][D]
  if (tw == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) o_red[(wave * G + j) * D + lt * 8 + e] = acc[j][e];
  }
  __syncthreads();

  // 5. this chunk's result: the output itself when it is the only chunk,
  // else a partial row
  constexpr int RS = D + 4;  // partial row stride (floats)
  for (int idx = threadIdx.x; idx < G * D; idx += NT) {
    const int j = idx / D, d = idx % D;
    float o = o_red[j * D + d];
#pragma unroll
    for (int w = 1; w < NW; ++w) o += o_red[(w * G + j) * D + d];
    const size_t h = (size_t)(g * G + j);
    if (a.S == 1)
      a.out[h * D + d] = (float)((double)o / (double)sum[j]);
    else
      a.part[(h * a.S + c) * RS + d] = o;
  }
  if (a.S > 1 && threadIdx.x < G) {
    const int j = threadIdx.x;
    float *p = a.part + ((size_t)(g * G + j) * a.S + c) * RS + D;
    p[0] = mx[j];
    p[1] = sum[j];
  }
}

// Block (h, slice): out[h, d] for kCombineDims dims d, merging the S <=
// kAttnMaxSplits chunk results of head h in fp64, all loads issued at once:
//   M = max_c m_c,  den = sum_c e^(m_c - M) l_c,  out = sum_c e^(m_c - M) o_c / den
// M and den: thread c of wave 0 holds chunk c; fixed DPP trees over that
// wave, ending in its last lane.  Thread (sub, dd) sums the chunks c = sub,
// sub + kCombineSubs, ... in order; the subranges are added in order.
__global__ __launch_bounds__(kAttnThreads) void attn_combine_kernel(
    const float *__restrict__ part, int S, int D, float *__restrict__ out) {
  static_assert(kAttnMaxSplits <= kAttnThreads, "one chunk per thread");
  __shared__ double f[kAttnMaxSplits];  // e^(m_c - M)
  __shared__ double den_s;
  __shared__ double num_s[kCombineSubs][kCombineDims];
  const int h = blockIdx.x;
  const int dd = threadIdx.x % kCombineDims, sub = threadIdx.x / kCombineDims;
  const int d = blockIdx.y * kCombineDims + dd;
  const int RS = D + 4;
  const float *ph = part + (size_t)h * S * RS;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;

  float mv = -INFINITY, lv = 0.0f;
  if (tid < S) {
    mv = ph[(size_t)tid * RS + D];
    lv = ph[(size_t)tid * RS + D + 1];
  }
  float ov[kCombineBatch];
#pragma unroll
  for (int u = 0; u < kCombineBatch; ++u) {  // past the end: weight 0
    const int c = sub + u * kCombineSubs;
    ov[u] = c < S ? ph[(size_t)c * RS + d] : 0.0f;
  }
  // Every chunk is in wave 0 (S <= 64): its lanes form M and the
  // denominator with DPP trees that end in the last lane; the weights e and
  // the denominator reach the other waves through LDS.
  if (wave == 0) {
    const double M = (double)__int_as_float(
        __builtin_amdgcn_readlane(__float_as_int(wave_max_last(mv)), kWave - 1));
    const double e = tid < S ? exp((double)mv - M) : 0.0;
    f[tid] = e;
    const double dsum = wave_sum_last(e * (double)lv);
    if (lane == kWave - 1) den_s = dsum;
  }
  __syncthreads();
  const double den = den_s;
  double num = 0.0;
#pragma unroll
  for (int u = 0; u < kCombineBatch; ++u) {
    const int c = sub + u * kCombineSubs;
    num = fma(c < S ? f[c] : 0.0, (double)ov[u], num);
  }
  num_s[sub][dd] = num;
  __syncthreads();
  if (sub == 0) {
    double t = num_s[0][dd];
#pragma unroll
    for (int q = 1; q < kCombineSubs; ++q) t += num_s[q][dd];
    out[(size_t)h * D + d] = (float)(t / den);
  }
}

// One pass of NW-wave blocks, chunks of whole steps, at most `smax` chunks
// per KV head.
template <int G, int D, int KT, int NW>
tq_status launch_attn(const float *q, const void *k, const void *v, int H,
                      int Hkv, int L, float scale, float *out, float *part,
                      int smax, hipStream_t s) {
  constexpr int STEP = AttnShape<G, D, KT, NW>::CH;
  const int steps = (L + STEP * smax - 1) / (STEP * smax);
  AttnArgs a;
  a.q = q;
  a.k = static_cast<const uint16_t *>(k);
  a.v = static_cast<const uint16_t *>(v);
  a.Hkv = Hkv;
  a.L = L;
  a.chunk = steps * STEP;
  a.S = (L + a.chunk - 1) / a.chunk;
  a.scale = scale;
  a.part = part;
  a.out = out;
  constexpr int kOutFloats = NW * G * D;
  const size_t lds = (size_t)(G * a.chunk > kOutFloats ? G * a.chunk : kOutFloats) * 4;
  if (tq_status st = allow_dynamic_lds((const void *)attn_chunk_kernel<G, D, KT, NW>, (int)lds))
    return st;
  if (tq_status st = launch(attn_chunk_kernel<G, D, KT, NW>, dim3(Hkv, a.S),
                            dim3(NW * kWave), lds, s, a))
    return st;
  if (a.S == 1) return TQ_OK;
  return launch(attn_combine_kernel, dim3(H, D / kCombineDims), dim3(kAttnThreads), 0, s,
                static_cast<const float *>(part), a.S, D, out);
}

// Launch plan by context length (measured on MI355X, 20 query / 5 KV heads,
// D = 128, graphs of 16 calls over >= 1 GiB of KV copies):
//  * short contexts whose 4-wave chunk blocks (64-token steps, up to 64
//    chunks per KV head) number at most one per CU keep that plan
//    (L = 2048: 10.3 us against 10.7 with the plan below);
//  * otherwise 8-wave blocks (steps twice as long, so half as many per
//    wave) with at most CUs / Hkv chunks per KV head, so no CU holds two
//    blocks: L = 4096 / 8192 11.8-12.0 / 14.1 us against 13.5 / 15.7 us,
//    L = 16384 / 32768 / 131072 17.5 / 24.4-24.9 / 66.0 us against
//    21.2 / 28.8-29.6 / 80.0-81.2 us for 4-wave blocks with up to 64 chunks
//    (capped 4-wave blocks: 28.0 us at 32768; uncapped 8-wave blocks:
//    33.3 us; two capped 8-wave blocks per CU: 33.2 us), at most 4 tokens
//    per lane slot and step at every length (8 per slot beyond L = 8192:
//    19.3-19.9 / 25.7-25.8 / 69.7-73.0 us).
constexpr int kAttnShortL = 8192;
constexpr int kAttnWideNW = 8;
constexpr int kAttnScoreLds = 128 * 1024;  // bytes of scores per chunk block
constexpr int kAttnOneChunkL = 256;        // longest one-chunk 8-wave call

template <int G, int D>
tq_status launch_attn_g(const float *q, const void *k, const void *v, int H,
                        int Hkv, int L, float scale, float *out, float *part,
                        int num_cus, hipStream_t s) {
  constexpr int KS = kt_of<G, D>();
  if (L <= kAttnShortL) {
    constexpr int STEP = AttnShape<G, D, KS, kAttnNW>::CH;
    const int steps = (L + STEP * kAttnMaxSplits - 1) / (STEP * kAttnMaxSplits);
    const int chunks = (L + steps * STEP - 1) / (steps * STEP);
    // up to kAttnOneChunkL tokens, one 8-wave chunk (one launch, no
    // combine) beats two launches: L = 256 7.9 against 8.4 us; at 512 10.7
    // against 8.5 us
    if (chunks > 1 && L <= kAttnOneChunkL)
      return launch_attn<G, D, KS, kAttnWideNW>(q, k, v, H, Hkv, L, scale, out, part, 1, s);
    if ((int64_t)Hkv * chunks <= num_cus)
      return launch_attn<G, D, KS, kAttnNW>(q, k, v, H, Hkv, L, scale, out, part,
                                            kAttnMaxSplits, s);
  }
  // At most one block per CU, but chunks short enough that the G score rows
  // of a chunk stay within kAttnScoreLds of LDS (G * chunk fp32).
  int cap = num_cus / Hkv;
  const int lds_min = (int)(((int64_t)L * G * 4 + kAttnScoreLds - 1) / kAttnScoreLds);
  cap = cap < lds_min ? lds_min : cap;
  cap = cap < 1 ? 1 : (cap > kAttnMaxSplits ? kAttnMaxSplits : cap);
  return launch_attn<G, D, KS, kAttnWideNW>(q, k, v, H, Hkv, L, scale, out, part, cap, s);
}

template <int D>
tq_status launch_attn_d(int G, const float *q, const void *k, const void *v,
                        int H, int Hkv, int L, float scale, float *out,
                        float *part, int num_cus, hipStream_t s) {
  switch (G) {
    case 1: return launch_attn_g<1, D>(q, k, v, H, Hkv, L, scale, out, part, num_cus, s);
    case 2: return launch_attn_g<2, D>(q, k, v, H, Hkv, L, scale, out, part, num_cus, s);
    case 4: return launch_attn_g<4, D>(q, k, v, H, Hkv, L, scale, out, part, num_cus, s);
    case 8: return launch_attn_g<8, D>(q, k, v, H, Hkv, L, scale, out, part, num_cus, s);
  }
  return TQ_ERR_SHAPE;
}

}  // namespace
}  // namespace tq

extern "C" tq_status tq_attn_decode(const float *q, const void *k_cache,
                                    const void *v_cache, int64_t H, int64_t Hkv,
                                    int64_t D, int64_t L, float scale,
                                    float *out, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  using namespace tq;
  if (H < 1 || Hkv < 1 || H % Hkv != 0 || H > 256) return TQ_ERR_SHAPE;
  const int64_t G = H / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return TQ_ERR_SHAPE;
  if (D != 64 && D != 128) return TQ_ERR_SHAPE;
  if (L < 1 || L > TQ_ATTN_MAX_L) return TQ_ERR_SHAPE;
  if (!q || !k_cache || !v_cache || !out || !workspace) return TQ_ERR_NULL;
  if (workspace_bytes < TQ_ATTN_WORKSPACE_BYTES(H, D, L)) return TQ_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(out, 4) || !aligned(workspace, 16))
    return TQ_ERR_ALIGN;
  DeviceInfo dev;
  if (tq_status s = current_device(&dev)) return s;
  auto *part = static_cast<float *>(workspace);
  return D == 128 ? launch_attn_d<128>((int)G, q, k_cache, v_cache, (int)H, (int)Hkv,
                                       (int)L, scale, out, part, dev.num_cus, stream)
                  : launch_attn_d<64>((int)G, q, k_cache, v_cache, (int)H, (int)Hkv,
                                      (int)L, scale, out, part, dev.num_cus, stream);
}

// ---------------------------------------------------------------------------
// tq_attn_decode_noalloc: the same kernels with the per-chunk partials in a
// fixed device array instead of a caller workspace, for callers that cannot
// allocate.  Room for TQ_ATTN_NOALLOC_MAX_H query heads x kAttnMaxSplits
// chunks x (128 + 4) floats; each GPU holds its own copy for the life of the
// process.  The chunk pass writes every partial the combine pass reads, so
// nothing has to start at zero.
namespace tq {
namespace {
constexpr size_t kScratchFloats =
    (size_t)TQ_ATTN_NOALLOC_MAX_H * kAttnMaxSplits * (128 + 4);
static_assert(kScratchFloats * 4 == TQ_ATTN_NOALLOC_SCRATCH_BYTES,
              "scratch size in the header");
}  // namespace
}  // namespace tq

static __device__ __align__(256) float scratch[tq::kScratchFloats];

namespace tq {
namespace {
// Device address of this GPU's copy of `scratch`.  In host code the array's
// name is only a stand-in: the address comes from the runtime, once per
// device (with that device current), and is kept.
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kScratchDevices];

tq_status scratch_address(int dev, float **out) {
  if (dev < 0 || dev >= kScratchDevices) return TQ_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return TQ_ERR_DEVICE;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<float *>(g_scratch_ptr[dev]);
  return TQ_OK;
}
}  // namespace
}  // namespace tq

extern "C" tq_status tq_attn_decode_noalloc(const float *q, const void *k_cache,
                                            const void *v_cache, int64_t H,
                                            int64_t Hkv, int64_t D, int64_t L,
                                            float scale, float *out,
                                            hipStream_t stream) {
  using namespace tq;
  if (H < 1 || Hkv < 1 || H % Hkv != 0 || H > TQ_ATTN_NOALLOC_MAX_H) return TQ_ERR_SHAPE;
  const int64_t G = H / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return TQ_ERR_SHAPE;
  if (D != 64 && D != 128) return TQ_ERR_SHAPE;
  if (L < 1 || L > TQ_ATTN_MAX_L) return TQ_ERR_SHAPE;
  if (!q || !k_cache || !v_cache || !out) return TQ_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(out, 4))
    return TQ_ERR_ALIGN;
  DeviceInfo dev;
  if (tq_status s = current_device(&dev)) return s;
  float *part = nullptr;
  if (tq_status s = scratch_address(dev.device, &part)) return s;
  // At most kAttnMaxSplits chunks of H rows of D + 4 floats are written.
  return D == 128 ? launch_attn_d<128>((int)G, q, k_cache, v_cache, (int)H, (int)Hkv,
                                       (int)L, scale, out, part, dev.num_cus, stream)
                  : launch_attn_d<64>((int)G, q, k_cache, v_cache, (int)H, (int)Hkv,
                                      (int)L, scale, out, part, dev.num_cus, stream);
}
