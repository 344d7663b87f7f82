// tq_gemm_small.hip -- the ternary product for a small batch of activation
// rows (tq_gemm_small, 2 <= M <= 64) and the M > 1 branch of
// tq_gate_up_relu2, on the gfx950 int8 matrix cores.
//
// Page "Blog · field notes" (1bit engine), post "Qwen3.8-27B at 45.7 tok/s":
// prompt processing is set by the GPU's matrix units while decode is set by
// memory bandwidth; post "One GPU, many users": one GPU serving several
// requests at once, i.e. several activation rows per weight read.
//
// Mapping: v_mfma_i32_16x16x64_i8 computes D[16x16] += A[16x64] * B[64x16].
// A = 16 packed weight rows of one plane, decoded to signed int8 {-1,0,+1}
// with one v_perm_b32 byte lookup per dword; B = 16 activation rows.  Lane
// l loads 16 bytes of packed row i0 + (l % 16) at k offset 16*(l / 16) of a
// 64-byte k step; that one load gives the A operands of all four planes
// (4 output row blocks).  B is the same 16-byte k block of activation row
// l % 16.  Because A and B take the same k block per lane, the sum over k
// does not depend on how the matrix core orders k inside its step.  The
// eight waves of a block own contiguous k ranges and keep U k steps of loads
// in flight; their partial tiles are summed in LDS with integer atomics
// (exact, order free).
#include "tq_device.h"
#include "tq_host.h"

namespace tq {

tq_status gemv_m1(const uint8_t *p0, float s0, const uint8_t *p1, float s1,
                  const int8_t *xq, const float *x_scale, int64_t N, int64_t K,
                  float *y, int32_t *acc0, int32_t *acc1, hipStream_t stream);

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kGemmWaves = 8;
constexpr int kGemmThreads = kGemmWaves * kWave;

struct GemmArgs {
  const uint8_t *p0, *p1;
  float s0, s1;
  const int8_t *xq;
  const float *x_scale;
  int M, n4, K;
  float *y;
  int32_t *acc0, *acc1;
};

// Plane j of a 16-byte piece as signed weights: codes {0,1,2} select the
// bytes 0xFF, 0x00, 0x01 (-1, 0, +1) of a 4-byte table.
__device__ __forceinline__ v4i signed_plane(const uint4 &w, int j) {
  constexpr uint32_t kTable = 0x000100FFu;
  const int sh = 2 * j;
  v4i a;
  a[0] = (int)__builtin_amdgcn_perm(0u, kTable, (w.x >> sh) & 0x03030303u);
  a[1] = (int)__builtin_amdgcn_perm(0u, kTable, (w.y >> sh) & 0x03030303u);
  a[2] = (int)__builtin_amdgcn_perm(0u, kTable, (w.z >> sh) & 0x03030303u);
  a[3] = (int)__builtin_amdgcn_perm(0u, kTable, (w.w >> sh) & 0x03030303u);
  return a;
}

template <int MT, int U, bool kGate>
__global__ __launch_bounds__(kGemmThreads) void gemm_small_kernel(GemmArgs g) {
  constexpr int NM = kGate ? 2 : 1;
  constexpr int kTileInts = 64 * 4;               // one 16x16 int32 tile
  constexpr int kRed = NM * 4 * MT * kTileInts;   // all tiles of the block
  __shared__ int red[kRed];

  for (int t = threadIdx.x; t < kRed; t += kGemmThreads) red[t] = 0;
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int i0 = blockIdx.x * 16;
  const int prow = min(i0 + (lane & 15), g.n4 - 1);  // past the end: reread
  const int kb = 16 * (lane >> 4);
  const int K = g.K;
  const int nsteps = (K + 63) / 64;
  const int per = (nsteps + kGemmWaves - 1) / kGemmWaves;
  const int s0 = min(wave * per, nsteps);
  const int s1 = min(s0 + per, nsteps);

  const uint8_t *P[NM];
  P[0] = g.p0 + (size_t)prow * K;
  if constexpr (kGate) P[NM - 1] = g.p1 + (size_t)prow * K;
  const int8_t *Q[MT];
  bool qrow_ok[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int row = 16 * t + (lane & 15);
    qrow_ok[t] = row < g.M;
    Q[t] = g.xq + (size_t)min(row, g.M - 1) * K;
  }

  v4i acc[NM][4][MT];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[m][j][t] = v4i{0, 0, 0, 0};

  for (int s = s0; s < s1; s += U) {
    // U k steps of loads in flight.  Slots past this wave's range (or past
    // K) read an in-bounds piece and get a zero activation operand.
    uint4 w[U][NM];
    v4i b[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = (s + u) * 64 + kb;
      const bool ok = s + u < s1 && kk < K;  // K % 64 may leave a ragged step
      const int k = ok ? kk : 0;
#pragma unroll
      for (int m = 0; m < NM; ++m)
        w[u][m] = load_stream16(reinterpret_cast<const uint4 *>(P[m] + k));
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const uint4 v = *reinterpret_cast<const uint4 *>(Q[t] + k);
        const bool use = ok && qrow_ok[t];
        b[u][t] = use ? v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w}
                      : v4i{0, 0, 0, 0};
      }
    }
    // Keep all U steps of loads ahead of the first MFMA.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v4i a = signed_plane(w[u][m], j);
#pragma unroll
          for (int t = 0; t < MT; ++t)
            acc[m][j][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[u][t],
                                                                 acc[m][j][t], 0, 0, 0);
        }
  }

  // Exact cross-wave reduction in LDS.
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          atomicAdd(&red[((m * 4 + j) * MT + t) * kTileInts + lane * 4 + i],
                    acc[m][j][t][i]);
  __syncthreads();

  // Epilogue.  Output tile layout of the 16x16 int32 result: lane l holds
  // rows 4*(l/16) + i (i = 0..3) of column l % 16.  Rows are packed rows
  // i0 + r of plane j (output n = j*N/4 + i0 + r); columns are activation
  // rows m = 16 t + c.
  const size_t N = (size_t)g.n4 * 4;
  for (int jt = wave; jt < 4 * MT; jt += kGemmWaves) {
    const int j = jt / MT, t = jt % MT;
    const int c = lane & 15;
    const int m = 16 * t + c;
    if (m >= g.M) continue;
    const float sx = g.x_scale[m];
    const float c0 = g.s0 * sx, c1 = g.s1 * sx;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * (lane >> 4) + i;
      if (i0 + r >= g.n4) break;
      const size_t n = (size_t)j * g.n4 + i0 + r;
      const size_t o = (size_t)m * N + n;
      const int v0 = red[((0 * 4 + j) * MT + t) * kTileInts + lane * 4 + i];
      if (g.acc0) g.acc0[o] = v0;
      if constexpr (kGate) {
        const int v1 = red[(((NM - 1) * 4 + j) * MT + t) * kTileInts + lane * 4 + i];
        if (g.acc1) g.acc1[o] = v1;
        g.y[o] = relu2_gate(rescale(v0, c0), rescale(v1, c1));
      } else {
        g.y[o] = rescale(v0, c0);
      }
    }
  }
}

// k steps in flight per wave: the whole per-wave range when it is short,
// fewer for larger M (the activation operands cost 4*MT VGPRs per step).
template <int MT, bool kGate>
tq_status launch_gemm_mt(const GemmArgs &a, hipStream_t s) {
  const dim3 grid((a.n4 + 15) / 16), block(kGemmThreads);
  const int nsteps = (a.K + 63) / 64;
  const int per = (nsteps + kGemmWaves - 1) / kGemmWaves;
  constexpr int kUMax = kGate ? (MT <= 1 ? 8 : (MT == 2 ? 4 : 2))
                              : (MT <= 2 ? 8 : 4);
  if constexpr (kUMax == 2) {
    return launch(gemm_small_kernel<MT, 2, kGate>, grid, block, 0, s, a);
  } else if constexpr (kUMax == 4) {
    if (per <= 2) return launch(gemm_small_kernel<MT, 2, kGate>, grid, block, 0, s, a);
    return launch(gemm_small_kernel<MT, 4, kGate>, grid, block, 0, s, a);
  } else {
    if (per <= 2) return launch(gemm_small_kernel<MT, 2, kGate>, grid, block, 0, s, a);
    if (per <= 4) return launch(gemm_small_kernel<MT, 4, kGate>, grid, block, 0, s, a);
    return launch(gemm_small_kernel<MT, 8, kGate>, grid, block, 0, s, a);
  }
}

template <bool kGate>
tq_status launch_gemm(int M, const GemmArgs &a, hipStream_t s) {
  switch ((M + 15) / 16) {
    case 1: return launch_gemm_mt<1, kGate>(a, s);
    case 2: return launch_gemm_mt<2, kGate>(a, s);
    case 3: return launch_gemm_mt<3, kGate>(a, s);
    case 4: return launch_gemm_mt<4, kGate>(a, s);
  }
  return TQ_ERR_SHAPE;
}

tq_status gemm_small(const uint8_t *p0, float s0, const uint8_t *p1, float s1,
                     const int8_t *xq, const float *x_scale, int64_t M,
                     int64_t N, int64_t K, float *y, int32_t *acc0,
                     int32_t *acc1, hipStream_t stream) {
  if (M == 1)
    return gemv_m1(p0, s0, p1, s1, xq, x_scale, N, K, y, acc0, acc1, stream);
  DeviceInfo dev;
  if (tq_status s = current_device(&dev)) return s;
  GemmArgs a;
  a.p0 = p0;
  a.p1 = p1;
  a.s0 = s0;
  a.s1 = s1;
  a.xq = xq;
  a.x_scale = x_scale;
  a.M = (int)M;
  a.n4 = (int)(N / 4);
  a.K = (int)K;
  a.y = y;
  a.acc0 = acc0;
  a.acc1 = acc1;
  return p1 ? launch_gemm<true>((int)M, a, stream)
            : launch_gemm<false>((int)M, a, stream);
}

tq_status check_common(const uint8_t *p, const int8_t *xq, const float *x_scale,
                       int64_t M, int64_t N, int64_t K, const float *y,
                       const int32_t *acc0, const int32_t *acc1) {
  if (tq_status s = check_nk(N, K)) return s;
  if (check_m(M) != TQ_OK) return TQ_ERR_SHAPE;
  if (M == 0 || N == 0) return TQ_OK;
  if (!y || !x_scale || (K > 0 && (!p || !xq))) return TQ_ERR_NULL;
  if (!aligned(p, 16) || !aligned(xq, 16) || !aligned(y, 4) ||
      !aligned(x_scale, 4) || !aligned(acc0, 4) || !aligned(acc1, 4))
    return TQ_ERR_ALIGN;
  return TQ_OK;
}

}  // namespace
}  // namespace tq

extern "C" tq_status tq_gemm_small(const uint8_t *packed, float w_scale,
                                   const int8_t *xq, const float *x_scale,
                                   int64_t M, int64_t N, int64_t K, float *y,
                                   int32_t *acc, hipStream_t stream) {
  using namespace tq;
  if (tq_status s = check_common(packed, xq, x_scale, M, N, K, y, acc, nullptr))
    return s;
  if (M == 0 || N == 0) return TQ_OK;
  return gemm_small(packed, w_scale, nullptr, 0.0f, xq, x_scale, M, N, K, y,
                    acc, nullptr, stream);
}

extern "C" tq_status tq_gate_up_relu2(const uint8_t *packed_gate, float s_gate,
                                      const uint8_t *packed_up, float s_up,
                                      const int8_t *xq, const float *x_scale,
                                      int64_t M, int64_t N, int64_t K, float *h,
                                      int32_t *acc_gate, int32_t *acc_up,
                                      hipStream_t stream) {
  using namespace tq;
  if (tq_status s = check_common(packed_gate, xq, x_scale, M, N, K, h,
                                 acc_gate, acc_up))
    return s;
  if (M == 0 || N == 0) return TQ_OK;
  if (K > 0 && !packed_up) return TQ_ERR_NULL;
  if (!aligned(packed_up, 16)) return TQ_ERR_ALIGN;
  // The kernels tell the gated form by a non-null second stream; with K == 0
  // both streams are empty, so any non-null stand-in keeps the gated path.
  const uint8_t *pu = packed_up ? packed_up : packed_gate;
  if (!pu) pu = reinterpret_cast<const uint8_t *>(h);
  return gemm_small(packed_gate, s_gate, pu, s_up, xq, x_scale, M, N, K, h,
                    acc_gate, acc_up, stream);
}
