// tq_gemm_small.hip -- the ternary product for a small batch of activation
// rows (tq_gemm_small, 2 <= M <= 64) and the M > 1 branch of
// tq_gate_up_relu2, on the gfx950 int8 matrix cores.
//
// Page "Blog · field notes" (1bit engine), post "Qwen3.8-27B at 45.7 tok/s":
// prompt processing is set by the GPU's matrix units while decode is set by
// memory bandwidth; post "One GPU, many users": one GPU serving several
// requests at once, i.e. several activation rows per weight read.
//
// v_mfma_i32_16x16x64_i8 computes D[16x16] += A[16x64] * B[64x16]; lane l
// supplies 16 bytes of A row l % 16 and of B column l % 16, both for the
// same k block (l / 16), so the k order inside a step never matters.  A rows
// are packed weight rows decoded to signed int8 {-1,0,+1} by one v_perm_b32
// byte lookup per dword; B columns are activation rows.
//
// Two kernel forms, both with one 16-row activation tile per block:
//  * direct (M <= 16): a tile is TP = 4 or 8 packed rows; MFMA row r is
//    packed row r / PL, plane r % PL + PL*h (PL = 16/TP planes per MFMA,
//    4/PL MFMAs per load).  The lanes that share a packed piece load the
//    same address, so a load touches only TP rows, and small TP gives enough
//    tiles to spread the weight stream over every CU.
//  * staged (M > 16): a tile is 16 packed rows (one plane per MFMA, four
//    MFMAs per load) and M is split over blocks, so each block reads as
//    many activation rows as weight rows.  Operands are loaded with
//    contiguous 256-byte row segments (4 rows per load instruction), written
//    to a wave-private LDS tile with a swizzle that keeps both the writes
//    (one row, 16 pieces) and the MFMA-layout reads (16 rows, one piece)
//    free of bank conflicts, then read back as MFMA operands.
// In both forms the waves of a block own contiguous k ranges; their partial
// tiles are summed in LDS with integer atomics (exact, order free).  Blocks
// are mapped to tiles XCD-aware: the M-split blocks of one weight tile run
// on one XCD, so all but the first read it from that XCD's L2.
#include "tq_device.h"
#include "tq_host.h"

namespace tq {

tq_status gemv_m1(const uint8_t *p0, float s0, const uint8_t *p1, float s1,
                  const int8_t *xq, const float *x_scale, int64_t N, int64_t K,
                  float *y, int32_t *acc0, int32_t *acc1, hipStream_t stream);
// 2 <= M <= 4 on the vector ALU (tq_gemm_dot4.hip).
bool gemm_dot4_fits(int64_t M, int64_t K);
tq_status gemm_dot4(const uint8_t *p, float s_w, const int8_t *xq, const float *x_scale,
                    int64_t M, int64_t N, int64_t K, float *y, int32_t *acc,
                    int num_cus, hipStream_t stream);

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kXcds = 8;  // MI355X: 8 XCDs, blocks dispatched round-robin

struct GemmArgs {
  const uint8_t *p0, *p1;
  float s0, s1;
  const int8_t *xq;
  const float *x_scale;
  int M, n4, K;
  float *y;
  int32_t *acc0, *acc1;
  int ntiles, mtiles;  // weight tiles, 16-row activation tiles
};

// Block -> (weight tile, activation tile).  The grid is padded to a
// multiple of kXcds * mtiles; block b runs on XCD b % kXcds, and the
// mtiles consecutive blocks of one XCD share a weight tile.  Returns false
// for padding blocks (the whole block exits before any barrier).
__device__ __forceinline__ bool block_tile(const GemmArgs &g, int &tile, int &mt) {
  const int b = blockIdx.x;
  const int slot = b / kXcds;
  tile = (slot / g.mtiles) * kXcds + b % kXcds;
  mt = slot % g.mtiles;
  return tile < g.ntiles;
}

// Signed weights of one plane of a 16-byte piece: codes {0,1,2} select the
// bytes 0xFF, 0x00, 0x01 (-1, 0, +1) of a 4-byte table.  sh = 2 * plane.
__device__ __forceinline__ v4i plane_operand(const u32x4 &w, int sh) {
  constexpr uint32_t kTable = 0x000100FFu;
  v4i a;
#pragma unroll
  for (int d = 0; d < 4; ++d)
    a[d] = (int)__builtin_amdgcn_perm(0u, kTable, (w[d] >> sh) & 0x03030303u);
  return a;
}

__device__ __forceinline__ v4i as_v4i(const u32x4 &v) {
  return v4i{(int)v[0], (int)v[1], (int)v[2], (int)v[3]};
}

// Rescale (and gate) one output (m, n) from its exact int32 sums.
template <bool kGate>
__device__ __forceinline__ void emit(const GemmArgs &g, int m, size_t n, int v0,
                                     int v1) {
  const size_t o = (size_t)m * g.n4 * 4 + n;
  const float sx = g.x_scale[m];
  if (g.acc0) g.acc0[o] = v0;
  if constexpr (kGate) {
    if (g.acc1) g.acc1[o] = v1;
    g.y[o] = relu2_gate(rescale(v0, g.s0 * sx), rescale(v1, g.s1 * sx));
  } else {
    g.y[o] = rescale(v0, g.s0 * sx);
  }
}

// ------------------------------------------------------------ direct form
template <int TP, int U, int W, bool kGate>
__global__ __launch_bounds__(W *kWave) void gemm_direct_kernel(GemmArgs g) {
  constexpr int NM = kGate ? 2 : 1;
  constexpr int PL = 16 / TP;  // planes per MFMA
  constexpr int NG = 4 / PL;   // MFMAs per loaded piece
  __shared__ int red[NM][NG][256];
  int tile, mt;
  if (!block_tile(g, tile, mt)) return;
  for (int t = threadIdx.x; t < NM * NG * 256; t += W * kWave) (&red[0][0][0])[t] = 0;
  __syncthreads();

  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int r = lane & 15;  // MFMA row (A) / column (B) of this lane
  const int i0 = tile * TP;
  const int prow = min(i0 + r / PL, g.n4 - 1);  // past the end: reread
  const int kb = 16 * (lane >> 4);
  const int K = g.K;
  const int nsteps = (K + 63) / 64;
  const int per = (nsteps + W - 1) / W;
  const int s0 = min(wave * per, nsteps), s1 = min(s0 + per, nsteps);
  const uint8_t *P[NM];
  P[0] = g.p0 + (size_t)prow * K;
  if constexpr (kGate) P[NM - 1] = g.p1 + (size_t)prow * K;
  const bool qok = r < g.M;  // one activation tile: M <= 16
  const int8_t *Q = g.xq + (size_t)min(r, g.M - 1) * K;

  v4i acc[NM][NG];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int h = 0; h < NG; ++h) acc[m][h] = v4i{0, 0, 0, 0};

  for (int s = s0; s < s1; s += U) {
    // U k steps of loads in flight.  Slots past this wave's range (or past
    // K: K % 64 may leave a ragged step) reread an in-bounds piece and get a
    // zero activation operand.
    u32x4 w[U][NM];
    v4i b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = (s + u) * 64 + kb;
      const bool ok = s + u < s1 && kk < K;
      const int k = ok ? kk : 0;
#pragma unroll
      for (int m = 0; m < NM; ++m)
        w[u][m] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(P[m] + k));
      const u32x4 v = *reinterpret_cast<const u32x4 *>(Q + k);
      b[u] = (ok && qok) ? as_v4i(v) : v4i{0, 0, 0, 0};
    }
    // Keep all U steps of loads ahead of the first MFMA.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int h = 0; h < NG; ++h)
          acc[m][h] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
              plane_operand(w[u][m], 2 * (r % PL + PL * h)), b[u], acc[m][h], 0, 0, 0);
  }

  // Exact cross-wave reduction, then the epilogue.  D element i of lane l is
  // row rr = 4*(l/16) + i (packed row i0 + rr/PL, plane rr%PL + PL*h) of
  // column l % 16 (activation row).
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int h = 0; h < NG; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) atomicAdd(&red[m][h][lane * 4 + i], acc[m][h][i]);
  __syncthreads();
  for (int h = wave; h < NG; h += W) {
    if (r >= g.M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 4 * (lane >> 4) + i;
      const int p = i0 + rr / PL;
      if (p >= g.n4) continue;
      const size_t n = (size_t)(rr % PL + PL * h) * g.n4 + p;
      emit<kGate>(g, r, n, red[0][h][lane * 4 + i], red[NM - 1][h][lane * 4 + i]);
    }
  }
}

// ------------------------------------------------------------ staged form
constexpr int kStageJ = 16;              // 16-byte pieces per row per batch
constexpr int kStageSlots = 16 * kStageJ;  // one 16-row operand tile

// LDS slot of piece j (k = batch base + 16 j) of tile row r (0..15).  The
// bank group of a slot is its index mod 16: (r + j) mod 16 differs across
// the 16 rows of one piece (MFMA reads) and across 16 pieces of one row
// (writes), so neither access conflicts.
__device__ __forceinline__ int stage_slot(int r, int j) {
  return (j >> 2) * 64 + (j & 3) * 16 + ((r + j) & 15);
}

template <int W, bool kGate>
__global__ __launch_bounds__(W *kWave) void gemm_staged_kernel(GemmArgs g) {
  constexpr int NM = kGate ? 2 : 1;
  constexpr int RPI = kWave / kStageJ;  // rows per load instruction (4)
  constexpr int NI = 16 / RPI;          // load instructions per operand tile
  __shared__ u32x4 stage[W][(NM + 1) * kStageSlots];
  __shared__ int red[NM][4][256];
  int tile, mt;
  if (!block_tile(g, tile, mt)) return;
  for (int t = threadIdx.x; t < NM * 4 * 256; t += W * kWave) (&red[0][0][0])[t] = 0;

  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  u32x4 *As = stage[wave];                      // NM weight tiles
  u32x4 *Bs = stage[wave] + NM * kStageSlots;   // activation tile
  const int i0 = tile * 16;
  const int K = g.K;
  const int m0 = mt * 16;
  const int mvalid = min(g.M - m0, 16);
  // Activation rows >= mvalid stay zero for the whole kernel.
  for (int t = lane; t < kStageSlots; t += kWave) Bs[t] = u32x4{0, 0, 0, 0};
  const int nb = (K + 16 * kStageJ - 1) / (16 * kStageJ);
  const int per = (nb + W - 1) / W;
  const int b0 = min(wave * per, nb), b1 = min(b0 + per, nb);
  const int lrow = lane / kStageJ, lj = lane % kStageJ;  // load-side mapping
  v4i acc[NM][4];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[m][j] = v4i{0, 0, 0, 0};
  __syncthreads();

  for (int bb = b0; bb < b1; ++bb) {
    const int k = bb * 16 * kStageJ + 16 * lj;
    const bool kok = k < K;
    const int kc = kok ? k : K - 16;  // in bounds; its activation is zeroed
    u32x4 wv[NM][NI], xv[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int prow = min(i0 + i * RPI + lrow, g.n4 - 1);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const uint8_t *p = (m == 0 ? g.p0 : g.p1) + (size_t)prow * K + kc;
        wv[m][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = min(m0 + i * RPI + lrow, g.M - 1);
      if (i * RPI < mvalid)  // uniform: some row of this load is valid
        xv[i] = *reinterpret_cast<const u32x4 *>(g.xq + (size_t)row * K + kc);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int m = 0; m < NM; ++m)
        As[m * kStageSlots + stage_slot(i * RPI + lrow, lj)] = wv[m][i];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = i * RPI + lrow;
      if (i * RPI < mvalid)
        Bs[stage_slot(r, lj)] = (kok && r < mvalid) ? xv[i] : u32x4{0, 0, 0, 0};
    }
    // The tile is private to this wave, and a wave's LDS accesses complete
    // in order; this only keeps the compiler from moving accesses across.
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int u = 0; u < kStageJ / 4; ++u) {
      const int slot = stage_slot(lane & 15, 4 * u + (lane >> 4));
      const v4i b = as_v4i(Bs[slot]);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const u32x4 a = As[m * kStageSlots + slot];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[m][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(plane_operand(a, 2 * j), b,
                                                            acc[m][j], 0, 0, 0);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) atomicAdd(&red[m][j][lane * 4 + i], acc[m][j][i]);
  __syncthreads();
  // D element i of lane l: packed row i0 + 4*(l/16) + i of plane j, column
  // (activation row m0 + l % 16).
  const int mrow = m0 + (lane & 15);
  for (int j = wave; j < 4; j += W) {
    if (mrow >= g.M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = i0 + 4 * (lane >> 4) + i;
      if (p >= g.n4) continue;
      emit<kGate>(g, mrow, (size_t)j * g.n4 + p, red[0][j][lane * 4 + i],
                  red[NM - 1][j][lane * 4 + i]);
    }
  }
}

// ------------------------------------------------------------ launch
// Grid: tiles padded so every XCD gets whole groups of mtiles blocks.
dim3 gemm_grid(const GemmArgs &a) {
  const int groups = (a.ntiles + kXcds - 1) / kXcds;
  return dim3((unsigned)(groups * kXcds * a.mtiles));
}

template <bool kGate>
tq_status launch_gemm(GemmArgs a, int num_cus, hipStream_t s) {
  if (a.M <= 16) {
    // Direct form.  Tile height: 8 packed rows while that still gives about
    // one tile per CU (measured: taller tiles cut activation re-reads),
    // else 4 so the weight stream is spread over every CU.
    a.mtiles = 1;
    if ((int64_t)a.n4 >= 8LL * num_cus * 3 / 4) {
      a.ntiles = (a.n4 + 7) / 8;
      return launch(gemm_direct_kernel<8, 4, 16, kGate>, gemm_grid(a),
                    dim3(16 * kWave), 0, s, a);
    }
    a.ntiles = (a.n4 + 3) / 4;
    if constexpr (kGate)
      return launch(gemm_direct_kernel<4, 4, 8, kGate>, gemm_grid(a),
                    dim3(8 * kWave), 0, s, a);
    else
      return launch(gemm_direct_kernel<4, 8, 8, kGate>, gemm_grid(a),
                    dim3(8 * kWave), 0, s, a);
  }
  // Staged form, M split into 16-row blocks.  About two 256-byte k batches
  // per wave (16 waves for long rows); the gated form holds two weight
  // tiles per wave, so it stays at 8 waves (LDS).
  a.mtiles = (a.M + 15) / 16;
  a.ntiles = (a.n4 + 15) / 16;
  const int nb = (a.K + 255) / 256;
  if (!kGate && nb >= 20)
    return launch(gemm_staged_kernel<16, false>, gemm_grid(a), dim3(16 * kWave), 0,
                  s, a);
  return launch(gemm_staged_kernel<8, kGate>, gemm_grid(a), dim3(8 * kWave), 0, s, a);
}

tq_status gemm_small(const uint8_t *p0, float s0, const uint8_t *p1, float s1,
                     const int8_t *xq, const float *x_scale, int64_t M,
                     int64_t N, int64_t K, float *y, int32_t *acc0,
                     int32_t *acc1, hipStream_t stream) {
  if (M == 1)
    return gemv_m1(p0, s0, p1, s1, xq, x_scale, N, K, y, acc0, acc1, stream);
  DeviceInfo dev;
  if (tq_status s = current_device(&dev)) return s;
  if (!p1 && gemm_dot4_fits(M, K))
    return gemm_dot4(p0, s0, xq, x_scale, M, N, K, y, acc0, dev.num_cus, stream);
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
  a.ntiles = a.mtiles = 0;  // set by the launcher
  return p1 ? launch_gemm<true>(a, dev.num_cus, stream)
            : launch_gemm<false>(a, dev.num_cus, stream);
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
