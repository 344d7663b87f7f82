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
// same k block (l / 16), so which k a byte stands for is free as long as A
// and B agree.  B columns are activation rows.
//
// Quad form.  MFMA row r = 4a + j is plane j of packed row a of a "quad" (4
// packed rows = 16 output rows).  A wave works on 256-byte k groups (four
// MFMA steps of 64).  Lane (kb, a, j) loads the 16 bytes of packed row a at
// group offset 64j + 16kb, so one load instruction covers 4 rows x 256
// contiguous bytes and every weight byte is loaded once.  For step u (group
// offset 64u + 16kb) lane (kb, a, j) takes the dwords of lane (kb, a, u) of
// its quad by a DPP quad broadcast folded into the AND that isolates its own
// plane: one VALU operation per dword.  The planes are used as offset codes
// c = w + 1 at scales 1, 4, 16 and, for plane 3, 64(c - 2) (bit 7 of every
// byte is flipped once per load, so the masked byte stays a valid int8); a
// fifth MFMA per step with A = all ones gives sum(x) per column, and
//   sum(w x) = D0 - S = D1/4 - S = D2/16 - S = D3/64 + S   (exact shifts).
// Activations are loaded 4 rows x 256 contiguous bytes per instruction and
// written to a wave-private LDS tile with a swizzle (piece c of row m at
// slot (c + m) mod 16) that makes both the writes and the MFMA-layout reads
// free of bank conflicts.
//
// A block owns RG quads and one 16-row activation tile; its W waves split K
// into groups (NQ per wave and pass, every load of a pass issued before the
// first MFMA).  Per-wave partial tiles are summed in LDS (padded slots,
// conflict free) and rescaled by RG * 64 threads.  Blocks map to tiles
// XCD-aware: each XCD takes a contiguous run of tiles, the activation tiles
// of one weight tile adjacent, so those share the weight tile in that XCD's
// L2 and neighbouring tiles' partial output lines merge there.
#include <algorithm>

#include "tq_device.h"
#include "tq_host.h"

namespace tq {

tq_status gemv_m1(bool gate, const uint8_t *p0, float s0, const uint8_t *p1, float s1,
                  const int8_t *xq, const float *x_scale, int64_t N, int64_t K,
                  float *y, int32_t *acc0, int32_t *acc1, hipStream_t stream);
// M = 2 on the vector ALU (tq_gemm_dot4.hip).
bool gemm_dot4_fits(int64_t M, int64_t K);
tq_status gemm_dot4(const uint8_t *p, float s_w, const int8_t *xq, const float *x_scale,
                    int64_t M, int64_t N, int64_t K, float *y, int32_t *acc,
                    int num_cus, hipStream_t stream);

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kXcds = 8;         // MI355X: 8 XCDs, blocks dispatched round-robin
constexpr int kGroup = 256;      // k bytes per group (4 MFMA steps)
constexpr int kTileSlots = 256;  // 16-byte slots of one 16-row x 256-byte tile
constexpr int kSlotPad = 17;     // padded stride of the partial tiles
constexpr int kLdsBytes = 160 * 1024;

struct GemmArgs {
  const uint8_t *p0, *p1;
  float s0, s1;
  const int8_t *xq;
  const float *x_scale;
  int M, n4, K;
  float *y;
  int32_t *acc0, *acc1;
  int ntiles, mtiles;  // quad tiles, 16-row activation tiles
  int per_xcd;         // blocks per XCD
};

// Block -> (weight tile, activation tile); false for padding blocks (the
// whole block exits before any barrier).
__device__ __forceinline__ bool block_tile(const GemmArgs &g, int &tile, int &mt) {
  const int b = blockIdx.x;
  const int t = (b % kXcds) * g.per_xcd + b / kXcds;
  tile = t / g.mtiles;
  mt = t % g.mtiles;
  return tile < g.ntiles;
}

// Lane U of each group of 4 lanes, to all 4 (DPP quad_perm [U,U,U,U]).
template <int U>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v) {
  constexpr int ctrl = U | (U << 2) | (U << 4) | (U << 6);
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, ctrl, 0xF, 0xF, true);
}

__device__ __forceinline__ v4i as_v4i(const u32x4 &v) {
  return v4i{(int)v[0], (int)v[1], (int)v[2], (int)v[3]};
}

// MFMA step U of group s: every quad of every matrix, then the ones column.
template <int U, int NQ, int NM, int RG>
__device__ __forceinline__ void quad_step(const u32x4 (&w)[NQ][NM][RG], int s, const v4i &b,
                                          uint32_t mask, v4i (&acc)[NM][RG], v4i &ones) {
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int q = 0; q < RG; ++q) {
      v4i a;
#pragma unroll
      for (int d = 0; d < 4; ++d) a[d] = (int)(quad_bcast<U>(w[s][m][q][d]) & mask);
      acc[m][q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[m][q], 0, 0, 0);
    }
  ones = __builtin_amdgcn_mfma_i32_16x16x64_i8(
      v4i{0x01010101, 0x01010101, 0x01010101, 0x01010101}, b, ones, 0, 0, 0);
}

// Partial tiles: slot ((m RG + q) 4 + kb) kSlotPad + r, then the wave:
// [slot][quad_wave_stride(W)].  The stride is odd, so 8 consecutive lanes
// (one LDS cycle of 16-byte accesses) hit 8 bank groups on the writes (one
// wave, consecutive r) and on the reads (consecutive slots of 17), and the
// W partials of a slot are one address plus immediate offsets.
__host__ __device__ constexpr int quad_wave_stride(int w) { return w | 1; }

// LDS: [W][NQ][kTileSlots] activation tiles, then the partial tiles and
// MAXW slots of slack (reads past the last wave).  blockDim.x = 64 W, W <=
// MAXW.
template <int RG, int NQ, bool kGate, int MAXW>
__global__ __launch_bounds__(MAXW *kWave) void gemm_quad_kernel(GemmArgs g) {
  constexpr int NM = kGate ? 2 : 1;
  extern __shared__ u32x4 lds[];
  int tile, mt;
  if (!block_tile(g, tile, mt)) return;
  const int W = blockDim.x / kWave;
  __builtin_assume(W >= 1 && W <= MAXW);
  const int PS = quad_wave_stride(W);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int kb = lane >> 4, r = lane & 15, j = r & 3;
  const int K = g.K, n4 = g.n4, M = g.M;
  const int m0 = mt * 16, i0 = tile * 4 * RG;
  u32x4 *xt = lds + (size_t)wave * NQ * kTileSlots;
  v4i *part = reinterpret_cast<v4i *>(lds + (size_t)W * NQ * kTileSlots);

  const uint8_t *wr[NM][RG];  // this lane's packed row of each quad
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int q = 0; q < RG; ++q)
      wr[m][q] = (m == 0 ? g.p0 : g.p1) + (size_t)min(i0 + 4 * q + (r >> 2), n4 - 1) * K;
  // plane j of a flipped byte: c, 4c, 16c, or 64(c - 2) for plane 3
  const uint32_t mask = j == 3 ? 0xC0C0C0C0u : (0x03030303u << (2 * j));

  v4i acc[NM][RG], ones = v4i{0, 0, 0, 0};
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int q = 0; q < RG; ++q) acc[m][q] = v4i{0, 0, 0, 0};

  // The epilogue's activation scale for this thread's first output slot,
  // loaded now: its latency hides behind the main loop instead of following
  // the final barrier.
  float sx_first = 0.0f;
  if ((int)threadIdx.x < RG * 64)
    sx_first = g.x_scale[min(m0 + (int)threadIdx.x / (4 * RG), M - 1)];

  const int groups = (K + kGroup - 1) / kGroup;
  for (int g0 = wave * NQ; g0 < groups; g0 += W * NQ) {
    // 1. Every load of the pass.  Past K (a ragged last group, or groups past
    // the end) weights re-read offset 0 and activations are zeroed below.
    u32x4 w[NQ][NM][RG], xv[NQ][4];
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
      const int kw = (g0 + s) * kGroup + 64 * j + 16 * kb;
      const int kc = kw < K ? kw : 0;
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int q = 0; q < RG; ++q)
          w[s][m][q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wr[m][q] + kc));
    }
#pragma unroll
    for (int s = 0; s < NQ; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // tile row `row`, slot lane & 15: piece (slot - row) mod 16 of the group
        const int row = 4 * i + (lane >> 4);
        const int k = (g0 + s) * kGroup + 16 * (((lane & 15) - row) & 15);
        const int8_t *xr = g.xq + (size_t)min(m0 + row, M - 1) * K;
        xv[s][i] = *reinterpret_cast<const u32x4 *>(xr + (k < K ? k : 0));
      }
    // Keep the loads ahead of the first MFMA.
    __builtin_amdgcn_sched_barrier(0);
    // 2. Activation tiles to LDS (rows past M and k past K as zeros).
#pragma unroll
    for (int s = 0; s < NQ; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * i + (lane >> 4);
        const int k = (g0 + s) * kGroup + 16 * (((lane & 15) - row) & 15);
        xt[s * kTileSlots + 64 * i + lane] =
            (m0 + row < M && k < K) ? xv[s][i] : u32x4{0, 0, 0, 0};
      }
    // The tile is private to this wave and a wave's LDS accesses complete in
    // order; this keeps the compiler from moving accesses across.
    __builtin_amdgcn_wave_barrier();
    // 3. Decode and multiply.
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int q = 0; q < RG; ++q)
#pragma unroll
          for (int d = 0; d < 4; ++d) w[s][m][q][d] ^= 0x80808080u;
      v4i b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        b[u] = as_v4i(xt[s * kTileSlots + 16 * r + ((4 * u + kb + r) & 15)]);
      quad_step<0>(w, s, b[0], mask, acc, ones);
      quad_step<1>(w, s, b[1], mask, acc, ones);
      quad_step<2>(w, s, b[2], mask, acc, ones);
      quad_step<3>(w, s, b[3], mask, acc, ones);
    }
    __builtin_amdgcn_wave_barrier();
  }

  // 4. True sums of this wave's k range (D element i of lane l: plane i of
  // packed row i0 + 4q + l/16, activation row m0 + l % 16).
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int q = 0; q < RG; ++q) {
      v4i v = acc[m][q];
      v[0] = v[0] - ones[0];
      v[1] = (v[1] >> 2) - ones[1];
      v[2] = (v[2] >> 4) - ones[2];
      v[3] = (v[3] >> 6) + ones[3];
      part[(((m * RG + q) * 4 + kb) * kSlotPad + r) * PS + wave] = v;
    }
  __syncthreads();
  // 5. Cross-wave sums (exact) and the epilogue.  Thread t: packed row
  // i0 + 4q + aa, activation row m0 + mm; consecutive threads, consecutive
  // output columns.  The scale is read before the stores (y may alias it).
  const size_t N = (size_t)n4 * 4;
  for (int t = threadIdx.x; t < RG * 64; t += blockDim.x) {
    const int aa = t & 3, q = (t >> 2) % RG, mm = t / (4 * RG);
    v4i v[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      v[m] = v4i{0, 0, 0, 0};
      // 8 reads in flight at a time; those past W (the next slot or the
      // slack) add nothing
      const v4i *ps = part + (((m * RG + q) * 4 + aa) * kSlotPad + mm) * PS;
#pragma unroll
      for (int c = 0; c < MAXW; c += 8) {
        v4i pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) pv[j] = ps[c + j];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[m] += c + j < W ? pv[j] : v4i{0, 0, 0, 0};
      }
    }
    const int p = i0 + 4 * q + aa, m = m0 + mm;
    if (p >= n4 || m >= M) continue;
    const float sx = t == (int)threadIdx.x ? sx_first : g.x_scale[m];
    const float c0 = g.s0 * sx, c1 = g.s1 * sx;
    const size_t o = (size_t)m * N + p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t oi = o + (size_t)i * n4;
      if (g.acc0) g.acc0[oi] = v[0][i];
      if constexpr (kGate) {
        if (g.acc1) g.acc1[oi] = v[NM - 1][i];
        g.y[oi] = relu2_gate(rescale(v[0][i], c0), rescale(v[NM - 1][i], c1));
      } else {
        g.y[oi] = rescale(v[0][i], c0);
      }
    }
  }
}

// ------------------------------------------------------------ launch
struct QuadPlan {
  int rg, nq, w;
};

// Largest NQ whose kernel stays within the register budget of its launch
// bound without spilling: 128 VGPRs for blocks of up to 16 waves, 256 for up
// to 8 (the compiler's gfx950 register counts of every RG x NQ x form; 0:
// no NQ fits; the gated form's epilogue alone needs more than 128).
constexpr int quad_max_nq(int nm, int rg, int maxw) {
  if (maxw > 8) return nm == 1 ? (rg == 1 ? 3 : rg == 2 ? 2 : rg <= 4 ? 1 : 0) : 0;
  return nm == 1 ? (rg <= 4 ? 4 : 3) : (rg <= 2 ? 4 : rg <= 4 ? 3 : 1);
}

constexpr int quad_lds(int rg, int nq, int nm, int w) {
  return w * nq * kTileSlots * 16 +
         (nm * rg * 4 * kSlotPad * quad_wave_stride(w) + (w > 8 ? 16 : 8)) * 16;
}

// Quads per block: the RG (of those instantiated) that moves the fewest
// bytes through the busiest CU, i.e. blocks per CU (rounded up) times the
// K x (4 RG nm + 16) bytes of weights and activation tile one block reads
// (operand arrival, set by how fast a CU's L1 fills, dominates a pass).
// Ties go to the larger RG.  This keeps the earlier plans (RG = 2 / 4 / 8 at
// M <= 16 / 32 / 64 for [6912,2560], RG = 1 / 2 at M <= 16 / 32 for
// [2560,6912]) and takes RG = 3 at M = 64 for [2560,6912] (216 blocks of
// 193 KB instead of 160 of 221 KB; measured on MI355X 7.6 against 8.1 us,
// the gated pair 9.6 against 10.6 us) and, for the gated pair, RG = 8 at
// M = 48 and 64 for [6912,2560] (one block per CU instead of two on most:
// 10.1 / 10.3 against 11.0 / 11.9-12.6 us; 231 VGPRs, no spills).  Then one
// group per wave and pass, with as many waves as the register table above
// and the LDS allow.
constexpr int kQuadRgs[] = {8, 4, 3, 2, 1};

QuadPlan plan_quad(int64_t M, int64_t n4, int64_t K, bool gate, int num_cus, int &mtiles) {
  const int nm = gate ? 2 : 1;
  mtiles = (int)((M + 15) / 16);
  QuadPlan pl{1, 1, 1};
  int64_t best = -1;
  for (int rg : kQuadRgs) {
    if (rg * nm > 16) continue;
    const int64_t blocks = (n4 + 4 * rg - 1) / (4 * rg) * mtiles;
    const int64_t cost = (blocks + num_cus - 1) / num_cus * (4 * rg * nm + 16);
    if (best < 0 || cost < best) {
      best = cost;
      pl.rg = rg;
    }
  }
  auto fits = [&](int nq, int w) {
    return nq <= quad_max_nq(nm, pl.rg, w > 8 ? 16 : 8) &&
           quad_lds(pl.rg, nq, nm, w) <= kLdsBytes;
  };
  // One 256-byte group per wave and pass, as many waves as the registers
  // and LDS allow (up to one per group): more waves hide more latency than
  // more groups per wave do.  Measured on MI355X, M = 64: [6912,2560]
  // 6.4-6.5 us with 8 waves of one group (two passes) against 7.7-8.1 us
  // with 5 waves of two (one pass); [2560,6912] 7.6-7.9 against 7.9-8.2 us
  // with 16 waves of one group against 7 of four.
  const int64_t groups = (K + kGroup - 1) / kGroup;
  int w = (int)std::min<int64_t>(16, std::max<int64_t>(1, groups));
  while (w > 1 && !fits(1, w)) --w;
  pl.nq = 1;
  pl.w = w;
  return pl;
}

template <int RG, int NQ, bool kGate, int MAXW>
tq_status launch_quad(const QuadPlan &pl, const GemmArgs &a, dim3 grid, hipStream_t s) {
  if constexpr (NQ > quad_max_nq(kGate ? 2 : 1, RG, MAXW)) {
    return TQ_ERR_LAUNCH;  // never planned
  } else {
    auto k = gemm_quad_kernel<RG, NQ, kGate, MAXW>;
    const int bytes = quad_lds(RG, NQ, kGate ? 2 : 1, pl.w);
    if (tq_status e = allow_dynamic_lds(reinterpret_cast<const void *>(k), bytes)) return e;
    return launch(k, grid, dim3(pl.w * kWave), bytes, s, a);
  }
}

template <int RG, int NQ, bool kGate>
tq_status launch_quad_w(const QuadPlan &pl, const GemmArgs &a, dim3 grid, hipStream_t s) {
  return pl.w <= 8 ? launch_quad<RG, NQ, kGate, 8>(pl, a, grid, s)
                   : launch_quad<RG, NQ, kGate, 16>(pl, a, grid, s);
}

template <int RG, bool kGate>
tq_status launch_quad_nq(const QuadPlan &pl, const GemmArgs &a, dim3 grid, hipStream_t s) {
  // The planner takes one group per wave and pass (NQ = 1).
  return pl.nq == 1 ? launch_quad_w<RG, 1, kGate>(pl, a, grid, s) : TQ_ERR_LAUNCH;
}

template <bool kGate>
tq_status launch_gemm(GemmArgs a, int num_cus, hipStream_t s) {
  const QuadPlan pl = plan_quad(a.M, a.n4, a.K, kGate, num_cus, a.mtiles);
  a.ntiles = (a.n4 + 4 * pl.rg - 1) / (4 * pl.rg);
  // Blocks per XCD: a whole number of activation tiles per weight tile.
  int per = (a.ntiles * a.mtiles + kXcds - 1) / kXcds;
  per = (per + a.mtiles - 1) / a.mtiles * a.mtiles;
  a.per_xcd = per;
  const dim3 grid((unsigned)(per * kXcds));
  switch (pl.rg) {
    case 1: return launch_quad_nq<1, kGate>(pl, a, grid, s);
    case 2: return launch_quad_nq<2, kGate>(pl, a, grid, s);
    case 3: return launch_quad_nq<3, kGate>(pl, a, grid, s);
    case 4: return launch_quad_nq<4, kGate>(pl, a, grid, s);
    case 8: return launch_quad_nq<8, kGate>(pl, a, grid, s);
  }
  return TQ_ERR_LAUNCH;
}

tq_status gemm_small(bool gate, const uint8_t *p0, float s0, const uint8_t *p1, float s1,
                     const int8_t *xq, const float *x_scale, int64_t M,
                     int64_t N, int64_t K, float *y, int32_t *acc0,
                     int32_t *acc1, hipStream_t stream) {
  if (M == 1)
    return gemv_m1(gate, p0, s0, p1, s1, xq, x_scale, N, K, y, acc0, acc1, stream);
  DeviceInfo dev;
  if (tq_status s = current_device(&dev)) return s;
  if (!gate && gemm_dot4_fits(M, K))
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
  a.ntiles = a.mtiles = a.per_xcd = 0;  // set by the launcher
  return gate ? launch_gemm<true>(a, dev.num_cus, stream)
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
  return gemm_small(false, packed, w_scale, nullptr, 0.0f, xq, x_scale, M, N, K, y,
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
  return gemm_small(true, packed_gate, s_gate, packed_up, s_up, xq, x_scale, M, N, K, h,
                    acc_gate, acc_up, stream);
}
