// tq_gemm_dot4.hip -- the small-batch product for M = 2 activation rows on
// the vector ALU (the M = 1 GEMV's structure with two rows of x).
//
// Page "Blog · field notes" (1bit engine), post "One GPU, many users": one
// GPU serving several requests at once, i.e. a few activation rows per
// weight read.  At M = 2 the work per weight is small: the four plane masks
// of a packed dword are shared by both rows, and each row adds 4 v_dot4
// (0.75 operations per weight), far below the VALU rate at HBM speed, while
// the matrix-core kernel works on a 16-row activation tile that is seven
// eighths empty.
//
// A team of LPR lanes owns one packed row (4 output rows per x row); lane l
// reads pieces l + t*LPR (t < NP); its MR x NP activation pieces are loaded
// once (coalesced: consecutive lanes, consecutive pieces) and held in VGPRs.
// Each x row's code offset sum(q) is folded into the accumulator start, as
// in the GEMV.  Results are bit-identical to the M = 1 GEMV per row.
#include "tq_device.h"
#include "tq_gemv_reg.h"
#include "tq_host.h"

namespace tq {
namespace {

struct Dot4Args {
  const uint8_t *p;      // packed [n4, K]
  float s_w;
  const int8_t *xq;      // [M, K]
  const float *x_scale;  // [M]
  int M, n4, kp;
  float *y;              // [M, N]
  int32_t *acc;          // optional [M, N]
};

template <int LPR, int NP, int MR, bool EXACT>
__global__ __launch_bounds__(reg_block_threads(LPR)) void gemm_dot4_kernel(Dot4Args g) {
  constexpr int BT = reg_block_threads(LPR);
  constexpr int G = BT / LPR;                         // teams per block
  constexpr int GL = LPR < kWave ? LPR : kWave;       // DPP reduction width
  constexpr int WPT = LPR > kWave ? LPR / kWave : 1;  // waves per team
  constexpr int NV = MR * 4;                          // sums per packed row
  __shared__ int red[2][BT / kWave][NV];

  const int kp = g.kp, n4 = g.n4, M = g.M;
  const size_t N = (size_t)n4 * 4;
  const int lane = threadIdx.x % LPR;
  const int team = threadIdx.x / LPR;
  const int wave = threadIdx.x / kWave;
  const int row_stride = gridDim.x * G;
  const int rb0 = blockIdx.x * G;  // < n4 for every launched block
  const int its = (n4 - 1 - rb0) / row_stride + 1;
  const uint4 *P = reinterpret_cast<const uint4 *>(g.p);
  auto piece = [&](int t) {
    const int p = lane + t * LPR;
    return EXACT ? p : min(p, kp - 1);
  };

  // 1. activations (rows past M and pieces past K are zero), then the first
  // row's weights
  uint4 xr[MR][NP];
  const uint4 *X = reinterpret_cast<const uint4 *>(g.xq);
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int t = 0; t < NP; ++t) {
      const int mm = m < M ? m : M - 1;
      xr[m][t] = X[(size_t)mm * kp + piece(t)];
    }
  __builtin_amdgcn_sched_barrier(0);
  auto issue = [&](uint4 (&w)[NP], int rbase) {
    const int row = min(rbase + team, n4 - 1);
    const uint4 *rp = P + (size_t)row * kp;
#pragma unroll
    for (int t = 0; t < NP; ++t) w[t] = load_stream16(rp + piece(t));
  };
  uint4 wa[NP];
  issue(wa, rb0);
  __builtin_amdgcn_sched_barrier(0);

  int init[MR][4];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    int sq = 0;
#pragma unroll
    for (int t = 0; t < NP; ++t) {
      const bool live = m < M && (EXACT || lane + t * LPR < kp);
      if (!live) xr[m][t] = make_uint4(0, 0, 0, 0);
      sq = sum_bytes16(xr[m][t], sq);
    }
    init[m][0] = -sq;
    init[m][1] = -4 * sq;
    init[m][2] = -16 * sq;
    init[m][3] = -16 * sq;
  }
  float c[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) c[m] = g.s_w * g.x_scale[m < M ? m : M - 1];

  int buf = 0;
  auto consume = [&](const uint4 (&w)[NP], int rbase) {
    int a[MR][4];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) a[m][j] = init[m][j];
#pragma unroll
    for (int t = 0; t < NP; ++t) {
      const uint32_t wd[4] = {w[t].x, w[t].y, w[t].z, w[t].w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int p0 = (int)(wd[d] & 0x03030303u);
        const int p1 = (int)(wd[d] & 0x0C0C0C0Cu);
        const int p2 = (int)(wd[d] & 0x30303030u);
        const int p3 = (int)((wd[d] >> 2) & 0x30303030u);
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          const uint32_t xv[4] = {xr[m][t].x, xr[m][t].y, xr[m][t].z, xr[m][t].w};
          const int x = (int)xv[d];
          a[m][0] = __builtin_amdgcn_sdot4(p0, x, a[m][0], false);
          a[m][1] = __builtin_amdgcn_sdot4(p1, x, a[m][1], false);
          a[m][2] = __builtin_amdgcn_sdot4(p2, x, a[m][2], false);
          a[m][3] = __builtin_amdgcn_sdot4(p3, x, a[m][3], false);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) a[m][j] = group_sum_to_last<GL>(a[m][j]);
    const int i = rbase + team;
    auto emit = [&](int m, int j, int v) {
      if (i >= n4 || m >= M) return;
      const int sh = j == 0 ? 0 : (j == 1 ? 2 : 4);
      const int t = v >> sh;  // exact: the sum is a multiple of 1 << sh
      const size_t n = (size_t)m * N + (size_t)j * n4 + i;
      if (g.acc) g.acc[n] = t;
      g.y[n] = rescale(t, c[m]);
    };
    if constexpr (WPT == 1) {
      if (lane == LPR - 1) {
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
          for (int j = 0; j < 4; ++j) emit(m, j, a[m][j]);
      }
    } else {
      if ((threadIdx.x & (kWave - 1)) == kWave - 1) {
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
          for (int j = 0; j < 4; ++j) red[buf][wave][m * 4 + j] = a[m][j];
      }
      __syncthreads();
      if (lane < NV) {
        int v = 0;
#pragma unroll
        for (int w2 = 0; w2 < WPT; ++w2) v += red[buf][team * WPT + w2][lane];
        emit(lane / 4, lane % 4, v);
      }
      buf ^= 1;  // the next row's partials go to the other buffer
    }
  };

  consume(wa, rb0);
  for (int it = 1; it < its; ++it) {
    issue(wa, rb0 + it * row_stride);
    consume(wa, rb0 + it * row_stride);
  }
}

template <int LPR, int NP, int MR>
tq_status launch_np(const RegPlan &pl, const Dot4Args &a, hipStream_t s) {
  const dim3 grid(pl.blocks), block(reg_block_threads(LPR));
  return pl.exact ? launch(gemm_dot4_kernel<LPR, NP, MR, true>, grid, block, 0, s, a)
                  : launch(gemm_dot4_kernel<LPR, NP, MR, false>, grid, block, 0, s, a);
}

template <int LPR, int MR>
tq_status launch_lpr(const RegPlan &pl, const Dot4Args &a, hipStream_t s) {
  switch (pl.np) {
    case 1: return launch_np<LPR, 1, MR>(pl, a, s);
    case 2: return launch_np<LPR, 2, MR>(pl, a, s);
    case 3: return launch_np<LPR, 3, MR>(pl, a, s);
    case 4: return launch_np<LPR, 4, MR>(pl, a, s);
  }
  return TQ_ERR_LAUNCH;
}

template <int MR>
tq_status launch_mr(const RegPlan &pl, const Dot4Args &a, hipStream_t s) {
  switch (pl.lpr) {
    case 16: return launch_lpr<16, MR>(pl, a, s);
    case 32: return launch_lpr<32, MR>(pl, a, s);
    case 64: return launch_lpr<64, MR>(pl, a, s);
    case 128: return launch_lpr<128, MR>(pl, a, s);
    case 256: return launch_lpr<256, MR>(pl, a, s);
  }
  return TQ_ERR_LAUNCH;
}

}  // namespace

// At most 4 pieces per lane (the MR x NP activation pieces stay in VGPRs).
constexpr int kDot4MaxNP = 4;

// Where this path is taken (measured on MI355X, pools of distinct weights):
// M = 2 (4.0 / 4.1 us at [6912,2560] / [2560,6912], against 4.1 / 4.7 us
// for the matrix-core kernel); from M = 3 on the matrix-core kernel is
// faster (4.1 / 4.7 us at M = 3 and 4, against 5.1 / 5.5 us here).
bool gemm_dot4_fits(int64_t M, int64_t K) {
  return M == 2 && K >= 16 && K / 16 <= 256 * kDot4MaxNP;
}

// The narrowest team with at most 4 pieces per lane, 64-lane teams when rows
// are few; persistent blocks, 3 per CU (2 for 512-thread blocks).
tq_status gemm_dot4(const uint8_t *p, float s_w, const int8_t *xq, const float *x_scale,
                    int64_t M, int64_t N, int64_t K, float *y, int32_t *acc,
                    int num_cus, hipStream_t stream) {
  const int64_t n4 = N / 4, kp = K / 16;
  RegPlan pl{};
  int lpr = 16;
  while ((kp + lpr - 1) / lpr > kDot4MaxNP) lpr *= 2;
  if (lpr < 64 && n4 * lpr < (int64_t)num_cus * 16 * kWave) lpr = 64;
  pl.lpr = lpr;
  pl.np = (int)((kp + lpr - 1) / lpr);
  pl.exact = (int64_t)pl.np * lpr == kp;
  const int bt = reg_block_threads(lpr);
  int64_t blocks = (n4 + bt / lpr - 1) / (bt / lpr);
  const int64_t cap = (int64_t)num_cus * (bt == 512 ? 2 : 3);
  if (blocks > cap) blocks = cap;
  pl.blocks = (int)(blocks < 1 ? 1 : blocks);
  Dot4Args a{p, s_w, xq, x_scale, (int)M, (int)n4, (int)kp, y, acc};
  return launch_mr<2>(pl, a, stream);
}

}  // namespace tq
