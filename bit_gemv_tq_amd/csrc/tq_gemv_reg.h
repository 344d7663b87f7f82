// tq_gemv_reg.h -- the M = 1 ternary GEMV with register-resident activations
// (K <= 32768, every decode shape), shared by tq_gemv and the M = 1 branch
// of tq_gate_up_relu2.
//
// Page "the full arc: how the 1bit.systems ternary stack got from broken to
// 76.7 tok/s", TL;DR: a hand-tuned ternary GEMV near the memory-bandwidth
// peak is the decode hot loop.  Page "BitNet" (news digest), first item:
// with weights in {-1,0,1} each product is an add, a subtract or a skip.
//
// Structure (gfx950, wave64).  A team of LPR lanes (16..256) owns one packed
// row at a time (4 output rows, one per plane).  Lane l of a team always
// reads the 16-byte pieces l + t*LPR (t < NP) of a row, so the int8
// activation pieces it needs are the same for every row: they are staged
// once per block through LDS and then held in VGPRs.  The hot loop is NP
// non-temporal 16-byte weight loads per lane and row plus 16 v_dot4 per
// piece (tq_device.h), with no LDS traffic.  Each lane starts its plane
// accumulators at -scale_j * sum(its activation bytes), so after the team
// reduction (DPP inside a wave, LDS across the waves of a 128/256-lane team)
// the code offset is already removed: sum(w*q) = sum((w+1)*q) - sum(q).
// Blocks are persistent and walk rows rb0, rb0 + gridDim*G, ...  All load
// counts are compile-time constants (indices are clamped instead of
// branched), so the compiler's vmcnt waits only cover the data they need:
// activation loads are issued first, then the first row's weight loads.
#pragma once

#include "tq_device.h"
#include "tq_host.h"

namespace tq {

constexpr int kRegThreads = 256;
constexpr int kRegMaxPieces = 2048;  // K <= 32768 bytes

struct RegArgs {
  const uint8_t *p0;  // packed [N/4,K] (gate when kGate)
  const uint8_t *p1;  // packed up (kGate only)
  float s0, s1;       // weight scales
  const int8_t *xq;   // [K]
  const float *x_scale;
  int n4;             // N/4
  int kp;             // K/16
  float *y;           // [N] (h when kGate)
  int32_t *acc0;      // optional [N]
  int32_t *acc1;      // optional [N] (kGate only)
};

template <int LPR, int NP, bool EXACT, bool kGate>
__global__ __launch_bounds__(kRegThreads) void gemv_reg_kernel(RegArgs g) {
  constexpr int NM = kGate ? 2 : 1;
  constexpr int G = kRegThreads / LPR;                // teams per block
  constexpr int GL = LPR < kWave ? LPR : kWave;       // DPP reduction width
  constexpr int WPT = LPR > kWave ? LPR / kWave : 1;  // waves per team
  constexpr int SPAN = NP * LPR;                      // pieces a team covers
  constexpr int SP = (SPAN + kRegThreads - 1) / kRegThreads;  // staging loads
  static_assert(NP >= 1 && SPAN <= kRegMaxPieces, "pieces per lane");
  __shared__ u32x4 x_lds[SP * kRegThreads];  // padded: stores unconditional
  __shared__ int red[2][kRegThreads / kWave][NM][4];

  const int kp = g.kp, n4 = g.n4;
  const int lane = threadIdx.x % LPR;
  const int team = threadIdx.x / LPR;
  const int wave = threadIdx.x / kWave;
  const int row_stride = gridDim.x * G;
  const int rb0 = blockIdx.x * G;  // < n4 for every launched block
  const int its = (n4 - 1 - rb0) / row_stride + 1;

  const uint4 *P[NM];
  P[0] = reinterpret_cast<const uint4 *>(g.p0);
  if constexpr (kGate) P[NM - 1] = reinterpret_cast<const uint4 *>(g.p1);

  // Piece index of slot t for this lane; past the row end it re-reads the
  // last piece (in bounds) and its activation slot is zero.
  auto piece = [&](int t) {
    const int p = lane + t * LPR;
    return EXACT ? p : min(p, kp - 1);
  };

  // 1. Activation loads first (static count).
  // (Native clang vectors: the compiler keeps these in VGPRs.)
  const u32x4 *xg = reinterpret_cast<const u32x4 *>(g.xq);
  u32x4 xs[SP];
#pragma unroll
  for (int s = 0; s < SP; ++s) {
    const int p = (int)threadIdx.x + s * kRegThreads;
    xs[s] = xg[EXACT ? min(p, SPAN - 1) : min(p, kp - 1)];
  }
  // Keep the scheduler from sinking these loads below the weight loads.
  __builtin_amdgcn_sched_barrier(0);

  // 2. Weight loads of the first row.
  auto issue = [&](uint4 (&w)[NM][NP], int rbase) {
    const int row = min(rbase + team, n4 - 1);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const uint4 *rp = P[m] + (size_t)row * kp;
#pragma unroll
      for (int t = 0; t < NP; ++t) w[m][t] = load_stream16(rp + piece(t));
    }
  };
  uint4 wa[NM][NP];
  issue(wa, rb0);
  __builtin_amdgcn_sched_barrier(0);

  // 3. Stage x through LDS; keep this lane's pieces in VGPRs.
#pragma unroll
  for (int s = 0; s < SP; ++s) x_lds[threadIdx.x + s * kRegThreads] = xs[s];
  __syncthreads();
  uint4 xr[NP];
  int sq = 0;
#pragma unroll
  for (int t = 0; t < NP; ++t) {
    const int p = lane + t * LPR;
    const u32x4 v = x_lds[p];
    xr[t] = (EXACT || p < kp) ? make_uint4(v[0], v[1], v[2], v[3])
                              : make_uint4(0, 0, 0, 0);
    sq = sum_bytes16(xr[t], sq);
  }
  // Per-plane accumulator start: -scale_j * (this lane's share of sum(q)).
  const int init[4] = {-sq, -4 * sq, -16 * sq, -16 * sq};

  const float sx = g.x_scale[0];
  const float c0 = g.s0 * sx;
  const float c1 = g.s1 * sx;

  int buf = 0;
  auto consume = [&](uint4 (&w)[NM][NP], int rbase) {
    int a[NM][4];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) a[m][j] = init[j];
#pragma unroll
    for (int t = 0; t < NP; ++t)
#pragma unroll
      for (int m = 0; m < NM; ++m) dot_planes16(w[m][t], xr[t], a[m]);
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) a[m][j] = group_sum_to_last<GL>(a[m][j]);
    const int i = rbase + team;
    auto emit = [&](int j, int v0, int v1) {
      if (i >= n4) return;
      const size_t n = (size_t)j * n4 + i;
      const int sh = j == 0 ? 0 : (j == 1 ? 2 : 4);
      const int t0 = v0 >> sh;  // exact: the sum is a multiple of 1 << sh
      if (g.acc0) g.acc0[n] = t0;
      if constexpr (kGate) {
        const int t1 = v1 >> sh;
        if (g.acc1) g.acc1[n] = t1;
        g.y[n] = relu2_gate(rescale(t0, c0), rescale(t1, c1));
      } else {
        g.y[n] = rescale(t0, c0);
      }
    };
    if constexpr (WPT == 1) {
      if (lane == LPR - 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) emit(j, a[0][j], a[NM - 1][j]);
      }
    } else {
      if ((threadIdx.x & (kWave - 1)) == kWave - 1) {
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int j = 0; j < 4; ++j) red[buf][wave][m][j] = a[m][j];
      }
      __syncthreads();
      if (lane < 4) {
        int v[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          v[m] = 0;
#pragma unroll
          for (int w2 = 0; w2 < WPT; ++w2) v[m] += red[buf][team * WPT + w2][m][lane];
        }
        emit(lane, v[0], v[NM - 1]);
      }
      buf ^= 1;  // the next row's partials go to the other buffer
    }
  };

  // 4. Row iterations: `its` is block-uniform, so every wave reaches the
  // same barriers.  (Other resident blocks hide this wave's load latency;
  // measured on MI355X, that beat a software prefetch of the next row,
  // which costs registers and so occupancy.)
  consume(wa, rb0);
  for (int it = 1; it < its; ++it) {
    issue(wa, rb0 + it * row_stride);
    consume(wa, rb0 + it * row_stride);
  }
}

// Launch one instantiation family (defined per LPR in tq_gemv_reg_l*.hip).
struct RegPlan {
  int lpr, np, blocks;
  bool exact;
};

template <int LPR>
tq_status launch_reg(const RegPlan &pl, bool gate, const RegArgs &a,
                     hipStream_t s);

#define TQ_REG_KERNEL(LPR, NPV, GATE)                                          \
  (pl.exact ? gemv_reg_kernel<LPR, NPV, true, GATE>                            \
            : gemv_reg_kernel<LPR, NPV, false, GATE>)

#define TQ_REG_NP_CASES(LPR, GATE)                                             \
  switch (pl.np) {                                                             \
    case 1: return launch(TQ_REG_KERNEL(LPR, 1, GATE), grid, block, 0, s, a);  \
    case 2: return launch(TQ_REG_KERNEL(LPR, 2, GATE), grid, block, 0, s, a);  \
    case 3: return launch(TQ_REG_KERNEL(LPR, 3, GATE), grid, block, 0, s, a);  \
    case 4: return launch(TQ_REG_KERNEL(LPR, 4, GATE), grid, block, 0, s, a);  \
    case 5: return launch(TQ_REG_KERNEL(LPR, 5, GATE), grid, block, 0, s, a);  \
    case 6: return launch(TQ_REG_KERNEL(LPR, 6, GATE), grid, block, 0, s, a);  \
    case 7: return launch(TQ_REG_KERNEL(LPR, 7, GATE), grid, block, 0, s, a);  \
    case 8: return launch(TQ_REG_KERNEL(LPR, 8, GATE), grid, block, 0, s, a);  \
  }                                                                            \
  return TQ_ERR_LAUNCH;

#define TQ_DEFINE_LAUNCH_REG(LPR)                                              \
  template <>                                                                  \
  tq_status launch_reg<LPR>(const RegPlan &pl, bool gate, const RegArgs &a,    \
                            hipStream_t s) {                                   \
    const dim3 grid(pl.blocks), block(kRegThreads);                            \
    if (gate) {                                                                \
      TQ_REG_NP_CASES(LPR, true)                                               \
    }                                                                          \
    TQ_REG_NP_CASES(LPR, false)                                                \
  }

}  // namespace tq
