// tq_gemv.hip -- the ternary matrix-vector product at M = 1 (tq_gemv) and
// the M = 1 dispatch of the fused gate/up + squared-ReLU projection.
//
// Page "the full arc: how the 1bit.systems ternary stack got from broken to
// 76.7 tok/s", TL;DR: a hand-tuned ternary GEMV running close to the memory-
// bandwidth peak is the decode hot loop.  Page "BitNet" (news digest), first
// item: with weights in {-1,0,1} every product is an add, a subtract or a
// skip.  Page "Feature request: BitNet 1.58-bit ternary inference on ROCm
// (gfx1151)", section "Architecture": the MLP gate is relu_squared.
//
// Two kernels.  For 1 <= K <= 32768 (every decode shape) the register-
// resident kernel of tq_gemv_reg.h runs: activations staged once per block
// and held in VGPRs, the packed weights streamed once with 16-byte
// non-temporal loads.  For K == 0 and K > 32768 the kernel below keeps the
// int8 activation row in LDS (dynamic, up to 128 KiB) and reads it per
// 16-byte piece: lane groups of LPR lanes own ROWS packed rows at a time and
// walk K in strides of 16*LPR bytes, UNR pieces per lane in flight.
#include "tq_device.h"
#include "tq_gemv_reg.h"
#include "tq_host.h"

namespace tq {
namespace {

constexpr int kGemvThreads = 256;

struct GemvArgs {
  const uint8_t *p0;   // packed [N/4,K] (gate when kGate)
  const uint8_t *p1;   // packed up (kGate only)
  float s0, s1;        // weight scales
  const int8_t *xq;    // [K]
  const float *x_scale;
  int n4;              // N/4
  int kp;              // K/16
  float *y;            // [N] (h when kGate)
  int32_t *acc0;       // optional [N]
  int32_t *acc1;       // optional [N] (kGate only)
};

template <int LPR, int ROWS, int UNR, bool kGate>
__global__ __launch_bounds__(kGemvThreads) void gemv_m1_kernel(GemvArgs g) {
  constexpr int NM = kGate ? 2 : 1;      // weight streams
  constexpr int G = kGemvThreads / LPR;  // lane groups per block
  extern __shared__ uint4 x_lds[];       // K/16 pieces of int8 activations
  __shared__ int sumq_lds[kGemvThreads / kWave];

  const int kp = g.kp;
  // Stage x once per block and form sum(q) for the code offset.
  int sq = 0;
  const uint4 *xg = reinterpret_cast<const uint4 *>(g.xq);
  for (int p = threadIdx.x; p < kp; p += kGemvThreads) {
    const uint4 v = xg[p];
    x_lds[p] = v;
    sq = sum_bytes16(v, sq);
  }
  sq = wave_sum(sq);
  if ((threadIdx.x & (kWave - 1)) == 0) sumq_lds[threadIdx.x / kWave] = sq;
  __syncthreads();
  int sumq = 0;
#pragma unroll
  for (int w = 0; w < kGemvThreads / kWave; ++w) sumq += sumq_lds[w];

  const float sx = g.x_scale[0];
  const float c0 = g.s0 * sx;
  const float c1 = g.s1 * sx;

  const int lane = threadIdx.x % LPR;
  const int group = threadIdx.x / LPR;
  const int stride = gridDim.x * G * ROWS;
  const uint4 *P[NM];
  P[0] = reinterpret_cast<const uint4 *>(g.p0);
  if constexpr (kGate) P[NM - 1] = reinterpret_cast<const uint4 *>(g.p1);

  for (int r0 = (blockIdx.x * G + group) * ROWS; r0 < g.n4; r0 += stride) {
    int a[NM][ROWS][4];
    const uint4 *row[NM][ROWS];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        a[m][r][0] = a[m][r][1] = a[m][r][2] = a[m][r][3] = 0;
        const int rr = min(r0 + r, g.n4 - 1);  // rows past the end: reread
        row[m][r] = P[m] + (size_t)rr * kp;
      }

    for (int p0 = lane; p0 < kp; p0 += LPR * UNR) {
      uint4 w[NM][ROWS][UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int p = p0 + u * LPR;
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int r = 0; r < ROWS; ++r)
            w[m][r][u] = p < kp ? load_stream16(row[m][r] + p)
                                : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int p = min(p0 + u * LPR, kp - 1);  // w is zero past the end
        const uint4 xv = x_lds[p];
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int r = 0; r < ROWS; ++r) dot_planes16(w[m][r][u], xv, a[m][r]);
      }
    }

#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int r = 0; r < ROWS; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) a[m][r][j] = group_sum_to_last<LPR>(a[m][r][j]);

    if (lane == LPR - 1) {
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        const int i = r0 + r;
        if (i >= g.n4) break;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const size_t n = (size_t)j * g.n4 + i;
          const int v0 = plane_value(j, a[0][r][j], sumq);
          if (g.acc0) g.acc0[n] = v0;
          if constexpr (kGate) {
            const int v1 = plane_value(j, a[NM - 1][r][j], sumq);
            if (g.acc1) g.acc1[n] = v1;
            g.y[n] = relu2_gate(rescale(v0, c0), rescale(v1, c1));
          } else {
            g.y[n] = rescale(v0, c0);
          }
        }
      }
    }
  }
}

struct GemvPlan {
  int lpr;
  int rows;
  int unr;
  int blocks;
};

GemvPlan plan_gemv_lds(int64_t n4, int64_t kp, int num_cus, int nm) {
  GemvPlan pl{};
  if (kp % 64 == 0) pl.lpr = 64;
  else if (kp % 32 == 0) pl.lpr = 32;
  else if (kp % 16 == 0) pl.lpr = 16;
  else pl.lpr = kp >= 256 ? 64 : 16;
  pl.rows = nm == 1 ? 2 : 1;
  pl.unr = 4;
  const int64_t groups = kGemvThreads / pl.lpr;
  const int64_t batches = (n4 + pl.rows - 1) / pl.rows;
  const int64_t k_bytes = kp * 16;
  int64_t per_cu = k_bytes > 0 ? (160 * 1024) / (k_bytes + 64) : 8;
  if (per_cu > 8) per_cu = 8;
  if (per_cu < 1) per_cu = 1;
  const int64_t cap = (int64_t)num_cus * per_cu;
  const int64_t iters = (batches + groups * cap - 1) / (groups * cap);
  int64_t blocks = (batches + groups * iters - 1) / (groups * iters);
  if (blocks < 1) blocks = 1;
  pl.blocks = (int)blocks;
  return pl;
}

template <bool kGate>
tq_status launch_gemv_lds(const GemvPlan &pl, const GemvArgs &a, size_t lds,
                          hipStream_t s) {
  const dim3 grid(pl.blocks), block(kGemvThreads);
#define TQ_GEMV_CASE(L, R, U)                                              \
  if (pl.lpr == L && pl.rows == R && pl.unr == U) {                        \
    auto k = gemv_m1_kernel<L, R, U, kGate>;                               \
    if (tq_status st = allow_dynamic_lds((const void *)k, (int)lds))       \
      return st;                                                           \
    return launch(k, grid, block, lds, s, a);                              \
  }
  TQ_GEMV_CASE(64, 2, 4)
  TQ_GEMV_CASE(32, 2, 4)
  TQ_GEMV_CASE(16, 2, 4)
  TQ_GEMV_CASE(64, 1, 4)
  TQ_GEMV_CASE(32, 1, 4)
  TQ_GEMV_CASE(16, 1, 4)
#undef TQ_GEMV_CASE
  return TQ_ERR_LAUNCH;
}

}  // namespace

// Register-path plan (from launch-shape sweeps on MI355X): the narrowest
// team that keeps at most 8 pieces per lane; 64-lane teams when that would
// leave the chip short of busy lanes (small N).  Persistent blocks, about
// 3 per CU (2 for the two-stream gate kernel).  Grids that give every team
// exactly the same number of rows measured slower (all waves reach their
// reductions at once), so the grid is not trimmed to a balanced count.
RegPlan plan_gemv_reg(int64_t n4, int64_t kp, int num_cus, bool gate, int xt) {
  RegPlan pl{};
  int lpr = 16;
  while ((kp + lpr - 1) / lpr > 8) lpr *= 2;
  const int64_t want_lanes = (int64_t)num_cus * 16 * kWave;
  // Narrow teams hold more loads per lane; where they give too few lanes the
  // teams are widened to 64 lanes -- except in the two-matrix gate form with
  // a raw (bf16/fp32) row, when 32-lane teams still fill 3/4 to all of the
  // CUs with one block each: half the blocks quantize the row in their
  // prologue.  Measured at the 2B-4T MLP, [6912,2560] x 2, fp32 row: 32-lane
  // teams on 216 blocks 4.24 us against 5.44 us for 64-lane teams on 432
  // blocks (kernel trace); with an int8 row the 64-lane plan stays faster
  // (4.3 against 4.5 us).
  const int64_t narrow_blocks = n4 / (kRegThreads / 32);
  const bool keep_narrow = gate && xt != kXInt8 && lpr == 32 &&
                           narrow_blocks * 4 >= (int64_t)num_cus * 3 &&
                           narrow_blocks <= num_cus;
  if (lpr < 64 && n4 * lpr < want_lanes && !keep_narrow) lpr = 64;
  pl.lpr = lpr;
  pl.np = (int)((kp + lpr - 1) / lpr);
  pl.exact = (int64_t)pl.np * lpr == kp;
  const int bt = gemv_block_threads(lpr, xt);
  const int64_t teams = bt / lpr;
  int64_t blocks = (n4 + teams - 1) / teams;
  // Resident blocks per CU (persistent grid): 12 waves per CU, measured best
  // on MI355X (at [8192,28672], 256-lane teams: 3 one-team blocks per CU
  // took 12.7 / 11.1 us with the bf16 / int8 row against 13.5 / 11.4 us for
  // 2 two-team blocks and 14.2 / 12.3 us for 4 one-team blocks); the
  // two-plane gate kernel holds more registers, 2 per CU; the 512-thread
  // fp32 and RMSNorm forms 2 and 1 (what their registers allow).  The
  // launcher lowers a persistent grid further where the compiled kernel
  // fits fewer blocks (launch_resident).
  // The gate form with short rows (at most 4 pieces per lane) takes 3
  // blocks per CU: measured on MI355X, [28672,4096] x 2 11.3 against
  // 12.2 us (int8 row), [24576,3072] x 2 8.4 against 9.2 us, [14336,4096] x 2
  // 7.5 against 7.9 us; from 5 pieces up 2 per CU stayed level or faster
  // ([28672,8192] x 2: 20.4 against 21.0 us).
  // Likewise the single-matrix form takes 4 blocks per CU with short rows:
  // [28672,4096] 7.2 against 7.5 us, [24576,3072] 5.5-5.7 against
  // 5.8-5.9 us, [49152,2048] 7.6-7.7 against 7.8-8.2 us (level at
  // [57344,4096] and [32768,4096]).
  const int gate_per_cu = pl.np <= 4 ? 3 : 2;
  const int plain_per_cu = pl.np <= 4 ? 4 : 3;
  const int per_cu = bt == 512 ? (gate || xt_rms(xt) ? 1 : 2) : (gate ? gate_per_cu : plain_per_cu);
  const int64_t cap = (int64_t)num_cus * per_cu;
  // One row per team when that takes at most one more block per CU than
  // the persistent grid: otherwise a few teams per CU walk a second row
  // while the rest idle (at [14336,4096], 3584 rows on 3072 teams: 6.2 us
  // against 5.4 us with 896 blocks of one row per team).
  const bool one_round = bt == kRegThreads && !gate &&
                         blocks <= (int64_t)num_cus * (per_cu + 1);
  pl.persistent = blocks > cap && !one_round;
  if (pl.persistent) blocks = cap;
  pl.blocks = (int)(blocks < 1 ? 1 : blocks);
  pl.cus = num_cus;
  // Rows by dispatch round, for one-team blocks that quantize a bf16 row in
  // the prologue.  The dispatcher places blocks breadth first (block b on a
  // CU in round b / CUs), and on MI355X the second and third block of a CU
  // receive their activation row 2.4 and 4.5 us after the first, behind that
  // block's weight misses (per-block timestamps at [8192,28672]).  Rows are
  // therefore split 4 : 3 : 1 between the rounds instead of evenly: 13.2-13.3
  // against 13.5-13.6 us per back-to-back launch there.  Only where every
  // block of every round gets a row (n4 >= 8 per CU) and the grid is exactly
  // three rounds.  (The int8 row arrives early enough in every round: a
  // split by round measured 0.3 us slower for tq_gemv.)  Which block takes
  // which row does not change any result.
  if (lpr == 256 && bt == kRegThreads && xt == kXBf16 && !gate &&
      pl.blocks == 3 * num_cus && n4 >= 8 * (int64_t)num_cus) {
    pl.round_cus = num_cus;
    pl.round_end0 = (int)(n4 * 4 / 8);
    pl.round_end1 = (int)(n4 * 7 / 8);
  }
  return pl;
}

tq_status launch_gemv_reg(const RegPlan &pl, bool gate, int xt,
                          const RegArgs &args, hipStream_t s) {
  RegArgs a = args;
  a.round_cus = pl.round_cus;
  a.round_end0 = pl.round_end0;
  a.round_end1 = pl.round_end1;
  switch (pl.lpr) {
    case 16: return launch_reg<16>(pl, gate, xt, a, s);
    case 32: return launch_reg<32>(pl, gate, xt, a, s);
    case 64: return launch_reg<64>(pl, gate, xt, a, s);
    case 128: return launch_reg<128>(pl, gate, xt, a, s);
    case 256: return launch_reg<256>(pl, gate, xt, a, s);
  }
  return TQ_ERR_LAUNCH;
}

// Shared by tq_gemv and the M = 1 branch of tq_gate_up_relu2 (gate: the
// two-matrix form, p1 the up projection).
tq_status gemv_m1(bool gate, const uint8_t *p0, float s0, const uint8_t *p1, float s1,
                  const int8_t *xq, const float *x_scale, int64_t N, int64_t K,
                  float *y, int32_t *acc0, int32_t *acc1, hipStream_t stream) {
  DeviceInfo dev;
  if (tq_status s = current_device(&dev)) return s;
  const int64_t n4 = N / 4, kp = K / 16;
  if (kp >= 1 && kp <= kRegMaxPieces) {
    RegArgs a{p0,  p1,   s0,   s1,      xq,      x_scale, (int)n4, (int)kp,
              y,   acc0, acc1, nullptr, nullptr, nullptr, nullptr};
    return launch_gemv_reg(plan_gemv_reg(n4, kp, dev.num_cus, gate, kXInt8), gate,
                           kXInt8, a, stream);
  }
  // K == 0 or K > 32768: activations read from LDS per piece.
  GemvArgs a;
  a.p0 = p0;
  a.p1 = p1;
  a.s0 = s0;
  a.s1 = s1;
  a.xq = xq;
  a.x_scale = x_scale;
  a.n4 = (int)n4;
  a.kp = (int)kp;
  a.y = y;
  a.acc0 = acc0;
  a.acc1 = acc1;
  const GemvPlan pl = plan_gemv_lds(n4, kp, dev.num_cus, gate ? 2 : 1);
  const size_t lds = (size_t)K;
  return gate ? launch_gemv_lds<true>(pl, a, lds, stream)
              : launch_gemv_lds<false>(pl, a, lds, stream);
}

// Per-token quantization of a raw activation row fused into the GEMV
// prologue (one launch); K == 0 or K > 32768 take two launches.
tq_status quant_gemv_m1(bool gate, const void *x, tq_dtype xt, const uint8_t *p0,
                        float s0, const uint8_t *p1, float s1, int64_t N,
                        int64_t K, float *y, int32_t *acc0, int32_t *acc1,
                        int8_t *xq, float *x_scale, const float *y_scale,
                        hipStream_t stream) {
  DeviceInfo dev;
  if (tq_status s = current_device(&dev)) return s;
  const int64_t n4 = N / 4, kp = K / 16;
  if (N > 0 && kp >= 1 && kp <= kRegMaxPieces) {
    RegArgs a{p0, p1,   s0,   s1, nullptr, nullptr, (int)n4, (int)kp,
              y,  acc0, acc1, x,  xq,      x_scale, y_scale};
    const int form = xt == TQ_BF16 ? kXBf16 : kXF32;
    return launch_gemv_reg(plan_gemv_reg(n4, kp, dev.num_cus, gate, form), gate, form,
                           a, stream);
  }
  if (tq_status s = tq_act_quant(x, xt, 1, K, xq, x_scale, stream)) return s;
  if (N == 0) return TQ_OK;
  return gemv_m1(gate, p0, s0, p1, s1, xq, y_scale ? y_scale : x_scale, N, K, y,
                 acc0, acc1, stream);
}

// The same with the sub-layer RMSNorm folded into the quantization.
tq_status rmsnorm_quant_gemv_m1(const void *x, tq_dtype xt, const void *gamma,
                                float eps, const uint8_t *p0, float s0, int64_t N,
                                int64_t K, float *y, int32_t *acc0, int8_t *xq,
                                float *x_scale, hipStream_t stream) {
  DeviceInfo dev;
  if (tq_status s = current_device(&dev)) return s;
  const int64_t n4 = N / 4, kp = K / 16;
  if (N > 0 && kp <= kRegMaxPieces) {  // kp >= 1: K > 0 is required
    RegArgs a{p0, nullptr, s0,   0.0f, nullptr, nullptr, (int)n4, (int)kp,
              y,  acc0,    nullptr, x, xq,      x_scale, nullptr};
    a.gamma = gamma;
    a.eps = eps;
    const int form = xt == TQ_BF16 ? kXBf16Rms : kXF32Rms;
    return launch_gemv_reg(plan_gemv_reg(n4, kp, dev.num_cus, false, form), false, form,
                           a, stream);
  }
  if (tq_status s = rmsnorm_act_quant(x, xt, gamma, eps, 1, K, xq, x_scale, stream))
    return s;
  if (N == 0) return TQ_OK;
  return gemv_m1(false, p0, s0, nullptr, 0.0f, xq, x_scale, N, K, y, acc0, nullptr,
                 stream);
}

tq_status check_quant_args(const void *x, tq_dtype xt, const uint8_t *p,
                           int64_t N, int64_t K, const float *y,
                           const int32_t *acc0, const int32_t *acc1,
                           const int8_t *xq, const float *x_scale,
                           const float *y_scale) {
  if (xt != TQ_BF16 && xt != TQ_F32) return TQ_ERR_DTYPE;
  if (tq_status s = check_nk(N, K)) return s;
  if (!x_scale || (K > 0 && (!x || !xq)) || (N > 0 && !y) ||
      (N > 0 && K > 0 && !p))
    return TQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(p, 16) || !aligned(xq, 16) ||
      !aligned(y, 4) || !aligned(acc0, 4) || !aligned(acc1, 4) ||
      !aligned(x_scale, 4) || !aligned(y_scale, 4))
    return TQ_ERR_ALIGN;
  return TQ_OK;
}

// Grouped form: `count` matrices sharing one raw activation row, one launch
// over their concatenated packed rows (the fallback for K == 0 or
// K > 32768 quantizes once and runs one GEMV per matrix).
tq_status quant_gemv_group(const void *x, tq_dtype xt, int count,
                           const uint8_t *const *packed, const float *w_scale,
                           const int64_t *N, int64_t K, float *const *y,
                           int32_t *const *acc, int8_t *xq, float *x_scale,
                           const float *y_scale, hipStream_t stream) {
  DeviceInfo dev;
  if (tq_status s = current_device(&dev)) return s;
  const int64_t kp = K / 16;
  RegArgs a{};
  int64_t total = 0;
  for (int i = 0; i < count; ++i) {
    if (N[i] == 0) continue;  // empty matrices take no rows
    const int q = a.seg.n++;
    total += N[i] / 4;
    a.seg.end[q] = (int)total;
    a.seg.p[q] = packed[i];
    a.seg.s[q] = w_scale[i];
    a.seg.y[q] = y[i];
    a.seg.acc[q] = acc ? acc[i] : nullptr;
  }
  if (total > 0 && kp >= 1 && kp <= kRegMaxPieces) {
    a.n4 = (int)total;
    a.kp = (int)kp;
    a.x = x;
    a.xq_out = xq;
    a.xs_out = x_scale;
    a.y_scale = y_scale;
    a.p0 = a.seg.p[0];  // unused by the grouped form; kept valid
    a.y = a.seg.y[0];
    const int form = xt == TQ_BF16 ? kXBf16 : kXF32;
    return launch_gemv_reg(plan_gemv_reg(total, kp, dev.num_cus, false, form), false,
                           form, a, stream);
  }
  if (tq_status s = tq_act_quant(x, xt, 1, K, xq, x_scale, stream)) return s;
  for (int i = 0; i < count; ++i) {
    if (N[i] == 0) continue;
    if (tq_status s = gemv_m1(false, packed[i], w_scale[i], nullptr, 0.0f, xq,
                              y_scale ? y_scale : x_scale, N[i], K, y[i],
                              acc ? acc[i] : nullptr, nullptr, stream))
      return s;
  }
  return TQ_OK;
}

}  // namespace tq

extern "C" tq_status tq_quant_gemv_group(const void *x, tq_dtype xt,
                                         int32_t count,
                                         const uint8_t *const *packed,
                                         const float *w_scale, const int64_t *N,
                                         int64_t K, float *const *y,
                                         int32_t *const *acc, int8_t *xq,
                                         float *x_scale, const float *y_scale,
                                         hipStream_t stream) {
  using namespace tq;
  if (xt != TQ_BF16 && xt != TQ_F32) return TQ_ERR_DTYPE;
  if (count < 1 || count > kMaxSeg) return TQ_ERR_SHAPE;
  if (!packed || !w_scale || !N || !y) return TQ_ERR_NULL;
  int64_t total = 0;
  for (int i = 0; i < count; ++i) {
    if (tq_status s = check_quant_args(x, xt, packed[i], N[i], K, y[i],
                                       acc ? acc[i] : nullptr, nullptr, xq,
                                       x_scale, y_scale))
      return s;
    total += N[i];
  }
  if (total / 4 > (int64_t)INT32_MAX) return TQ_ERR_SHAPE;
  return quant_gemv_group(x, xt, count, packed, w_scale, N, K, y, acc, xq,
                          x_scale, y_scale, stream);
}

extern "C" tq_status tq_quant_gemv(const void *x, tq_dtype xt,
                                   const uint8_t *packed, float w_scale,
                                   int64_t N, int64_t K, float *y,
                                   int32_t *acc, int8_t *xq, float *x_scale,
                                   const float *y_scale, hipStream_t stream) {
  using namespace tq;
  if (tq_status s = check_quant_args(x, xt, packed, N, K, y, acc, nullptr, xq,
                                     x_scale, y_scale))
    return s;
  return quant_gemv_m1(false, x, xt, packed, w_scale, nullptr, 0.0f, N, K, y, acc,
                       nullptr, xq, x_scale, y_scale, stream);
}

extern "C" tq_status tq_rmsnorm_quant_gemv(const void *x, tq_dtype xt,
                                           const void *gamma, float eps,
                                           const uint8_t *packed, float w_scale,
                                           int64_t N, int64_t K, float *y,
                                           int32_t *acc, int8_t *xq,
                                           float *x_scale, hipStream_t stream) {
  using namespace tq;
  if (tq_status s = check_quant_args(x, xt, packed, N, K, y, acc, nullptr, xq,
                                     x_scale, nullptr))
    return s;
  if (tq_status s = check_rms(gamma, eps, K)) return s;
  return rmsnorm_quant_gemv_m1(x, xt, gamma, eps, packed, w_scale, N, K, y, acc,
                               xq, x_scale, stream);
}

extern "C" tq_status tq_quant_gate_up_relu2(
    const void *x, tq_dtype xt, const uint8_t *packed_gate, float s_gate,
    const uint8_t *packed_up, float s_up, int64_t N, int64_t K, float *h,
    int32_t *acc_gate, int32_t *acc_up, int8_t *xq, float *x_scale,
    const float *y_scale, hipStream_t stream) {
  using namespace tq;
  if (tq_status s = check_quant_args(x, xt, packed_gate, N, K, h, acc_gate,
                                     acc_up, xq, x_scale, y_scale))
    return s;
  if (N > 0 && K > 0 && !packed_up) return TQ_ERR_NULL;
  if (!aligned(packed_up, 16)) return TQ_ERR_ALIGN;
  return quant_gemv_m1(true, x, xt, packed_gate, s_gate, packed_up, s_up, N, K, h, acc_gate,
                       acc_up, xq, x_scale, y_scale, stream);
}

extern "C" tq_status tq_gemv(const uint8_t *packed, float w_scale,
                             const int8_t *xq, const float *x_scale, int64_t N,
                             int64_t K, float *y, int32_t *acc,
                             hipStream_t stream) {
  using namespace tq;
  if (tq_status s = check_nk(N, K)) return s;
  if (N == 0) return TQ_OK;
  if (!y || !x_scale || (K > 0 && (!packed || !xq))) return TQ_ERR_NULL;
  if (!aligned(packed, 16) || !aligned(xq, 16) || !aligned(y, 4) ||
      !aligned(acc, 4) || !aligned(x_scale, 4))
    return TQ_ERR_ALIGN;
  return gemv_m1(false, packed, w_scale, nullptr, 0.0f, xq, x_scale, N, K, y, acc,
                 nullptr, stream);
}
