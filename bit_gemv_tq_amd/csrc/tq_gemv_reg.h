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
// once per block through LDS (a 256-lane team, alone in its block, loads
// exactly its own pieces and skips LDS) and then held in VGPRs.  Blocks
// have 256 threads (512, two teams, for the fp32 and RMSNorm forms of
// 256-lane teams).  The hot loop is NP
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

#include <atomic>
#include <type_traits>

#include "tq_device.h"
#include "tq_host.h"

namespace tq {

constexpr int kRegThreads = 256;

// Block size of the five-per-byte GEMV and the M = 2 vector kernel, which
// share the team structure: 256-lane teams run two to a 512-thread block.
constexpr int reg_block_threads(int lpr) { return lpr >= 256 ? 512 : kRegThreads; }
constexpr int kRegMaxPieces = 2048;  // K <= 32768 bytes

// Activation forms: kXInt8 = int8 row + scale given (tq_gemv); kXBf16 /
// kXF32 = raw row, quantized in the prologue (tq_quant_gemv); kXBf16Rms /
// kXF32Rms = raw row with the sub-layer RMSNorm folded into that
// quantization (tq_rmsnorm_quant_gemv).
constexpr int kXInt8 = 0, kXBf16 = 1, kXF32 = 2, kXBf16Rms = 3, kXF32Rms = 4;
constexpr bool xt_rms(int xt) { return xt == kXBf16Rms || xt == kXF32Rms; }
constexpr bool xt_bf16(int xt) { return xt == kXBf16 || xt == kXBf16Rms; }

// Block size of the GEMV: 256 threads, one 256-lane team or several
// narrower ones.  The fp32 and RMSNorm prologues of a 256-lane team hold
// too many registers for one team per block (up to 400 VGPRs), so those run
// two teams per 512-thread block, sharing the staged row.
constexpr int gemv_block_threads(int lpr, int xt) {
  return lpr >= 256 && (xt == kXF32 || xt_rms(xt)) ? 512 : kRegThreads;
}

// Grouped form: several weight matrices with the same K that read one
// activation row (e.g. the q, k and v projections), run as one packed-row
// range.  Segment q holds global packed rows [end[q-1], end[q]).
constexpr int kMaxSeg = 4;
struct RegSegs {
  int n;                         // 0: single matrix (p0, s0, y, acc0)
  int end[kMaxSeg];              // cumulative packed-row counts
  const uint8_t *p[kMaxSeg];     // packed [N_q/4, K]
  float s[kMaxSeg];              // weight scales
  float *y[kMaxSeg];             // [N_q] outputs
  int32_t *acc[kMaxSeg];         // optional [N_q]
};

struct RegArgs {
  const uint8_t *p0;     // packed [N/4,K] (gate when kGate)
  const uint8_t *p1;     // packed up (kGate only)
  float s0, s1;          // weight scales
  const int8_t *xq;      // [K] int8 activations (kXInt8)
  const float *x_scale;  // [1] their scale (kXInt8)
  int n4;                // N/4
  int kp;                // K/16
  float *y;              // [N] (h when kGate)
  int32_t *acc0;         // optional [N]
  int32_t *acc1;         // optional [N] (kGate only)
  const void *x;         // [K] raw bf16/fp32 row (kXBf16, kXF32)
  int8_t *xq_out;        // [K] quantized row, written by block 0 (raw forms)
  float *xs_out;         // [1] its scale s_x, written by block 0 (raw forms)
  const float *y_scale;  // optional [1]: activation scale used in the
                         // rescale instead of s_x (raw forms)
  RegSegs seg;           // grouped form (not with kGate); n4 = total rows
  const void *gamma;     // [K] RMSNorm weights, dtype of x (kX*Rms)
  float eps;             // RMSNorm epsilon (kX*Rms)
  // Rows by dispatch round (one-team blocks; 0 = off): block b is in round
  // b / round_cus and walks the rows [0, end0), [end0, end1) or [end1, n4)
  // of its round, strided by round_cus.  Set by the launcher from the plan.
  int round_cus, round_end0, round_end1;
};

// Segment of global packed row i (grouped form): its first row and index.
__device__ __forceinline__ int seg_of(const RegSegs &sg, int i, int &start) {
  int q = 0;
  start = 0;
#pragma unroll
  for (int t = 1; t < kMaxSeg; ++t)
    if (t < sg.n && i >= sg.end[t - 1]) {
      q = t;
      start = sg.end[t - 1];
    }
  return q;
}

// Unrolled selects (q may differ between lanes) of candidates pinned in
// scalar registers by an empty asm statement: left alone, the compiler turns
// the selects into a vector load of the argument block indexed by q, and the
// wait for that load (vmcnt 0) costs every output row a memory round trip
// (70B-class q/k/v in one launch: 8.4 against 6.9 us for one concatenated
// matrix of the same bytes).
template <typename T>
__device__ __forceinline__ T seg_pick(const T (&v)[kMaxSeg], int q) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "scalar-register candidates");
  using B = typename std::conditional<sizeof(T) == 4, uint32_t, uint64_t>::type;
  B r = __builtin_bit_cast(B, v[0]);
  asm volatile("" : "+s"(r));
#pragma unroll
  for (int t = 1; t < kMaxSeg; ++t) {
    B c = __builtin_bit_cast(B, v[t]);
    asm volatile("" : "+s"(c));
    r = q == t ? c : r;
  }
  return __builtin_bit_cast(T, r);
}

// Global-memory views of output pointers (see the grouped emit).
typedef __attribute__((address_space(1))) float gfloat;
typedef __attribute__((address_space(1))) int32_t gint32;

// Segment q's packed matrix, for the weight loads.  The candidates pass
// through an empty asm statement that pins them in scalar registers: left
// alone, the compiler folds the selects into an indexed vector load of the
// argument block, whose wait (vmcnt 0) would also wait for every activation
// load issued before it, so no weight load could start before the whole
// activation row had arrived.  The result is marked as a global-memory
// address again, so the weight loads stay global (not flat) loads.
typedef __attribute__((address_space(1))) const uint8_t gbyte;
__device__ __forceinline__ const uint8_t *seg_matrix(const RegSegs &sg, int q) {
  uint64_t r = reinterpret_cast<uint64_t>(sg.p[0]);
#pragma unroll
  for (int t = 1; t < kMaxSeg; ++t) {
    uint64_t v = reinterpret_cast<uint64_t>(sg.p[t]);
    asm volatile("" : "+s"(v));
    r = q == t ? v : r;
  }
  return (const uint8_t *)reinterpret_cast<gbyte *>(r);
}

template <int LPR, int NP, bool EXACT, bool kGate, int XT, int BT = kRegThreads>
__global__ __launch_bounds__(BT) void gemv_reg_kernel(RegArgs g) {
  constexpr int NM = kGate ? 2 : 1;
  constexpr int G = BT / LPR;                         // teams per block
  constexpr int GL = LPR < kWave ? LPR : kWave;       // DPP reduction width
  constexpr int WPT = LPR > kWave ? LPR / kWave : 1;  // waves per team
  constexpr int SPAN = NP * LPR;                      // pieces a team covers
  constexpr int SP = (SPAN + BT - 1) / BT;  // staging loads
  // One team per block (256-lane teams): thread i stages pieces i + s*BT,
  // which are exactly its own pieces lane + t*LPR (SP == NP), so the row
  // needs no LDS round trip and no barrier between staging and use.
  constexpr bool kOwn = G == 1;
  static_assert(NP >= 1 && SPAN <= kRegMaxPieces, "pieces per lane");
  constexpr int VPP = XT == kXInt8 ? 1 : (xt_bf16(XT) ? 2 : 4);  // words/piece
  constexpr bool kRms = xt_rms(XT);
  constexpr int GPP = kRms ? VPP : 1;  // gamma words per piece (unused: 1)
  __shared__ u32x4 x_lds[kOwn ? 1 : SP * BT];  // padded: stores unconditional
  // Team sums across waves.  Several 256-lane teams in one block (the fp32
  // and RMSNorm forms) reduce without a block barrier: each wave adds its
  // partial sums to the slot of the row iteration and counts itself in, and
  // the team's last wave emits the row, so one team never waits for another
  // (measured on MI355X at [8192,28672]: the RMSNorm form 13.9 against
  // 15.2 us, the fp32 row 14.5 against 15.0 us, bit-identical).  A one-team
  // block, and two-wave teams, keep the barrier (the counter's atomic
  // measured 0.1-0.4 us slower there).
  constexpr bool kFreeTeams = G > 1 && WPT >= 4;
  constexpr int kSlots = kFreeTeams ? 8 : 2;
  __shared__ int red[kSlots][BT / kWave][NM][4];
  __shared__ int cnt[kFreeTeams ? kSlots * G : 1];
  __shared__ float amax_lds[BT / kWave];
  __shared__ double ss_lds[kRms ? BT / kWave : 1];

  // Zeroed before the staging barrier below, which every wave passes before
  // its first count.
  if constexpr (kFreeTeams) {
    if ((int)threadIdx.x < kSlots * G) cnt[threadIdx.x] = 0;
  }
  const int kp = g.kp, n4 = g.n4;
  const int lane = threadIdx.x % LPR;
  const int team = threadIdx.x / LPR;
  const int wave = threadIdx.x / kWave;
  int row_stride = gridDim.x * G;
  int rb0 = blockIdx.x * G;  // < n4 for every launched block
  int its;
  if (kOwn && g.round_cus > 0) {
    const int rnd = blockIdx.x / g.round_cus;
    const int start = rnd == 0 ? 0 : (rnd == 1 ? g.round_end0 : g.round_end1);
    const int end = rnd == 0 ? g.round_end0 : (rnd == 1 ? g.round_end1 : n4);
    row_stride = g.round_cus;
    rb0 = start + (int)blockIdx.x % g.round_cus;
    if (rb0 >= end) return;  // the whole block, before any barrier
    its = (end - 1 - rb0) / row_stride + 1;
  } else {
    its = (n4 - 1 - rb0) / row_stride + 1;
  }

  // A row index that is the same in every lane of a wave (teams of 64 or
  // more lanes), made visibly uniform so that the grouped form's segment
  // lookups are scalar operations.
  auto wave_row = [&](int r) {
    if constexpr (LPR >= kWave) return __builtin_amdgcn_readfirstlane(r);
    else return r;
  };

  const uint4 *P[NM];
  P[0] = reinterpret_cast<const uint4 *>(g.p0);
  if constexpr (kGate) P[NM - 1] = reinterpret_cast<const uint4 *>(g.p1);

  // Piece index of slot t for this lane; past the row end it re-reads the
  // last piece (in bounds) and its activation slot is zero.
  auto piece = [&](int t) {
    const int p = lane + t * LPR;
    return EXACT ? p : min(p, kp - 1);
  };

  // 1. Activation loads first (static count).  Thread i stages pieces
  // i + s*BT.  (Native clang vectors: the compiler keeps these in VGPRs.)
  const u32x4 *xg = reinterpret_cast<const u32x4 *>(
      XT == kXInt8 ? static_cast<const void *>(g.xq) : g.x);
  u32x4 xs[SP][VPP];
  u32x4 gs[SP][GPP];  // RMSNorm weights of the same pieces (kRms)
#pragma unroll
  for (int s = 0; s < SP; ++s) {
    const int p = (int)threadIdx.x + s * BT;
    const int pc = EXACT ? min(p, SPAN - 1) : min(p, kp - 1);
#pragma unroll
    for (int v = 0; v < VPP; ++v) xs[s][v] = xg[pc * VPP + v];
    if constexpr (kRms) {
#pragma unroll
      for (int v = 0; v < VPP; ++v)
        gs[s][v] = reinterpret_cast<const u32x4 *>(g.gamma)[pc * VPP + v];
    }
  }
  // Keep the scheduler from sinking these loads below the weight loads.
  __builtin_amdgcn_sched_barrier(0);

  // 2. Weight loads of the first row.
  auto issue = [&](uint4 (&w)[NM][NP], int rbase) {
    const int row = min(rbase + team, n4 - 1);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const uint4 *rp = P[m] + (size_t)row * kp;
      if (!kGate && g.seg.n > 0) {  // grouped: the row's own matrix
        int start;
        const int q = seg_of(g.seg, wave_row(row), start);
        rp = reinterpret_cast<const uint4 *>(seg_matrix(g.seg, q)) +
             (size_t)(row - start) * kp;
      }
#pragma unroll
      for (int t = 0; t < NP; ++t) w[m][t] = load_stream16(rp + piece(t));
    }
  };
  uint4 wa[NM][NP];
  issue(wa, rb0);
  __builtin_amdgcn_sched_barrier(0);

  // 3. Stage x through LDS (quantizing a raw row first); keep this lane's
  // pieces in VGPRs.  With one team per block the staged pieces stay in
  // the thread's registers (own[]).
  float sx;
  u32x4 own[kOwn ? SP : 1];
  if constexpr (XT == kXInt8) {
#pragma unroll
    for (int s = 0; s < SP; ++s) {
      if constexpr (kOwn) own[s] = xs[s][0];
      else x_lds[threadIdx.x + s * BT] = xs[s][0];
    }
    sx = g.x_scale[0];
  } else {
    // Per-token absmax over the whole row (every block, redundantly), then
    // q = rne(x * (127/a')) exactly as tq_act_quant.  With the RMSNorm
    // folded in, the same on u = x * gamma, and s_x = (a'/127) * r with
    // r = 1/sqrt(mean(x^2) + eps): every block sums the squares in the same
    // order, so all get the same r.
    constexpr bool kBf16 = xt_bf16(XT);
    auto raw = [&](int s) {
      RawPiece<kBf16> r;
#pragma unroll
      for (int v = 0; v < VPP; ++v) r.w[v] = xs[s][v];
      return r;
    };
    // Values that are quantized: the raw row, or u = x * gamma (fp32).
    using QPiece = RawPiece<kRms ? false : kBf16>;
    QPiece qv[SP];
    double ss = 0.0;
#pragma unroll
    for (int s = 0; s < SP; ++s) {
      if constexpr (kRms) {
        RawPiece<kBf16> gr;
#pragma unroll
        for (int v = 0; v < VPP; ++v) gr.w[v] = gs[s][v];
        double sq = 0.0;
        qv[s] = scale_piece<kBf16>(raw(s), gr, sq);
        // slots past the row end re-read an in-row piece: not summed again
        if ((int)threadIdx.x + s * BT < kp) ss += sq;
      } else {
        qv[s] = raw(s);
      }
    }
    constexpr bool kQBf16 = kRms ? false : kBf16;
    // Slots past the row end hold a re-read of an in-row piece (clamped
    // index), so they cannot change the maximum.
    uint32_t mb = 0;
#pragma unroll
    for (int s = 0; s < SP; ++s) mb = absmax_bits<kQBf16>(qv[s], mb);
    float a = wave_max(absmax_value<kQBf16>(mb));
    if ((threadIdx.x & (kWave - 1)) == 0) amax_lds[wave] = a;
    if constexpr (kRms) {
      ss = wave_sum_f64(ss);
      if ((threadIdx.x & (kWave - 1)) == 0) ss_lds[wave] = ss;
    }
    __syncthreads();
    a = amax_lds[0];
#pragma unroll
    for (int w = 1; w < BT / kWave; ++w) a = fmaxf(a, amax_lds[w]);
    const float ap = a > 1e-5f ? a : 1e-5f;
    const float inv = 127.0f / ap;  // correctly rounded fp32 division
    float s_x = ap / 127.0f;
    if constexpr (kRms) {
      double t = ss_lds[0];
#pragma unroll
      for (int w = 1; w < BT / kWave; ++w) t += ss_lds[w];
      s_x = s_x * rms_factor(t, (int64_t)kp * 16, g.eps);
    }
    const bool writer = blockIdx.x == 0;
#pragma unroll
    for (int s = 0; s < SP; ++s) {
      const int p = (int)threadIdx.x + s * BT;
      const u32x4 q = quant_piece<kQBf16>(qv[s], inv);
      if constexpr (kOwn) own[s] = q;
      else x_lds[threadIdx.x + s * BT] = q;
      if (writer && p < kp)
        reinterpret_cast<u32x4 *>(g.xq_out)[p] = q;
    }
    if (writer && threadIdx.x == 0) g.xs_out[0] = s_x;
    sx = g.y_scale ? g.y_scale[0] : s_x;
  }
  if constexpr (!kOwn) __syncthreads();
  uint4 xr[NP];
  int sq = 0;
#pragma unroll
  for (int t = 0; t < NP; ++t) {
    const int p = lane + t * LPR;
    u32x4 v;
    if constexpr (kOwn) v = own[t];
    else v = x_lds[p];
    xr[t] = (EXACT || p < kp) ? make_uint4(v[0], v[1], v[2], v[3])
                              : make_uint4(0, 0, 0, 0);
    sq = sum_bytes16(xr[t], sq);
  }
  // Per-plane accumulator start: -scale_j * (this lane's share of sum(q)).
  const int init[4] = {-sq, -4 * sq, -16 * sq, -16 * sq};

  const float c0 = g.s0 * sx;
  const float c1 = g.s1 * sx;

  auto consume = [&](uint4 (&w)[NM][NP], int rbase, int it) {
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
    // The row's outputs: y, acc, scale and row count of its matrix.  In the
    // grouped form one segment lookup per row serves all four outputs (a
    // lookup per output, with its selects pinned apart by the asm statements,
    // made the emit dozens of dependent instructions per output: 2.4 us per
    // launch).  Stores go through global-memory pointers (a selected pointer
    // is generic to the compiler, and would give flat stores).
    gfloat *yo = (gfloat *)g.y;
    gint32 *ao = (gint32 *)g.acc0;
    float co = c0;
    int n4o = n4, io = i;
    if (!kGate && g.seg.n > 0) {
      int start;
      const int q = seg_of(g.seg, wave_row(i), start);
      n4o = seg_pick(g.seg.end, q) - start;
      io = i - start;
      yo = (gfloat *)seg_pick(g.seg.y, q);
      ao = (gint32 *)seg_pick(g.seg.acc, q);
      co = seg_pick(g.seg.s, q) * sx;
    }
    auto emit = [&](int j, int v0, int v1) {
      if (i >= n4) return;
      const int sh = j == 0 ? 0 : (j == 1 ? 2 : 4);
      const int t0 = v0 >> sh;  // exact: the sum is a multiple of 1 << sh
      if constexpr (kGate) {
        const size_t n = (size_t)j * n4 + i;
        const int t1 = v1 >> sh;
        if (g.acc0) g.acc0[n] = t0;
        if (g.acc1) g.acc1[n] = t1;
        g.y[n] = relu2_gate(rescale(t0, c0), rescale(t1, c1));
      } else {
        const size_t n = (size_t)j * n4o + io;
        if (ao) ao[n] = t0;
        yo[n] = rescale(t0, co);
      }
    };
    if constexpr (WPT == 1) {
      if (lane == LPR - 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) emit(j, a[0][j], a[NM - 1][j]);
      }
    } else if constexpr (!kFreeTeams) {
      const int slot = it & 1;  // the next row's partials go to the other slot
      if ((threadIdx.x & (kWave - 1)) == kWave - 1) {
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int j = 0; j < 4; ++j) red[slot][wave][m][j] = a[m][j];
      }
      __syncthreads();
      if (lane < 4) {
        int v[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          v[m] = 0;
#pragma unroll
          for (int w2 = 0; w2 < WPT; ++w2) v[m] += red[slot][team * WPT + w2][m][lane];
        }
        emit(lane, v[0], v[NM - 1]);
      }
    } else {
      // The partial sums are stored before the count (release); the wave
      // that sees the team's count complete reads the others' sums after it
      // (acquire).  Counts only grow: the WPT waves of a team add one each
      // per row, so the last is the one that finds count % WPT == WPT - 1.
      const int slot = it % kSlots;
      const int wl = threadIdx.x & (kWave - 1);
      int seen = 0;
      if (wl == kWave - 1) {
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int j = 0; j < 4; ++j) red[slot][wave][m][j] = a[m][j];
        seen = __hip_atomic_fetch_add(&cnt[slot * G + team], 1, __ATOMIC_ACQ_REL,
                                      __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      seen = __builtin_amdgcn_readlane(seen, kWave - 1);
      if (seen % WPT == WPT - 1 && wl < 4) {
        int v[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          v[m] = 0;
#pragma unroll
          for (int w2 = 0; w2 < WPT; ++w2) v[m] += red[slot][team * WPT + w2][m][wl];
        }
        emit(wl, v[0], v[NM - 1]);
      }
      // A barrier every kSlots rows keeps any wave from reusing a slot
      // before its team's last wave of that row has read it (`its` is
      // block-uniform, so every wave reaches it).
      if (slot == kSlots - 1) __syncthreads();
    }
  };

  // 4. Row iterations: `its` is block-uniform, so every wave reaches the
  // same barriers.  (Other resident blocks hide this wave's load latency;
  // measured on MI355X, that beat a software prefetch of the next row,
  // which costs registers and so occupancy.)
  consume(wa, rb0, 0);
  for (int it = 1; it < its; ++it) {
    issue(wa, rb0 + it * row_stride);
    // Left alone, the scheduler starts decoding the row's first piece
    // between its loads, and that wait holds the last loads back for a
    // memory round trip.  Keeping every load ahead of the decode pays only
    // for one-team blocks that quantize a raw row (measured on MI355X, same
    // box, back to back: [8192,28672] bf16 12.37 against 12.67 us); for the
    // int8 row and for narrower teams the interleaved order measured 0.1 to
    // 0.2 us faster, so it is kept there.
    if constexpr (kOwn && XT != kXInt8) __builtin_amdgcn_sched_barrier(0);
    consume(wa, rb0 + it * row_stride, it);
  }
}

// Launch one instantiation family (defined per LPR in tq_gemv_reg_l*.hip).
struct RegPlan {
  int lpr, np, blocks;
  bool exact;
  int round_cus, round_end0, round_end1;  // rows by dispatch round (0: off)
  bool persistent;  // blocks = resident blocks per CU x CUs, rows walked
  int cus;
};

// Launch of a persistent grid, capped at the blocks of this kernel that one
// CU can hold (asked of the runtime once per kernel and cached in `occ`):
// the planner's blocks per CU assume a register count that a few forms
// exceed (the RMSNorm prologue with 128-lane teams at 7-8 pieces per lane,
// the fp32 row with two 256-lane teams at 8 pieces), and the blocks beyond
// the resident ones would run as a second wave (measured on MI355X: the
// RMSNorm form at [16384,14336] 13.7 against 15.7 us, the fp32 row at
// [8192,30720] 14.4 against 17.2 us).  A capped grid walks its rows evenly
// (no split by round).
template <typename K>
tq_status launch_resident(K kernel, std::atomic<int> &occ, const RegPlan &pl, dim3 block,
                          hipStream_t s, const RegArgs &args) {
  int blocks = pl.blocks;
  RegArgs a = args;
  if (pl.persistent) {
    const int n = resident_blocks(kernel, (int)block.x, occ);  // -1: keep the plan
    if (n > 0 && (int64_t)blocks > (int64_t)n * pl.cus) {
      blocks = n * pl.cus;
      a.round_cus = 0;
    }
  }
  return launch(kernel, dim3(blocks), block, 0, s, a);
}

template <int LPR>
tq_status launch_reg(const RegPlan &pl, bool gate, int xt, const RegArgs &a,
                     hipStream_t s);

#define TQ_REG_KERNEL(LPR, NPV, GATE, XT)                                      \
  (pl.exact ? gemv_reg_kernel<LPR, NPV, true, GATE, XT, gemv_block_threads(LPR, XT)>  \
            : gemv_reg_kernel<LPR, NPV, false, GATE, XT, gemv_block_threads(LPR, XT)>)

// One case: the instance's launch, with its resident-block count cached per
// exact/ragged form.
#define TQ_REG_NP_CASE(LPR, NPV, GATE, XT)                                      \
  case NPV: {                                                                  \
    static std::atomic<int> occ[2];                                            \
    return launch_resident(TQ_REG_KERNEL(LPR, NPV, GATE, XT), occ[pl.exact ? 1 : 0], \
                           pl, block, s, a);                                   \
  }

#define TQ_REG_NP_CASES(LPR, GATE, XT)                                         \
  const dim3 block(gemv_block_threads(LPR, XT));                               \
  switch (pl.np) {                                                             \
    TQ_REG_NP_CASE(LPR, 1, GATE, XT)                                           \
    TQ_REG_NP_CASE(LPR, 2, GATE, XT)                                           \
    TQ_REG_NP_CASE(LPR, 3, GATE, XT)                                           \
    TQ_REG_NP_CASE(LPR, 4, GATE, XT)                                           \
    TQ_REG_NP_CASE(LPR, 5, GATE, XT)                                           \
    TQ_REG_NP_CASE(LPR, 6, GATE, XT)                                           \
    TQ_REG_NP_CASE(LPR, 7, GATE, XT)                                           \
    TQ_REG_NP_CASE(LPR, 8, GATE, XT)                                           \
  }                                                                            \
  return TQ_ERR_LAUNCH;

#define TQ_REG_XT_CASES(LPR, GATE)                                             \
  switch (xt) {                                                                \
    case kXInt8: { TQ_REG_NP_CASES(LPR, GATE, kXInt8) }                        \
    case kXBf16: { TQ_REG_NP_CASES(LPR, GATE, kXBf16) }                        \
    case kXF32: { TQ_REG_NP_CASES(LPR, GATE, kXF32) }                          \
  }                                                                            \
  return TQ_ERR_DTYPE;

// The RMSNorm forms exist for the plain GEMV only.
#define TQ_REG_XT_CASES_RMS(LPR)                                               \
  switch (xt) {                                                                \
    case kXInt8: { TQ_REG_NP_CASES(LPR, false, kXInt8) }                       \
    case kXBf16: { TQ_REG_NP_CASES(LPR, false, kXBf16) }                       \
    case kXF32: { TQ_REG_NP_CASES(LPR, false, kXF32) }                         \
    case kXBf16Rms: { TQ_REG_NP_CASES(LPR, false, kXBf16Rms) }                 \
    case kXF32Rms: { TQ_REG_NP_CASES(LPR, false, kXF32Rms) }                   \
  }                                                                            \
  return TQ_ERR_DTYPE;

#define TQ_DEFINE_LAUNCH_REG(LPR, GATE)                                        \
  template <>                                                                  \
  tq_status launch_reg_part<LPR, GATE>(const RegPlan &pl, int xt,              \
                                       const RegArgs &a, hipStream_t s) {      \
    TQ_REG_XT_CASES(LPR, GATE)                                                 \
  }

#define TQ_DEFINE_LAUNCH_REG_GEMV(LPR)                                         \
  template <>                                                                  \
  tq_status launch_reg_part<LPR, false>(const RegPlan &pl, int xt,             \
                                        const RegArgs &a, hipStream_t s) {     \
    TQ_REG_XT_CASES_RMS(LPR)                                                   \
  }

template <int LPR, bool GATE>
tq_status launch_reg_part(const RegPlan &pl, int xt, const RegArgs &a,
                          hipStream_t s);

// Explicit specializations, each defined in its own tq_gemv_reg_l*.hip.
#define TQ_DECLARE_LAUNCH_REG(LPR, GATE)                                       \
  template <>                                                                  \
  tq_status launch_reg_part<LPR, GATE>(const RegPlan &pl, int xt,              \
                                       const RegArgs &a, hipStream_t s);
TQ_DECLARE_LAUNCH_REG(16, false)
TQ_DECLARE_LAUNCH_REG(16, true)
TQ_DECLARE_LAUNCH_REG(32, false)
TQ_DECLARE_LAUNCH_REG(32, true)
TQ_DECLARE_LAUNCH_REG(64, false)
TQ_DECLARE_LAUNCH_REG(64, true)
TQ_DECLARE_LAUNCH_REG(128, false)
TQ_DECLARE_LAUNCH_REG(128, true)
TQ_DECLARE_LAUNCH_REG(256, false)
TQ_DECLARE_LAUNCH_REG(256, true)
#undef TQ_DECLARE_LAUNCH_REG

template <int LPR>
tq_status launch_reg(const RegPlan &pl, bool gate, int xt, const RegArgs &a,
                     hipStream_t s) {
  return gate ? launch_reg_part<LPR, true>(pl, xt, a, s)
              : launch_reg_part<LPR, false>(pl, xt, a, s);
}

}  // namespace tq
