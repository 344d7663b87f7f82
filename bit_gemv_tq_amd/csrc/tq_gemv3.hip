// tq_gemv3.hip -- tq_pack3 and tq_gemv3: the M = 1 ternary GEMV on the denser
// five-weights-per-byte layout (1.6 bits per weight).
//
// Page "Feature request: BitNet 1.58-bit ternary inference on ROCm
// (gfx1151)", section "Context", names the "TQ1_0" family of ternary formats
// only; the layout is this library's reading.  The packed array is
// [N5, K], N5 = ceil(N/5); byte [i,k] holds rows j*N5 + i (j = 0..4) of
// column k as the base-3 number v = sum_j c_j 3^j of their codes c = w + 1
// (rows past N are zero weights), stored as q = ceil(256 v / 243).
//
// Decode.  Read as the fraction q/256 ~ v/243, the digits come out most
// significant first: with r_j = q*3^j mod 256, digit 4-j is t_j =
// floor(3 r_j / 256), and r_{j+1} = 3 r_j - 256 t_j.  So per row
//   S_{4-j} = sum_k t_j(k) x_k = (3 G_j - G_{j+1}) / 256,  G_j = sum_k r_j(k) x_k,
// six dot products that are linear in the bytes r_j and need no digit
// extraction per weight.  The bytes r_j are formed four at a time: with
// e = d ^ 0x80808080 (each byte q ^ 128), the even and odd bytes of e go to
// the four 16-bit fields of one 64-bit register, and one 64-bit shift-add
// (p << 1) + p per level triples all four fields at once.  No field
// overflows (255 * 3^5 < 2^16), and a field's low byte is q*3^j + 128 mod
// 256, because (q ^ 128) differs from q + 128 by a multiple of 256 and
// 128 * 3^j = 128 mod 256; one byte permute gathers the four low bytes.  The
// +128 turns r_j into the signed byte r_j - 128 that v_dot4_i32_i8 takes
// (e itself is that byte for j = 0); accumulating G'_j = sum (r_j - 128) x
// instead of G_j changes 3 G_j - G_{j+1} by 3*128 X - 128 X = 256 X
// (X = sum x), which is exactly the code offset: 3 G'_j - G'_{j+1} =
// 256 * sum_k (c - 1) x_k = 256 * sum_k w x.  Per dword (20 weights): 1 xor,
// 2 splits, 5 shift-adds, 5 permutes, 6 dot4 -- 19 VALU operations, against
// 21 per 64 weights for the two-bit layout.  (The former form, two 24-bit
// multiply-adds per level on 32-bit registers, took 24.)
//
// Structure as the two-bit register kernel (tq_gemv_reg.h): a team of LPR
// lanes owns one packed row (5 output rows); lane l reads pieces l + t*LPR;
// its activation pieces are staged once per block through LDS and held in
// VGPRs; persistent blocks; DPP and LDS team reductions of the six sums.
#include "tq_device.h"
#include "tq_gemv_reg.h"
#include "tq_host.h"

namespace tq {
namespace {

struct Gemv3Args {
  const uint8_t *p;      // packed [n5, K]
  float s_w;
  const int8_t *xq;      // [K]
  const float *x_scale;  // [1]
  int N, n5, kp;
  float *y;              // [N]
  int32_t *acc;          // optional [N]
};

// 3 * p on a 64-bit register in one v_lshl_add_u64 ((p << 1) + p).  Written
// as an asm statement because the compiler turns the plain expression into a
// 32-bit multiply chain; pure VALU, no memory operand.
__device__ __forceinline__ uint64_t times3(uint64_t p) {
  uint64_t r;
  asm("v_lshl_add_u64 %0, %1, 1, %1" : "=v"(r) : "v"(p));
  return r;
}

// Adds the six level sums of one dword d of packed bytes against the int8
// activations x of the same four columns.
__device__ __forceinline__ void dot_levels(uint32_t d, int x, int (&g)[6]) {
  const uint32_t e = d ^ 0x80808080u;                         // q ^ 128
  g[0] = __builtin_amdgcn_sdot4((int)e, x, g[0], false);
  const uint32_t a = e & 0x00ff00ffu;                         // bytes 0, 2
  const uint32_t b = __builtin_amdgcn_perm(0u, e, 0x0c030c01u);  // bytes 1, 3
  uint64_t p = ((uint64_t)b << 32) | a;                       // fields 0 2 | 1 3
#pragma unroll
  for (int j = 1; j < 6; ++j) {
    p = times3(p);
    const uint32_t r =
        __builtin_amdgcn_perm((uint32_t)(p >> 32), (uint32_t)p, 0x06020400u);
    g[j] = __builtin_amdgcn_sdot4((int)r, x, g[j], false);
  }
}

template <int LPR, int NP, bool EXACT>
__global__ __launch_bounds__(reg_block_threads(LPR)) void gemv3_kernel(Gemv3Args g) {
  constexpr int BT = reg_block_threads(LPR);
  constexpr int G = BT / LPR;                         // teams per block
  constexpr int GL = LPR < kWave ? LPR : kWave;       // DPP reduction width
  constexpr int WPT = LPR > kWave ? LPR / kWave : 1;  // waves per team
  constexpr int SPAN = NP * LPR;
  constexpr int SP = (SPAN + BT - 1) / BT;
  static_assert(NP >= 1 && SPAN <= kRegMaxPieces, "pieces per lane");
  __shared__ u32x4 x_lds[SP * BT];
  __shared__ int red[2][BT / kWave][6];

  const int kp = g.kp, n5 = g.n5;
  const int lane = threadIdx.x % LPR;
  const int team = threadIdx.x / LPR;
  const int wave = threadIdx.x / kWave;
  const int row_stride = gridDim.x * G;
  const int rb0 = blockIdx.x * G;  // < n5 for every launched block
  const int its = (n5 - 1 - rb0) / row_stride + 1;
  const uint4 *P = reinterpret_cast<const uint4 *>(g.p);
  auto piece = [&](int t) {
    const int p = lane + t * LPR;
    return EXACT ? p : min(p, kp - 1);
  };

  // 1. activation loads (static count), then the first row's weights
  const u32x4 *xg = reinterpret_cast<const u32x4 *>(g.xq);
  u32x4 xs[SP];
#pragma unroll
  for (int s = 0; s < SP; ++s) {
    const int p = (int)threadIdx.x + s * BT;
    xs[s] = xg[EXACT ? min(p, SPAN - 1) : min(p, kp - 1)];
  }
  __builtin_amdgcn_sched_barrier(0);
  auto issue = [&](uint4 (&w)[NP], int rbase) {
    const int row = min(rbase + team, n5 - 1);
    const uint4 *rp = P + (size_t)row * kp;
#pragma unroll
    for (int t = 0; t < NP; ++t) w[t] = load_stream16(rp + piece(t));
  };
  uint4 wa[NP];
  issue(wa, rb0);
  __builtin_amdgcn_sched_barrier(0);

  // 2. stage x through LDS; keep this lane's pieces in VGPRs (zero past K)
#pragma unroll
  for (int s = 0; s < SP; ++s) x_lds[threadIdx.x + s * BT] = xs[s];
  __syncthreads();
  uint4 xr[NP];
#pragma unroll
  for (int t = 0; t < NP; ++t) {
    const int p = lane + t * LPR;
    const u32x4 v = x_lds[p];
    xr[t] = (EXACT || p < kp) ? make_uint4(v[0], v[1], v[2], v[3]) : make_uint4(0, 0, 0, 0);
  }
  const float c = g.s_w * g.x_scale[0];

  int buf = 0;
  auto consume = [&](uint4 (&w)[NP], int rbase) {
    int a[6] = {0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < NP; ++t) {
      dot_levels(w[t].x, (int)xr[t].x, a);
      dot_levels(w[t].y, (int)xr[t].y, a);
      dot_levels(w[t].z, (int)xr[t].z, a);
      dot_levels(w[t].w, (int)xr[t].w, a);
    }
#pragma unroll
    for (int j = 0; j < 6; ++j) a[j] = group_sum_to_last<GL>(a[j]);
    const int i = rbase + team;
    // digit 4-j of packed row i is output row (4-j)*n5 + i
    auto emit = [&](const int (&v)[6], int j) {
      const int n = (4 - j) * n5 + i;
      if (i >= n5 || n >= g.N) return;
      const int t = (int)(3u * (uint32_t)v[j] - (uint32_t)v[j + 1]) >> 8;  // exact
      if (g.acc) g.acc[n] = t;
      g.y[n] = rescale(t, c);
    };
    if constexpr (WPT == 1) {
      if (lane == LPR - 1) {
#pragma unroll
        for (int j = 0; j < 5; ++j) emit(a, j);
      }
    } else {
      if ((threadIdx.x & (kWave - 1)) == kWave - 1) {
#pragma unroll
        for (int j = 0; j < 6; ++j) red[buf][wave][j] = a[j];
      }
      __syncthreads();
      if (lane < 5) {
        int v[6];
#pragma unroll
        for (int j = 0; j < 6; ++j) {
          v[j] = 0;
#pragma unroll
          for (int w2 = 0; w2 < WPT; ++w2) v[j] += red[buf][team * WPT + w2][j];
        }
        emit(v, lane);
      }
      buf ^= 1;  // the next row's partials go to the other buffer
    }
  };

  consume(wa, rb0);
  for (int it = 1; it < its; ++it) {
    issue(wa, rb0 + it * row_stride);
    // Every load of the row ahead of its decode (left alone, the scheduler
    // waits for the first pieces after issuing two loads and spreads the
    // rest of the row's loads over the decode).
    __builtin_amdgcn_sched_barrier(0);
    consume(wa, rb0 + it * row_stride);
  }
}

struct Plan3 {
  int lpr, np, blocks;
  bool exact;
  bool persistent;  // 256-thread blocks capped per CU, rows walked
  int cus;
};

// As the two-bit kernel's plan: the narrowest team with at most 8 pieces per
// lane, 64-lane teams when rows are few; grids of at most 5 blocks per CU
// for 256-thread blocks, lowered at launch to what the compiled kernel lets
// a CU hold (this VALU-heavy decode gains from more waves per SIMD:
// measured on MI355X, [28672,8192] 14.0 against 14.6 us with 3 per CU,
// [57344,4096] 14.4 against 15.2 us), and 4 for 512-thread blocks.  A CU
// holds 3 of the 512-thread blocks at 7 pieces per lane (76 VGPRs) and 2 at
// 8 (96), so a grid of one row per team beyond that runs as a second,
// partial wave of blocks; measured on MI355X it still beat a grid of 2
// blocks per CU whose teams walk two rows (15.9 against 16.8 us at
// [8192,28672] with the former 24-operation decode: 820 blocks of one row
// per team), so those grids are not lowered.
Plan3 plan3(int64_t n5, int64_t kp, int num_cus) {
  Plan3 pl{};
  int lpr = 16;
  while ((kp + lpr - 1) / lpr > 8) lpr *= 2;
  const int64_t want_lanes = (int64_t)num_cus * 16 * kWave;
  if (lpr < 64 && n5 * lpr < want_lanes) lpr = 64;
  pl.lpr = lpr;
  pl.np = (int)((kp + lpr - 1) / lpr);
  pl.exact = (int64_t)pl.np * lpr == kp;
  const int bt = reg_block_threads(lpr);
  const int64_t teams = bt / lpr;
  int64_t blocks = (n5 + teams - 1) / teams;
  const int64_t cap = (int64_t)num_cus * (bt == 512 ? 4 : 5);
  pl.persistent = blocks > cap && bt != 512;
  if (blocks > cap) blocks = cap;
  pl.blocks = (int)(blocks < 1 ? 1 : blocks);
  pl.cus = num_cus;
  return pl;
}

template <int LPR, int NP, bool EXACT>
tq_status launch3_form(const Plan3 &pl, const Gemv3Args &a, hipStream_t s) {
  auto kernel = gemv3_kernel<LPR, NP, EXACT>;
  const dim3 block(reg_block_threads(LPR));
  int blocks = pl.blocks;
  if (pl.persistent) {
    static std::atomic<int> occ;
    const int n = resident_blocks(kernel, (int)block.x, occ);
    if (n > 0 && (int64_t)blocks > (int64_t)n * pl.cus) blocks = n * pl.cus;
  }
  return launch(kernel, dim3(blocks), block, 0, s, a);
}

template <int LPR, int NP>
tq_status launch3_np(const Plan3 &pl, const Gemv3Args &a, hipStream_t s) {
  return pl.exact ? launch3_form<LPR, NP, true>(pl, a, s)
                  : launch3_form<LPR, NP, false>(pl, a, s);
}

template <int LPR>
tq_status launch3_lpr(const Plan3 &pl, const Gemv3Args &a, hipStream_t s) {
  switch (pl.np) {
    case 1: return launch3_np<LPR, 1>(pl, a, s);
    case 2: return launch3_np<LPR, 2>(pl, a, s);
    case 3: return launch3_np<LPR, 3>(pl, a, s);
    case 4: return launch3_np<LPR, 4>(pl, a, s);
    case 5: return launch3_np<LPR, 5>(pl, a, s);
    case 6: return launch3_np<LPR, 6>(pl, a, s);
    case 7: return launch3_np<LPR, 7>(pl, a, s);
    case 8: return launch3_np<LPR, 8>(pl, a, s);
  }
  return TQ_ERR_LAUNCH;
}

// ------------------------------------------------------------------ pack
// One thread per 16 packed bytes: five 16-byte pieces of weights (rows
// j*n5 + i, zero past N) -> one piece.  A weight outside {-1,0,1} makes its
// byte the reserved value 1 (no v encodes to 1).
__global__ __launch_bounds__(256) void pack3_kernel(const uint4 *__restrict__ w,
                                                    int64_t N, int64_t n5, int64_t kp,
                                                    uint4 *__restrict__ packed) {
  const int64_t total = n5 * kp;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = t / kp, p = t % kp;
    uint32_t v[16], bad[16];
#pragma unroll
    for (int b = 0; b < 16; ++b) v[b] = bad[b] = 0;
    uint32_t p3 = 1;
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const int64_t n = j * n5 + i;
      u32x4 r = {0, 0, 0, 0};  // padding rows: weight 0
      if (n < N) {
        const uint4 q = w[n * kp + p];
        r = u32x4{q.x, q.y, q.z, q.w};
      }
#pragma unroll
      for (int b = 0; b < 16; ++b) {
        const int wv = (int)(int8_t)((r[b / 4] >> (8 * (b % 4))) & 0xffu);
        bad[b] |= (wv < -1 || wv > 1);
        v[b] += (uint32_t)(wv + 1) * p3;
      }
      p3 *= 3;
    }
    u32x4 o = {0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const uint32_t q = bad[b] ? 1u : (v[b] * 256u + 242u) / 243u;
      o[b / 4] |= q << (8 * (b % 4));
    }
    packed[t] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

}  // namespace
}  // namespace tq

extern "C" tq_status tq_pack3(const int8_t *w, int64_t N, int64_t K, uint8_t *packed,
                              hipStream_t stream) {
  using namespace tq;
  if (N < 0 || K < 0 || K % 16 != 0) return TQ_ERR_SHAPE;
  if (N == 0 || K == 0) return TQ_OK;
  if (!w || !packed) return TQ_ERR_NULL;
  if (!aligned(w, 16) || !aligned(packed, 16)) return TQ_ERR_ALIGN;
  DeviceInfo dev;
  if (tq_status s = current_device(&dev)) return s;
  const int64_t n5 = (N + 4) / 5, kp = K / 16;
  const int64_t total = n5 * kp;
  int64_t blocks = (total + 255) / 256;
  const int64_t cap = (int64_t)dev.num_cus * 16;
  if (blocks > cap) blocks = cap;
  return launch(pack3_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                reinterpret_cast<const uint4 *>(w), N, n5, kp,
                reinterpret_cast<uint4 *>(packed));
}

extern "C" tq_status tq_gemv3(const uint8_t *packed, float w_scale, const int8_t *xq,
                              const float *x_scale, int64_t N, int64_t K, float *y,
                              int32_t *acc, hipStream_t stream) {
  using namespace tq;
  if (N < 0 || K < 16 || K % 16 != 0 || K > 16 * kRegMaxPieces) return TQ_ERR_SHAPE;
  if ((N + 4) / 5 > (int64_t)INT32_MAX) return TQ_ERR_SHAPE;
  if (N == 0) return TQ_OK;
  if (!packed || !xq || !x_scale || !y) return TQ_ERR_NULL;
  if (!aligned(packed, 16) || !aligned(xq, 16) || !aligned(y, 4) ||
      !aligned(acc, 4) || !aligned(x_scale, 4))
    return TQ_ERR_ALIGN;
  DeviceInfo dev;
  if (tq_status s = current_device(&dev)) return s;
  Gemv3Args a;
  a.p = packed;
  a.s_w = w_scale;
  a.xq = xq;
  a.x_scale = x_scale;
  a.N = (int)N;
  a.n5 = (int)((N + 4) / 5);
  a.kp = (int)(K / 16);
  a.y = y;
  a.acc = acc;
  const Plan3 pl = plan3(a.n5, a.kp, dev.num_cus);
  switch (pl.lpr) {
    case 16: return launch3_lpr<16>(pl, a, stream);
    case 32: return launch3_lpr<32>(pl, a, stream);
    case 64: return launch3_lpr<64>(pl, a, stream);
    case 128: return launch3_lpr<128>(pl, a, stream);
    case 256: return launch3_lpr<256>(pl, a, stream);
  }
  return TQ_ERR_LAUNCH;
}
