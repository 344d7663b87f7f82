// tq_device.h -- device-side building blocks shared by the gfx950 kernels.
//
// Packed ternary layout (see include/tq.h): byte [i,k] of a [N/4,K] array
// holds the code w+1 of row j*(N/4)+i in bits 2j..2j+1.  A dword of a packed
// row therefore carries 4 consecutive k of 4 rows ("planes"); one 16-byte
// load carries 16 k of 4 rows = 64 weights.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

constexpr int kWave = 64;

// ---------------------------------------------------------------- loads
// 16-byte streaming load of weights: read once, so hint non-temporal.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream16(const uint4 *p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// ---------------------------------------------------------------- decode
// Offset codes c = w + 1 in {0,1,2}.  For one dword d of a packed row:
//   plane 0: d & 0x03030303         -> c0          (bytes 0..2)
//   plane 1: d & 0x0C0C0C0C         -> 4*c1        (bytes 0..8)
//   plane 2: d & 0x30303030         -> 16*c2       (bytes 0..32)
//   plane 3: (d >> 2) & 0x30303030  -> 16*c3       (bytes 0..32)
// Every byte stays a non-negative int8, so v_dot4_i32_i8 with the int8
// activations gives 1x, 4x, 16x, 16x the plane sums sum(c*q); the scale is
// removed exactly by an arithmetic shift after the reduction, and
// sum(w*q) = sum(c*q) - sum(q).
__device__ __forceinline__ void dot_planes(uint32_t d, int x, int &a0, int &a1,
                                           int &a2, int &a3) {
  a0 = __builtin_amdgcn_sdot4((int)(d & 0x03030303u), x, a0, false);
  a1 = __builtin_amdgcn_sdot4((int)(d & 0x0C0C0C0Cu), x, a1, false);
  a2 = __builtin_amdgcn_sdot4((int)(d & 0x30303030u), x, a2, false);
  a3 = __builtin_amdgcn_sdot4((int)((d >> 2) & 0x30303030u), x, a3, false);
}

__device__ __forceinline__ void dot_planes16(const uint4 &w, const uint4 &x,
                                             int (&a)[4]) {
  dot_planes(w.x, (int)x.x, a[0], a[1], a[2], a[3]);
  dot_planes(w.y, (int)x.y, a[0], a[1], a[2], a[3]);
  dot_planes(w.z, (int)x.z, a[0], a[1], a[2], a[3]);
  dot_planes(w.w, (int)x.w, a[0], a[1], a[2], a[3]);
}

// Undo the per-plane scale and the code offset: exact int32.
__device__ __forceinline__ int plane_value(int j, int scaled, int sumq) {
  const int sh = j == 0 ? 0 : (j == 1 ? 2 : 4);
  return (scaled >> sh) - sumq;
}

// Sum of the 4 int8 lanes of each dword of a 16-byte piece.
__device__ __forceinline__ int sum_bytes16(const uint4 &v, int acc) {
  acc = __builtin_amdgcn_sdot4((int)v.x, 0x01010101, acc, false);
  acc = __builtin_amdgcn_sdot4((int)v.y, 0x01010101, acc, false);
  acc = __builtin_amdgcn_sdot4((int)v.z, 0x01010101, acc, false);
  acc = __builtin_amdgcn_sdot4((int)v.w, 0x01010101, acc, false);
  return acc;
}

// ---------------------------------------------------------------- DPP
// DPP controls (GCN/CDNA encoding).
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114,
              kRowShr8 = 0x118, kRowBcast15 = 0x142, kRowBcast31 = 0x143;

template <int Ctrl, int RowMask = 0xf>
__device__ __forceinline__ int dpp_i32(int v) {
  // Lanes whose source is outside the row (or whose row is masked off)
  // receive 0, so "v + dpp(v)" leaves them unchanged.
  return __builtin_amdgcn_update_dpp(0, v, Ctrl, RowMask, 0xf, false);
}

// Sum over aligned groups of G lanes (G = 16, 32 or 64).  The total lands in
// the LAST lane of each group (lane G-1 mod G); other lanes hold partials.
template <int G>
__device__ __forceinline__ int group_sum_to_last(int v) {
  static_assert(G == 16 || G == 32 || G == 64, "group size");
  v += dpp_i32<kRowShr1>(v);
  v += dpp_i32<kRowShr2>(v);
  v += dpp_i32<kRowShr4>(v);
  v += dpp_i32<kRowShr8>(v);
  if constexpr (G >= 32) v += dpp_i32<kRowBcast15, 0xa>(v);
  if constexpr (G >= 64) v += dpp_i32<kRowBcast31, 0xc>(v);
  return v;
}

// All-reduce over the wave with no LDS round trip, result in every lane:
// the two halves, then the two rows of each half, exchanged by gfx950's
// v_permlane32_swap / v_permlane16_swap (called with one value as both
// operands, the two results hold the two partners of every lane pair), then
// DPP rotates by 8, 4, 2, 1 within each 16-lane row (after rotating by 8,
// each lane holds lanes {i, i+8}; after 4, {i, i+4, i+8, i+12}; and so on).
// For an associative, commutative, exact op (max, integer sums) every
// pairing gives the same result.
constexpr int kRowRor1 = 0x121, kRowRor2 = 0x122, kRowRor4 = 0x124, kRowRor8 = 0x128;

template <typename Op>
__device__ __forceinline__ uint32_t wave_allreduce(uint32_t v, Op op) {
  const auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = op(h[0], h[1]);
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op(r[0], r[1]);
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowRor8, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowRor4, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowRor2, 0xf, 0xf, false));
  return op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowRor1, 0xf, 0xf, false));
}

// Float max over the whole wave, result valid in every lane.
__device__ __forceinline__ float wave_max(float v) {
  return __uint_as_float(wave_allreduce(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}

__device__ __forceinline__ int wave_sum(int v) {
  return (int)wave_allreduce((uint32_t)v, [](uint32_t a, uint32_t b) { return a + b; });
}

// ---------------------------------------------------------------- act quant
// One piece = 16 consecutive activations of a row, kept in its raw input form
// (bf16: two 16-byte words; fp32: four).
template <bool kBf16>
struct RawPiece {
  static constexpr int kWords = kBf16 ? 2 : 4;
  u32x4 w[kWords];
};

template <bool kBf16>
__device__ __forceinline__ RawPiece<kBf16> load_piece(const void *x,
                                                      int64_t piece) {
  const u32x4 *p = reinterpret_cast<const u32x4 *>(x) + piece * RawPiece<kBf16>::kWords;
  RawPiece<kBf16> r;
#pragma unroll
  for (int i = 0; i < RawPiece<kBf16>::kWords; ++i) r.w[i] = p[i];
  return r;
}

// Absmax on bit patterns.  For finite floats, |x| orders exactly like the
// bit pattern with the sign bit cleared, so the row maximum of |x| can be
// taken with unsigned integer max on raw words: bf16 pairs with one packed
// 16-bit max per word, fp32 with one 32-bit max.  `m` carries the running
// maximum (bf16: two halves, folded by absmax_value).
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

template <bool kBf16>
__device__ __forceinline__ uint32_t absmax_bits(const RawPiece<kBf16> &r,
                                                uint32_t m) {
#pragma unroll
  for (int i = 0; i < RawPiece<kBf16>::kWords; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (kBf16) {
        const u16x2 a = __builtin_bit_cast(u16x2, r.w[i][j] & 0x7fff7fffu);
        const u16x2 b = __builtin_bit_cast(u16x2, m);
        m = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
      } else {
        const uint32_t a = r.w[i][j] & 0x7fffffffu;
        m = a > m ? a : m;
      }
    }
  return m;
}

template <bool kBf16>
__device__ __forceinline__ float absmax_value(uint32_t m) {
  if constexpr (kBf16) {
    const uint32_t lo = m & 0xffffu, hi = m >> 16;
    return __uint_as_float((lo > hi ? lo : hi) << 16);
  } else {
    return __uint_as_float(m);
  }
}

// Four fp32 values -> four int8 codes rne(v * inv) in one dword.
//
// Rounding: for |y| < 2^22, fl(y + 1.5*2^23) = 1.5*2^23 + rne(y) exactly
// (the sum's ulp is 1 and the add rounds half to even), so the low byte of
// its bit pattern is rne(y) in two's complement.  The product y = fl(v*inv)
// is rounded on its own first (no contraction into an fma).
// Clamp: every v of the row has |v| <= a' and inv = fl(127/a'), so
// |y| <= fl(a' * fl(127/a')) <= 127 + 2^-17 and |rne(y)| <= 127: the clamp
// to [-127, 127] of the quantization rule never binds and is not applied.
constexpr float kRneMagic = 12582912.0f;  // 1.5 * 2^23

__device__ __forceinline__ uint32_t quant4(const float (&v)[4], float inv) {
#pragma clang fp contract(off)
  uint32_t b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float y = v[i] * inv;
    b[i] = __float_as_uint(y + kRneMagic);
  }
  // v_perm_b32 byte selects: {src0, src1} = bytes 7..4, 3..0; 0x0c -> 0x00.
  const uint32_t lo = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// A whole piece -> 16 int8 codes (16 bytes, in k order).
template <bool kBf16>
__device__ __forceinline__ u32x4 quant_piece(const RawPiece<kBf16> &r,
                                             float inv) {
  u32x4 q;
  if constexpr (kBf16) {
    // word i, dword j holds k = 8i + 2j (low half) and 8i + 2j + 1 (high).
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t w0 = r.w[d / 2][2 * (d % 2)];
      const uint32_t w1 = r.w[d / 2][2 * (d % 2) + 1];
      const float v[4] = {__uint_as_float(w0 << 16),
                          __uint_as_float(w0 & 0xffff0000u),
                          __uint_as_float(w1 << 16),
                          __uint_as_float(w1 & 0xffff0000u)};
      q[d] = quant4(v, inv);
    }
  } else {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float v[4] = {__uint_as_float(r.w[d][0]), __uint_as_float(r.w[d][1]),
                          __uint_as_float(r.w[d][2]), __uint_as_float(r.w[d][3])};
      q[d] = quant4(v, inv);
    }
  }
  return q;
}

// ---------------------------------------------------------------- RMSNorm
// Sub-layer RMSNorm folded into the quantization: the codes are those of
// u = x * gamma (one fp32 rounding per value), and 1/sqrt(mean(x^2) + eps)
// goes into the scale.  Value k (0..15) of a raw piece:
template <bool kBf16>
__device__ __forceinline__ float piece_value(const RawPiece<kBf16> &r, int k) {
  if constexpr (kBf16) {
    const uint32_t w = r.w[k / 8][(k % 8) / 2];
    return __uint_as_float(k % 2 ? (w & 0xffff0000u) : (w << 16));
  } else {
    return __uint_as_float(r.w[k / 4][k % 4]);
  }
}

// u = x * gamma for one piece, as an fp32 piece; adds sum(x^2) to `ss` in
// fp64 (each square is exact there; fma and mul + add agree).
template <bool kBf16>
__device__ __forceinline__ RawPiece<false> scale_piece(const RawPiece<kBf16> &x,
                                                       const RawPiece<kBf16> &g,
                                                       double &ss) {
#pragma clang fp contract(off)
  RawPiece<false> u;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const float xv = piece_value<kBf16>(x, k);
    u.w[k / 4][k % 4] = __float_as_uint(xv * piece_value<kBf16>(g, k));
    ss = fma((double)xv, (double)xv, ss);
  }
  return u;
}

// The value of lane (lane ^ OFF), one 32-bit word, with no LDS round trip:
// OFF = 8 is a DPP rotate by 8 within each 16-lane row; OFF = 4 takes
// lane + 4 in the first and third 4-lane bank of each row and lane - 4 in
// the others (two DPP shifts, each restricted by the bank mask); OFF = 2
// and 1 are quad permutations.
template <int OFF>
__device__ __forceinline__ uint32_t lane_xor_dpp(uint32_t v) {
  static_assert(OFF == 8 || OFF == 4 || OFF == 2 || OFF == 1, "DPP lane offset");
  const int x = (int)v;
  if constexpr (OFF == 8) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, x, kRowRor8, 0xf, 0xf, false);
  } else if constexpr (OFF == 4) {
    const int t = __builtin_amdgcn_update_dpp(x, x, 0x104 /* row_shl:4 */, 0xf, 0x5, false);
    return (uint32_t)__builtin_amdgcn_update_dpp(t, x, 0x114 /* row_shr:4 */, 0xf, 0xa, false);
  } else if constexpr (OFF == 2) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x4e /* quad_perm 2,3,0,1 */, 0xf, 0xf, false);
  } else {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0xb1 /* quad_perm 1,0,3,2 */, 0xf, 0xf, false);
  }
}

// fp64 sum over a wave as an xor butterfly (lanes 32, 16, 8, 4, 2, 1 apart):
// every lane ends with the same value, since each step adds the same two
// partial sums in either order.  The pairs 32 and 16 apart come from the
// row-swap instructions, the rest from DPP, each on both halves of the
// double; no LDS round trip.
__device__ __forceinline__ double wave_sum_f64(double v) {
  auto halves = [](double d, uint32_t &lo, uint32_t &hi) {
    const unsigned long long b = (unsigned long long)__double_as_longlong(d);
    lo = (uint32_t)b;
    hi = (uint32_t)(b >> 32);
  };
  auto join = [](uint32_t lo, uint32_t hi) {
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
  };
  uint32_t lo, hi;
  halves(v, lo, hi);
  {
    const auto l = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto h = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    v = join(l[0], h[0]) + join(l[1], h[1]);
  }
  halves(v, lo, hi);
  {
    const auto l = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto h = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    v = join(l[0], h[0]) + join(l[1], h[1]);
  }
  halves(v, lo, hi);
  v += join(lane_xor_dpp<8>(lo), lane_xor_dpp<8>(hi));
  halves(v, lo, hi);
  v += join(lane_xor_dpp<4>(lo), lane_xor_dpp<4>(hi));
  halves(v, lo, hi);
  v += join(lane_xor_dpp<2>(lo), lane_xor_dpp<2>(hi));
  halves(v, lo, hi);
  return v + join(lane_xor_dpp<1>(lo), lane_xor_dpp<1>(hi));
}

// The RMS factor, rounded once to fp32: 1 / sqrt(ss / K + eps) in fp64.
__device__ __forceinline__ float rms_factor(double ss, int64_t K, float eps) {
  return (float)(1.0 / sqrt(ss / (double)K + (double)eps));
}

// ---------------------------------------------------------------- epilogue
// y = (float)acc * (s_w * s_x): two fp32 roundings, in this order.
__device__ __forceinline__ float rescale(int acc, float c) {
  return (float)acc * c;
}

__device__ __forceinline__ float relu2_gate(float g, float u) {
  const float r = g > 0.0f ? g : 0.0f;
  return (r * r) * u;
}

}  // namespace tq
