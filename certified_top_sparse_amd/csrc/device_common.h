// Device-side helpers shared by the libctopk kernels (gfx950 / CDNA4).
//
// Selection order (Abstract of "A Mathematical Theory of Top-k Sparse
// Attention via Total Variation Distance", arXiv 2512.07647: the head H is the
// k largest-score keys; equal scores are ordered by index ascending, the lower
// index entering the head first) is encoded as one 64-bit integer per key:
//
//   key64(s, i) = ukey(s) << 32 | (0xFFFFFFFF - i)
//
// where ukey is the order-preserving map of an fp32 score to uint32 (-0.0 is
// folded onto +0.0 first, so the two compare equal).  A larger key64 means
// "earlier in the order".  All key64 values of one row are distinct, so the
// head is exactly { i : key64(s_i, i) >= key64 of its last member }.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ctopk {

constexpr int kWave = 64;

// Digit schedule of the mass-weighted radix select over key64: 5 x 11 + 9 bits.
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;
constexpr int kLevels = 6;

__device__ __forceinline__ int digit_width(int level) { return level < 5 ? 11 : 9; }

__device__ __forceinline__ uint32_t ukey(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;  // -0.0 -> +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float ukey_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t key64(float s, uint32_t idx) {
  return (static_cast<uint64_t>(ukey(s)) << 32) | static_cast<uint64_t>(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ uint32_t key64_index(uint64_t k) {
  return 0xFFFFFFFFu - static_cast<uint32_t>(k & 0xFFFFFFFFull);
}

__device__ __forceinline__ float key64_score(uint64_t k) {
  return ukey_to_float(static_cast<uint32_t>(k >> 32));
}

// Unnormalised softmax weight w = exp(s - m) in fp32 (s <= m).  The fp32
// difference d = s - m carries a rounding error err that two-sum recovers
// exactly; d * log2(e) is split with an fma into th + tl (log2(e) itself in
// two fp32 parts).  Then exp(s - m) = 2^th * 2^tl * e^err, and to first order
// w = e2 * (1 + tl ln2 + err) with e2 = 2^th from the hardware base-2
// exponential, so w carries about the error of that one instruction rather
// than that of an exponential at a rounded argument.  Every kernel uses this
// one definition, so the selection, tau and the output all see identical
// weights.  Results below 2^-126 (weights under ~1e-38 of the row maximum)
// may flush to zero.
__device__ __forceinline__ float weight(float s, float m) {
  const float d = s - m;
  const float bv = d - s;
  const float av = d - bv;
  const float err = (s - av) + (-m - bv);
  constexpr float kLog2e = 1.44269502162933349609375f;   // log2(e) rounded to fp32
  constexpr float kLog2eLo = 1.925963033500011079e-8f;  // log2(e) - kLog2e
  constexpr float kLn2 = 0.693147182464599609375f;      // ln(2) rounded to fp32
  const float th = d * kLog2e;
  const float tl = fmaf(d, kLog2eLo, fmaf(d, kLog2e, -th));
  const float e2 = __builtin_amdgcn_exp2f(th);
  return fmaf(e2, fmaf(tl, kLn2, err), e2);
}

// 16-byte load of data that is streamed once (K in the score scan, V in the
// value stream): the non-temporal hint keeps it from displacing reused lines
// (scores, partials) in the caches.
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 x = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}

// ---------------------------------------------------------------------------
// DPP lane exchanges (full-rate VALU, no LDS traffic)
// ---------------------------------------------------------------------------
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within each 8
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i within each 16

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Maximum over the 64 lanes, returned in every lane (DPP within rows of 16,
// then the four row results through scalar lane reads).
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  v = fmaxf(v, dpp<kDppMirror>(v));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(u & 0xFFFFFFFFu), CTRL, 0xF, 0xF, false));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(u >> 32), CTRL, 0xF, 0xF, false));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// Sum over each row of 16 lanes, in every lane of the row: quad exchanges,
// then the mirror patterns that pair each lane with one in the other half
// (every lane of a row ends with the bitwise-same value, a + b == b + a).
__device__ __forceinline__ double row_sum_f64(double v) {
  v += dpp_f64<kDppXor1>(v);
  v += dpp_f64<kDppXor2>(v);
  v += dpp_f64<kDppHalfMirror>(v);
  v += dpp_f64<kDppMirror>(v);
  return v;
}

// ---------------------------------------------------------------------------
// Cross-row adds (gfx950): v_permlane16_swap exchanges rows 0 <-> 1 and
// 2 <-> 3 of a wave between its two operands, v_permlane32_swap the two
// 32-lane halves; each is one VALU instruction with no LDS traffic.  Given
// the same value twice, the two results hold, in both lanes of a pair (l and
// l ^ 16, or l and l ^ 32), that pair's two values, so their sum is the
// bitwise-same number in both lanes.  Every lane of the wave must be active.
// ---------------------------------------------------------------------------
// The two values of the lane pair (l, l ^ X), X = 16 or 32, in both lanes
// of the pair (callers use them in ways that do not depend on their order).
template <int X>
__device__ __forceinline__ uint2 lane_pair(uint32_t v) {
  static_assert(X == 16 || X == 32, "cross-row pair");
  if constexpr (X == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return make_uint2(p[0], p[1]);
  } else {
    const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return make_uint2(p[0], p[1]);
  }
}

// The value of lane l ^ X, as __shfl_xor(v, X) for X = 16 or 32: of the
// pair's two values the one that is not this lane's own (equal values: the
// same number either way).
template <int X>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  const uint2 p = lane_pair<X>(v);
  return p.x == v ? p.y : p.x;
}
template <int X>
__device__ __forceinline__ int xor_lane(int v) {
  return static_cast<int>(xor_lane<X>(static_cast<uint32_t>(v)));
}
template <int X>
__device__ __forceinline__ float xor_lane(float v) {
  return __uint_as_float(xor_lane<X>(__float_as_uint(v)));
}
template <int X>
__device__ __forceinline__ double xor_lane(double v) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const uint32_t lo = xor_lane<X>(static_cast<uint32_t>(u));
  const uint32_t hi = xor_lane<X>(static_cast<uint32_t>(u >> 32));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

__device__ __forceinline__ float xrow16_sum(float v) {
  const uint2 p = lane_pair<16>(__float_as_uint(v));
  return __uint_as_float(p.x) + __uint_as_float(p.y);
}

__device__ __forceinline__ float xrow32_sum(float v) {
  const uint2 p = lane_pair<32>(__float_as_uint(v));
  return __uint_as_float(p.x) + __uint_as_float(p.y);
}

__device__ __forceinline__ double join_f64(uint32_t hi, uint32_t lo) {
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

template <int X>
__device__ __forceinline__ double xrow_sum_f64(double v) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const uint2 pl = lane_pair<X>(static_cast<uint32_t>(u));
  const uint2 ph = lane_pair<X>(static_cast<uint32_t>(u >> 32));
  return join_f64(ph.x, pl.x) + join_f64(ph.y, pl.y);
}
__device__ __forceinline__ double xrow16_sum(double v) { return xrow_sum_f64<16>(v); }
__device__ __forceinline__ double xrow32_sum(double v) { return xrow_sum_f64<32>(v); }

// Sum over aligned groups of L consecutive lanes (L a power of two <= 64);
// on return every lane of a group holds the group's sum.  After the two quad
// steps all lanes of a quad agree, so the mirror patterns (which pair each
// lane with one in the other half) complete the 8- and 16-lane sums.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (L >= 2) v += dpp<kDppXor1>(v);
  if constexpr (L >= 4) v += dpp<kDppXor2>(v);
  if constexpr (L >= 8) v += dpp<kDppHalfMirror>(v);
  if constexpr (L >= 16) v += dpp<kDppMirror>(v);
  if constexpr (L >= 32) v = xrow16_sum(v);
  if constexpr (L >= 64) v = xrow32_sum(v);
  return v;
}

// Sum over the 64 lanes in a fixed tree, (row 0 + row 1) + (row 2 + row 3)
// of the row sums, the same value in every lane.
__device__ __forceinline__ double wave_sum_f64(double v) {
  return xrow32_sum(xrow16_sum(row_sum_f64(v)));
}

// Sum over the lanes that share their position modulo S (S = 8, 16 or 32:
// lanes l ^ 8 within a row, then across rows), in every lane, in a fixed
// tree.  Every lane of the wave must be active.
constexpr int kDppRowRor8 = 0x128;  // lane i <- lane (i + 8) mod 16 within each 16
template <int S, typename A>
__device__ __forceinline__ A stride_sum(A v) {
  static_assert(S == 8 || S == 16 || S == 32, "lane stride");
  if constexpr (S == 8) {
    if constexpr (sizeof(A) == 8) {
      v += dpp_f64<kDppRowRor8>(v);
    } else {
      v += dpp<kDppRowRor8>(v);
    }
  }
  if constexpr (S <= 16) v = xrow16_sum(v);
  return xrow32_sum(v);
}

__device__ __forceinline__ uint32_t wave_sum_u32_dpp(uint32_t v) {
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kDppXor1, 0xF, 0xF, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kDppXor2, 0xF, 0xF, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kDppHalfMirror, 0xF, 0xF, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kDppMirror, 0xF, 0xF, false));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 0)) +
         static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 16)) +
         static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 32)) +
         static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 48));
}

// Inclusive prefix sums across the 64 lanes with DPP: shifts by 1, 2, 4 and 8
// within each row of 16 (lanes shifted in from outside the row add 0), then
// each row takes the running total of the rows before it (row broadcasts of
// lanes 15 and 31).
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROWS, 0xF, true));
}

template <int CTRL, int ROWS>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long v) {
  const uint32_t lo = dpp_u32<CTRL, ROWS>(static_cast<uint32_t>(v));
  const uint32_t hi = dpp_u32<CTRL, ROWS>(static_cast<uint32_t>(v >> 32));
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

__device__ __forceinline__ unsigned long long wave_incl_scan_u64_dpp(unsigned long long v) {
  v += dpp_u64<kDppRowShr1, 0xF>(v);
  v += dpp_u64<kDppRowShr2, 0xF>(v);
  v += dpp_u64<kDppRowShr4, 0xF>(v);
  v += dpp_u64<kDppRowShr8, 0xF>(v);
  v += dpp_u64<kDppRowBcast15, 0xA>(v);
  v += dpp_u64<kDppRowBcast31, 0xC>(v);
  return v;
}

__device__ __forceinline__ uint32_t wave_incl_scan_u32_dpp(uint32_t v) {
  v += dpp_u32<kDppRowShr1, 0xF>(v);
  v += dpp_u32<kDppRowShr2, 0xF>(v);
  v += dpp_u32<kDppRowShr4, 0xF>(v);
  v += dpp_u32<kDppRowShr8, 0xF>(v);
  v += dpp_u32<kDppRowBcast15, 0xA>(v);
  v += dpp_u32<kDppRowBcast31, 0xC>(v);
  return v;
}

// Inclusive prefix sum of fp64 values across the 64 lanes, in the same
// pattern as the integer scans above (a fixed tree; lanes shifted in from
// outside a row, and rows a broadcast skips, add +0.0).
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64_bc(double v) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  return join_f64(dpp_u32<CTRL, ROWS>(static_cast<uint32_t>(u >> 32)),
                  dpp_u32<CTRL, ROWS>(static_cast<uint32_t>(u)));
}

__device__ __forceinline__ double wave_incl_scan_f64_dpp(double v) {
  v += dpp_f64_bc<kDppRowShr1, 0xF>(v);
  v += dpp_f64_bc<kDppRowShr2, 0xF>(v);
  v += dpp_f64_bc<kDppRowShr4, 0xF>(v);
  v += dpp_f64_bc<kDppRowShr8, 0xF>(v);
  v += dpp_f64_bc<kDppRowBcast15, 0xA>(v);
  v += dpp_f64_bc<kDppRowBcast31, 0xC>(v);
  return v;
}

// Minimum and maximum of 64-bit keys over the 64 lanes, in every lane (DPP
// within rows, then the cross-row swaps).  Every lane must be active.
template <bool MAX>
__device__ __forceinline__ unsigned long long pick_u64(unsigned long long a, unsigned long long b) {
  return MAX ? (a > b ? a : b) : (a < b ? a : b);
}

template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_u64_row(unsigned long long v) {
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v)), CTRL, 0xF, 0xF, false));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v >> 32)), CTRL, 0xF, 0xF, false));
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

template <bool MAX>
__device__ __forceinline__ unsigned long long wave_pick_u64(unsigned long long v) {
  v = pick_u64<MAX>(v, dpp_u64_row<kDppXor1>(v));
  v = pick_u64<MAX>(v, dpp_u64_row<kDppXor2>(v));
  v = pick_u64<MAX>(v, dpp_u64_row<kDppHalfMirror>(v));
  v = pick_u64<MAX>(v, dpp_u64_row<kDppMirror>(v));
  const uint2 a = lane_pair<16>(static_cast<uint32_t>(v));
  const uint2 b = lane_pair<16>(static_cast<uint32_t>(v >> 32));
  v = pick_u64<MAX>((static_cast<unsigned long long>(b.x) << 32) | a.x,
                    (static_cast<unsigned long long>(b.y) << 32) | a.y);
  const uint2 c = lane_pair<32>(static_cast<uint32_t>(v));
  const uint2 e = lane_pair<32>(static_cast<uint32_t>(v >> 32));
  return pick_u64<MAX>((static_cast<unsigned long long>(e.x) << 32) | c.x,
                       (static_cast<unsigned long long>(e.y) << 32) | c.y);
}

// What the select of a row hands to the value stream of the same launch,
// each word once with a device-scope store: first the level-0 bin that
// holds the cut, then the head's softmax mass (relative to the row maximum,
// fp64) and the cut key64.  Every word is zero before its store and non-zero
// after (the head holds at least the row's maximum, weight 1; ukey of a
// float is never zero).
struct CutPub {
  uint64_t cut;  // key64 of the cut
  double den;    // the head's mass
  uint64_t bin;  // (ukey(f0), ukey(f1)) of the level-0 bin [f0, f1) holding the cut
};

// Per-row scalars handed from the selection to the output kernel.
struct RowSel {
  float m;        // row maximum of the fp32 scores (weight reference)
  float lo;       // row minimum (lower edge of the level-0 value bins)
  double Z;       // sum of weights over the row (fp64)
  uint64_t thr;   // key64 of the last head member: key i is kept iff key64 >= thr
};

// Level-0 bins of the select: kBins equal-width value bins over [lo, hi].
// lin_bin is non-decreasing in s (IEEE subtraction and multiplication by a
// non-negative constant are monotone, as is truncation of a non-negative
// value), so every bin holds a contiguous range of the key64 order; any such
// partition serves the radix descent, and equal-width bins split Gaussian-like
// scores far more evenly than the top bits of the float encoding do.
__device__ __forceinline__ float lin_scale(float lo, float hi) {
  const float r = hi - lo;
  const float inv = static_cast<float>(kBins) / r;
  return (r > 0.0f && isfinite(inv)) ? inv : 0.0f;
}

__device__ __forceinline__ int lin_bin(float s, float lo, float inv) {
  const float x = (s - lo) * inv;
  return x < static_cast<float>(kBins) ? static_cast<int>(x) : kBins - 1;
}

// lin_bin for scores that may lie below lo (a range not taken from the row's
// own minimum): those fall into bin 0.  Equal to lin_bin for s >= lo.
__device__ __forceinline__ int lin_bin_clamped(float s, float lo, float inv) {
  const float x = fmaxf((s - lo) * inv, 0.0f);
  return x < static_cast<float>(kBins) ? static_cast<int>(x) : kBins - 1;
}

// Cooperative zeroing of a byte range by all blocks of a grid (16-byte units).
__device__ __forceinline__ void zero_slice(void* base, size_t bytes, size_t block_linear,
                                           size_t nblocks) {
  if (base == nullptr || bytes == 0) return;
  const size_t units = bytes / 16;
  uint4* p = reinterpret_cast<uint4*>(base);
  const size_t per = (units + nblocks - 1) / nblocks;
  const size_t lo = block_linear * per;
  size_t hi = lo + per;
  if (hi > units) hi = units;
  for (size_t u = lo + threadIdx.x; u < hi; u += blockDim.x) p[u] = make_uint4(0, 0, 0, 0);
}

}  // namespace ctopk
