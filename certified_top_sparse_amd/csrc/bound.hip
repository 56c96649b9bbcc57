// Blockwise deterministic bound and its certified truncation: the
// "blockwise variants" of the deterministic bounds that control TV from the
// ordered logits (Abstract of "A Mathematical Theory of Top-k Sparse
// Attention via Total Variation Distance", arXiv 2512.07647; the page prints
// no formula, so the bound below is this library's reading).
//
// Blocks are the score scan's tiles of kScanTile keys, with maxima M_B and
// sizes |B|; m = max M_B.  The softmax mass (relative to e^m) of the keys
// scoring below t is at most
//   U(t) = sum_{M_B < t} |B| e^{M_B - m} + sum_{M_B >= t} (|B| - 1) e^{t - m}
// (a block whose maximum is below t lies wholly below t; any other block has
// at most |B| - 1 keys below t, each of weight below e^{t - m}).  U is
// non-decreasing in t and equals A_j + c_j e^{t - m} on the interval
// (M_(j-1), M_(j)] between consecutive sorted maxima (A_j: sum of |B| e^{M_B
// - m} over the j smallest maxima; c_j: sum of |B| - 1 over the others), so
// the largest t with U(t) <= eps Z is min(M_(j), m + log((eps Z - A_j) / c_j))
// for the last interval where that exceeds M_(j-1).  The row keeps every key
// scoring at or above the largest fp32 threshold f with U(f) <= eps Z: TV of
// the truncation <= U(f) / Z <= eps, certified without selecting keys one by
// one.  Z comes from the scan's per-tile masses: Z = sum_B e^{M_B - m} z_B.
//
// On the device f is found without sorting the maxima: U(t) needs one pass
// over the tiles, so each of the 16 waves of the row's workgroup evaluates U
// at its own candidate and a round narrows the interval of fp32 thresholds
// (in the order-preserving key space) 17-fold; eight or nine rounds cover the
// 2^32 keys.  Every candidate taken is one whose U was evaluated and found
// within the budget, so the certificate never rests on U being monotone in
// floating point; monotonicity only makes the answer the largest such f.
// The workgroup is latency-bound (one per row), so reductions use DPP and
// scalar lane reads instead of LDS round trips, the round's decision is two
// ballots, and the count pass keeps 32 score loads per lane in flight.
#include <cfloat>

#include "kernels.h"

namespace ctopk {
namespace {

constexpr int kBoundThreads = 1024;
constexpr int kBoundWaves = kBoundThreads / kWave;
constexpr int kTilesPerThread = kBoundMaxTiles / kBoundThreads;
constexpr int kCountUnroll = 32;  // score loads in flight per lane in the count pass
static_assert(kBoundMaxTiles % kBoundThreads == 0, "whole tiles per thread");
static_assert(kBoundWaves <= 16, "per-wave results fit one DPP row");

struct BoundShared {
  float2 Mx[kBoundMaxTiles];  // (M_B, |B| e^{M_B - m}) per tile
  double wd[kBoundWaves];     // per-wave partial results
  double U[kBoundWaves];      // U at each wave's candidate
  int feas[kBoundWaves];      // 1: within the budget, 0: not, -1: no candidate
};

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(u & 0xFFFFFFFFu), CTRL, 0xF, 0xF, false));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(u >> 32), CTRL, 0xF, 0xF, false));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u & 0xFFFFFFFFu), l));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u >> 32), l));
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

// Sum over the 64 lanes in a fixed tree, the same value in every lane.
__device__ __forceinline__ double wave_sum_f64(double v) {
  v = row_sum_f64(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
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

// Workgroup sum in a fixed order (each wave's sum, then the per-wave sums
// across the lanes of one DPP row), the same value in every thread.
__device__ double block_sum(double v, BoundShared& sh) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  v = wave_sum_f64(v);
  __syncthreads();
  if (lane == 0) sh.wd[wave] = v;
  __syncthreads();
  const double p = row_sum_f64(lane < kBoundWaves ? sh.wd[lane] : 0.0);
  return readlane_f64(p, 0);
}

__device__ float block_max(float v, BoundShared& sh) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  v = wave_max_dpp(v);
  __syncthreads();
  if (lane == 0) sh.wd[wave] = v;
  __syncthreads();
  return wave_max_dpp(lane < kBoundWaves ? static_cast<float>(sh.wd[lane]) : -INFINITY);
}

__global__ __launch_bounds__(kBoundThreads) void bound_kernel(
    const float* __restrict__ scores, int64_t n, const float2* __restrict__ blkstat,
    const float* __restrict__ blkz, int nblk, double eps, RowSel* __restrict__ rs,
    int32_t* __restrict__ k_eps, double* __restrict__ tau, double* __restrict__ lse,
    uint32_t* __restrict__ sel_mask) {
  __shared__ BoundShared sh;
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = t / kWave;
  const float2* bs = blkstat + static_cast<size_t>(row) * nblk;
  const float* bz = blkz + static_cast<size_t>(row) * nblk;
  // every tile holds kScanTile keys but the last
  const int last_sz = static_cast<int>(n - static_cast<int64_t>(nblk - 1) * kScanTile);

  // Tiles: maxima and masses loaded together; the row maximum m, Z, and
  // (M_B, |B| e^{M_B - m}) staged in LDS.
  float Mv[kTilesPerThread], zv[kTilesPerThread];
#pragma unroll
  for (int u = 0; u < kTilesPerThread; ++u) {
    const int b = t + u * kBoundThreads;
    Mv[u] = b < nblk ? bs[b].y : -INFINITY;
    zv[u] = b < nblk ? bz[b] : 0.0f;
  }
  float mloc = -INFINITY;
#pragma unroll
  for (int u = 0; u < kTilesPerThread; ++u) mloc = fmaxf(mloc, Mv[u]);
  const float m = block_max(mloc, sh);
  double zloc = 0.0;
#pragma unroll
  for (int u = 0; u < kTilesPerThread; ++u) {
    const int b = t + u * kBoundThreads;
    if (b < nblk) {
      const double e = exp(static_cast<double>(Mv[u]) - static_cast<double>(m));
      zloc += e * static_cast<double>(zv[u]);
      sh.Mx[b] = make_float2(Mv[u], static_cast<float>(static_cast<double>(b == nblk - 1 ? last_sz : kScanTile) * e));
    }
  }
  const double Z = block_sum(zloc, sh);  // its barriers also publish sh.Mx
  const double budget = eps * Z;

  // Search over fp32 thresholds in key space.  klo is always a threshold
  // within the budget (U(-FLT_MAX) = 0: no key scores below it), and the
  // answer is at most ukey(m) (above m, U is at least Z).
  uint32_t klo = ukey(-FLT_MAX), khi = ukey(m);
  double Ulo = 0.0;
  for (int round = 0; round < 16 && khi != klo; ++round) {
    const uint32_t span = khi - klo;
    const bool fine = span <= static_cast<uint32_t>(kBoundWaves);
    auto cand = [&](int w) -> uint32_t {  // candidate w, strictly above klo, at most khi
      return fine ? klo + static_cast<uint32_t>(w) + 1u
                  : klo + static_cast<uint32_t>((static_cast<uint64_t>(span) * (w + 1)) /
                                                (kBoundWaves + 1));
    };
    const uint32_t cw = cand(wave);
    if (cw <= khi) {
      const float tc = ukey_to_float(cw);
      double a = 0.0;   // sum of |B| e^{M_B - m} over tiles wholly below tc
      uint32_t c = 0u;  // sum of |B| - 1 over the others
      for (int b0 = 0; b0 < nblk; b0 += 4 * kWave) {
        float2 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int b = b0 + u * kWave + lane;
          v[u] = b < nblk ? sh.Mx[b] : make_float2(-INFINITY, 0.0f);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int b = b0 + u * kWave + lane;
          const bool below = v[u].x < tc;
          a += below ? static_cast<double>(v[u].y) : 0.0;
          c += (below || b >= nblk) ? 0u : static_cast<uint32_t>((b == nblk - 1 ? last_sz : kScanTile) - 1);
        }
      }
      a = wave_sum_f64(a);
      c = wave_sum_u32_dpp(c);
      const double U = a + static_cast<double>(c) * exp(static_cast<double>(tc) - static_cast<double>(m));
      if (lane == 0) {
        sh.U[wave] = U;
        sh.feas[wave] = U <= budget ? 1 : 0;
      }
    } else if (lane == 0) {
      sh.feas[wave] = -1;
    }
    __syncthreads();
    // Every thread takes the same decision from the same LDS values: the
    // largest candidate within the budget becomes klo, the first one above
    // it that is not bounds khi.
    const int fl = lane < kBoundWaves ? sh.feas[lane] : -1;
    const uint64_t ok = __ballot(fl == 1);
    const uint64_t over = __ballot(fl == 0);
    const int best = ok ? 63 - __clzll(ok) : -1;
    if (best >= 0) {
      Ulo = sh.U[best];
    }
    const uint64_t above = best >= 0 ? (best >= 63 ? 0ull : (over >> (best + 1)) << (best + 1)) : over;
    const uint32_t nhi = above ? cand(__ffsll(static_cast<unsigned long long>(above)) - 1) - 1u : khi;
    if (best >= 0) klo = cand(best);
    khi = nhi;
    __syncthreads();  // sh.feas and sh.U are rewritten next round
  }
  const uint32_t kf = klo;  // the key of f

  // Keep every key whose key order is at or above f's (the value stream's
  // test): count them and write the mask, kCountUnroll loads per lane in
  // flight; wave w takes 64-key groups w, w + 16, ...
  // n <= kBoundMaxTiles * kScanTile, so key and word indices fit in int.
  const float* sr = scores + static_cast<size_t>(row) * static_cast<size_t>(n);
  const int nn = static_cast<int>(n);
  const int nwords = (nn + 31) / 32;
  uint32_t* mrow = sel_mask ? sel_mask + static_cast<size_t>(row) * static_cast<size_t>(nwords) : nullptr;
  const int ngroups = (nn + kWave - 1) / kWave;
  uint32_t cnt = 0u;
  for (int g0 = wave; g0 < ngroups; g0 += kBoundWaves * kCountUnroll) {
    float v[kCountUnroll];
#pragma unroll
    for (int u = 0; u < kCountUnroll; ++u) v[u] = sr[min((g0 + u * kBoundWaves) * kWave + lane, nn - 1)];
#pragma unroll
    for (int u = 0; u < kCountUnroll; ++u) {
      const int g = g0 + u * kBoundWaves;
      const bool kept = g * kWave + lane < nn && ukey(v[u]) >= kf;
      const uint64_t bits = __ballot(kept);
      cnt += static_cast<uint32_t>(__popcll(bits));
      if (mrow != nullptr && g < ngroups) {
        if (lane == 0) mrow[2 * g] = static_cast<uint32_t>(bits);
        if (lane == 1 && 2 * g + 1 < nwords) mrow[2 * g + 1] = static_cast<uint32_t>(bits >> 32);
      }
    }
  }
  if (lane == 0) sh.feas[wave] = static_cast<int>(cnt);  // the search's last barrier preceded this
  __syncthreads();

  if (t == 0) {
    int64_t k = 0;
    for (int w = 0; w < kBoundWaves; ++w) k += sh.feas[w];
    rs[row].m = m;
    rs[row].lo = m;
    rs[row].Z = Z;
    rs[row].thr = static_cast<uint64_t>(kf) << 32;  // key64 >= this iff ukey(s) >= ukey(f)
    k_eps[row] = static_cast<int32_t>(k);
    tau[row] = Ulo / Z;
    if (lse) lse[row] = static_cast<double>(m) + log(Z);
  }
}

}  // namespace

hipError_t launch_bound(const float* scores, int64_t n, int rows, const float2* blkstat,
                        const float* blkz, int nblk, double eps, RowSel* rs, int32_t* k_eps,
                        double* tau, double* lse, uint32_t* sel_mask, hipStream_t st) {
  if (nblk < 1 || nblk > kBoundMaxTiles) return hipErrorInvalidValue;
  return launch(bound_kernel, dim3(rows), dim3(kBoundThreads), 0, st, scores, n, blkstat, blkz,
                nblk, eps, rs, k_eps, tau, lse, sel_mask);
}

}  // namespace ctopk
