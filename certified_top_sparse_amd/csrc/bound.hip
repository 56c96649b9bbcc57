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
// On the device f is found without sorting the maxima.  Each round tests 64
// candidate thresholds at once: every tile adds its mass |B| e^{M_B - m}
// (fixed point, rounded up, so the sums are exact, order-free and never
// below the real ones) and |B| - 1 to the bucket of the candidates its
// maximum reaches, with LDS integer atomics; one wave's prefix scan over the
// 64 buckets then gives U at every candidate.  Round 0 spreads the
// candidates over [m + log(eps Z / n), m] (U(t) <= n e^{t - m}, so the lower
// end is within the budget, and nothing above m is); later rounds subdivide
// the interval between the largest candidate within the budget and the next
// one over it, 65-fold, until no fp32 value lies between them or six rounds
// are done.  Every threshold taken is one whose U was evaluated and found
// within the budget, so the certificate does not rest on U being monotone in
// floating point.  The count pass settles whole tiles from their (min, max)
// and reads scores only for tiles that straddle f.
#include <cfloat>

#include "kernels.h"

namespace ctopk {
namespace {

constexpr int kBoundThreads = 1024;
constexpr int kBoundWaves = kBoundThreads / kWave;
constexpr int kTilesPerThread = kBoundMaxTiles / kBoundThreads;
constexpr int kCand = kWave;      // candidates per round, one per lane of the deciding wave
constexpr int kRounds = 6;
constexpr int kStraddleUnroll = 8;  // straddling tiles per wave in flight in the count pass
constexpr double kFix = 17592186044416.0;  // 2^44: sum over 2^18 keys of |B| e^{..} * 2^44 < 2^63
static_assert(kBoundMaxTiles % kBoundThreads == 0, "whole tiles per thread");
static_assert(kBoundWaves <= 16, "per-wave results fit one DPP row");
static_assert(static_cast<int64_t>(kBoundMaxTiles) * kScanTile <= (1 << 18), "fixed-point range");

struct BoundShared {
  unsigned long long xb[2][kCand];  // per-bucket fixed-point mass (two sets, alternating rounds)
  uint32_t cb[2][kCand];            // per-bucket sum of |B| - 1
  float cand[kCand];                // this round's candidate thresholds, non-decreasing
  double wd[kBoundWaves];           // per-wave partial results
  uint32_t wi[kBoundWaves];
  float lo, hi;                     // lo: within the budget; hi: smallest candidate over it
  double Ulo;                       // U(lo), fixed-point masses
  unsigned long long Alo;           // fixed-point mass of the tiles wholly below lo
  uint32_t Clo;                     // and their sum of |B| - 1
  int active;                       // another round follows
  int nlist;                        // straddling tiles listed for the count pass
  int list[kBoundMaxTiles];
};

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u & 0xFFFFFFFFu), l));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u >> 32), l));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

__device__ __forceinline__ float readlane_f32(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
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

__device__ __forceinline__ float round_down_f32(double x) {
  float f = static_cast<float>(x);
  if (static_cast<double>(f) > x) f = nextafterf(f, -INFINITY);
  return f;
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
  const int nn = static_cast<int>(n);  // n <= kBoundMaxTiles * kScanTile
  // every tile holds kScanTile keys but the last
  const int last_sz = nn - (nblk - 1) * kScanTile;
  const uint32_t ctot = static_cast<uint32_t>(nn - nblk);  // sum over tiles of |B| - 1

  // This thread's tiles t, t + 1024, ...: (min, max) and mass, loaded together.
  float Nv[kTilesPerThread], Mv[kTilesPerThread], zv[kTilesPerThread];
#pragma unroll
  for (int u = 0; u < kTilesPerThread; ++u) {
    const int b = t + u * kBoundThreads;
    const float2 mm = b < nblk ? bs[b] : make_float2(INFINITY, -INFINITY);
    Nv[u] = mm.x;
    Mv[u] = mm.y;
    zv[u] = b < nblk ? bz[b] : 0.0f;
  }
  if (t < 2 * kCand) {
    sh.xb[t / kCand][t % kCand] = 0ull;
    sh.cb[t / kCand][t % kCand] = 0u;
  }
  if (t == 0) sh.nlist = 0;
  float mloc = -INFINITY;
#pragma unroll
  for (int u = 0; u < kTilesPerThread; ++u) mloc = fmaxf(mloc, Mv[u]);
  const float m = block_max(mloc, sh);
  double zloc = 0.0;
  unsigned long long X[kTilesPerThread];  // ceil(|B| e^{M_B - m} 2^44)
#pragma unroll
  for (int u = 0; u < kTilesPerThread; ++u) {
    const int b = t + u * kBoundThreads;
    X[u] = 0ull;
    if (b < nblk) {
      const double e = exp(static_cast<double>(Mv[u]) - static_cast<double>(m));
      zloc += e * static_cast<double>(zv[u]);
      X[u] = static_cast<unsigned long long>(
          ceil(static_cast<double>(b == nblk - 1 ? last_sz : kScanTile) * e * kFix));
    }
  }
  const double Z = block_sum(zloc, sh);
  const double budget = eps * Z;

  // Round 0's candidates: t_L + j (m - t_L) / 63, the last one m itself.
  const double tl = static_cast<double>(m) + log(budget / static_cast<double>(nn));
  if (wave == 0) sh.cand[lane] = lane == kCand - 1 ? m : round_down_f32(tl + (static_cast<double>(m) - tl) * lane / (kCand - 1));
  __syncthreads();

  float lo = -FLT_MAX, hi = INFINITY;  // U(-FLT_MAX) = 0: no key scores below it
  double Ulo = 0.0;
  // Tiles with M_B < lo lie below every later candidate and tiles with M_B
  // >= hi below none, so only tiles with lo <= M_B < hi are bucketed; the
  // former enter through (Alo, Clo), carried from round to round.
  unsigned long long Alo = 0ull;
  uint32_t Clo = 0u;
  for (int round = 0; round < kRounds; ++round) {
    const int set = round & 1;
    // Bucket of each tile: the number of candidates at or below its maximum
    // (an arithmetic guess, corrected against the candidates themselves).
    const float a0 = round == 0 ? static_cast<float>(tl) : lo;
    const float inv_w = round == 0 ? static_cast<float>((kCand - 1) / (static_cast<double>(m) - tl))
                                   : static_cast<float>((kCand + 1) / (static_cast<double>(hi) - static_cast<double>(lo)));
    const float off = round == 0 ? 1.0f : 0.0f;
#pragma unroll
    for (int u = 0; u < kTilesPerThread; ++u) {
      const int b = t + u * kBoundThreads;
      if (b < nblk && Mv[u] >= lo && Mv[u] < hi) {
        const float M = Mv[u];
        const float g = (M - a0) * inv_w + off;  // a guess only: any value is corrected below
        int j = g > 0.0f ? (g < static_cast<float>(kCand) ? static_cast<int>(g) : kCand) : 0;
        while (j < kCand && sh.cand[j] <= M) ++j;
        while (j > 0 && sh.cand[j - 1] > M) --j;
        if (j < kCand) {  // below every candidate from j on
          atomicAdd(&sh.xb[set][j], X[u]);
          atomicAdd(&sh.cb[set][j], static_cast<uint32_t>((b == nblk - 1 ? last_sz : kScanTile) - 1));
        }
      }
    }
    __syncthreads();
    if (wave == 0) {
      // U at every candidate from the bucket prefix sums; the decision.
      const float cj = sh.cand[lane];
      const unsigned long long xs = Alo + wave_incl_scan_u64_dpp(sh.xb[set][lane]);
      const uint32_t cs = Clo + wave_incl_scan_u32_dpp(sh.cb[set][lane]);
      sh.xb[set][lane] = 0ull;  // this set serves again two rounds on
      sh.cb[set][lane] = 0u;
      const bool valid = round == 0 || (cj > lo && cj < hi);
      const double U = static_cast<double>(xs) * (1.0 / kFix) +
                       static_cast<double>(ctot - cs) * exp(static_cast<double>(cj) - static_cast<double>(m));
      const bool ok = valid && U <= budget;
      const uint64_t okm = __ballot(ok);
      const uint64_t overm = __ballot(valid && !ok);
      float nlo = lo, nhi = hi;
      double nU = Ulo;
      unsigned long long nA = Alo;
      uint32_t nC = Clo;
      const int best = okm ? 63 - __clzll(okm) : -1;
      if (best >= 0) {
        nlo = readlane_f32(cj, best);
        nU = readlane_f64(U, best);
        nA = static_cast<unsigned long long>(__builtin_amdgcn_readlane(static_cast<int>(xs & 0xFFFFFFFFu), best)) & 0xFFFFFFFFull;
        nA |= static_cast<unsigned long long>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(xs >> 32), best))) << 32;
        nC = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(cs), best));
      }
      const uint64_t above = best < 0 ? overm : (best == 63 ? 0ull : overm & (~0ull << (best + 1)));
      if (above) nhi = readlane_f32(cj, __ffsll(static_cast<unsigned long long>(above)) - 1);
      // Next round's candidates: lo + (j + 1) (hi - lo) / 65.
      const bool bounded = nhi < INFINITY;
      const double step = (static_cast<double>(nhi) - static_cast<double>(nlo)) * (1.0 / (kCand + 1));
      const float nc = bounded ? round_down_f32(static_cast<double>(nlo) + step * (lane + 1)) : nlo;
      const bool more = __ballot(bounded && nc > nlo && nc < nhi) != 0ull;
      sh.cand[lane] = nc;
      if (lane == 0) {
        sh.lo = nlo;
        sh.hi = nhi;
        sh.Ulo = nU;
        sh.Alo = nA;
        sh.Clo = nC;
        sh.active = more ? 1 : 0;
      }
    }
    __syncthreads();
    lo = sh.lo;
    hi = sh.hi;
    Ulo = sh.Ulo;
    Alo = sh.Alo;
    Clo = sh.Clo;
    if (!sh.active) break;  // uniform: every thread read the same flag
  }
  const uint32_t kf = ukey(lo);  // f = lo; a key is kept iff ukey(s) >= kf

  // Count and mask: whole tiles from their (min, max); the tiles that
  // straddle f (and a short last tile) listed for a read of their scores.
  const int nwords = (nn + 31) / 32;
  uint32_t* mrow = sel_mask ? sel_mask + static_cast<size_t>(row) * static_cast<size_t>(nwords) : nullptr;
  uint32_t cnt = 0u;
#pragma unroll
  for (int u = 0; u < kTilesPerThread; ++u) {
    const int b = t + u * kBoundThreads;
    if (b < nblk) {
      const bool whole = b < nblk - 1 || last_sz == kScanTile;
      if (whole && ukey(Nv[u]) >= kf) {
        cnt += kScanTile;
        if (mrow != nullptr) {
          mrow[2 * b] = ~0u;
          mrow[2 * b + 1] = ~0u;
        }
      } else if (whole && ukey(Mv[u]) < kf) {
        if (mrow != nullptr) {
          mrow[2 * b] = 0u;
          mrow[2 * b + 1] = 0u;
        }
      } else {
        sh.list[atomicAdd(&sh.nlist, 1)] = b;
      }
    }
  }
  __syncthreads();
  const float* sr = scores + static_cast<size_t>(row) * static_cast<size_t>(n);
  const int nl = sh.nlist;
  uint32_t scnt = 0u;  // kept keys of this wave's straddling tiles (wave-uniform)
  for (int e0 = wave; e0 < nl; e0 += kBoundWaves * kStraddleUnroll) {
    int bl[kStraddleUnroll];
    float v[kStraddleUnroll];
#pragma unroll
    for (int u = 0; u < kStraddleUnroll; ++u) {
      const int e = e0 + u * kBoundWaves;
      bl[u] = e < nl ? sh.list[e] : -1;
      v[u] = sr[min(max(bl[u], 0) * kScanTile + lane, nn - 1)];
    }
#pragma unroll
    for (int u = 0; u < kStraddleUnroll; ++u) {
      if (bl[u] >= 0) {  // wave-uniform
        const int i = bl[u] * kScanTile + lane;
        const uint64_t bits = __ballot(i < nn && ukey(v[u]) >= kf);
        scnt += static_cast<uint32_t>(__popcll(bits));
        if (mrow != nullptr) {
          if (lane == 0) mrow[2 * bl[u]] = static_cast<uint32_t>(bits);
          if (lane == 1 && 2 * bl[u] + 1 < nwords) mrow[2 * bl[u] + 1] = static_cast<uint32_t>(bits >> 32);
        }
      }
    }
  }
  const uint32_t wsum = wave_sum_u32_dpp(cnt + (lane == 0 ? scnt : 0u));
  if (lane == 0) sh.wi[wave] = wsum;
  __syncthreads();

  if (t == 0) {
    int64_t k = 0;
    for (int w2 = 0; w2 < kBoundWaves; ++w2) k += sh.wi[w2];
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
  if (nblk < 1 || nblk > kBoundMaxTiles || n > static_cast<int64_t>(kBoundMaxTiles) * kScanTile)
    return hipErrorInvalidValue;
  return launch(bound_kernel, dim3(rows), dim3(kBoundThreads), 0, st, scores, n, blkstat, blkz,
                nblk, eps, rs, k_eps, tau, lse, sel_mask);
}

}  // namespace ctopk
