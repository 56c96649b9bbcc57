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
// scoring at or above that threshold (rounded down to fp32, where U is
// recomputed from its definition): TV of the truncation <= U / Z <= eps,
// certified without selecting keys one by one.  Z comes from the scan's
// per-tile masses: Z = sum_B e^{M_B - m} z_B.
#include "kernels.h"

namespace ctopk {
namespace {

constexpr int kBoundThreads = 1024;
constexpr int kBoundWaves = kBoundThreads / kWave;
constexpr int kPerThread = kBoundMaxTiles / kBoundThreads;
static_assert(kBoundMaxTiles % kBoundThreads == 0, "whole tiles per thread");

struct BoundShared {
  float M[kBoundMaxTiles];  // tile maxima, sorted ascending (padding: +inf)
  int sz[kBoundMaxTiles];   // their sizes (padding: 0)
  double wd[kBoundWaves];   // per-wave partial results
  int wi[kBoundWaves];
};

// Workgroup reductions in a fixed order (wave butterflies, then waves in
// order), so every thread gets the same value on every run.
__device__ double block_sum(double v, BoundShared& sh) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) sh.wd[wave] = v;
  __syncthreads();
  double s = 0.0;
  for (int w = 0; w < kBoundWaves; ++w) s += sh.wd[w];
  return s;
}

__device__ double block_max(double v, BoundShared& sh) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o, kWave));
  __syncthreads();
  if (lane == 0) sh.wd[wave] = v;
  __syncthreads();
  double s = sh.wd[0];
  for (int w = 1; w < kBoundWaves; ++w) s = fmax(s, sh.wd[w]);
  return s;
}

// Exclusive prefix sums over [0, kBoundMaxTiles) of x (double) and y (int),
// thread t holding entries kPerThread * t + u.
__device__ void block_scan(double (&x)[kPerThread], int (&y)[kPerThread], BoundShared& sh) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  double xs = 0.0;
  int ys = 0;
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    xs += x[u];
    ys += y[u];
  }
  const double xi = wave_incl_scan(xs, lane);
  const uint32_t yi = wave_incl_scan_u32(static_cast<uint32_t>(ys), lane);
  __syncthreads();
  if (lane == kWave - 1) {
    sh.wd[wave] = xi;
    sh.wi[wave] = static_cast<int>(yi);
  }
  __syncthreads();
  double xb = 0.0;
  int yb = 0;
  for (int w = 0; w < wave; ++w) {
    xb += sh.wd[w];
    yb += sh.wi[w];
  }
  double xr = xb + xi - xs;  // exclusive prefix of this thread's first entry
  int yr = yb + static_cast<int>(yi) - ys;
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    const double xv = x[u];
    const int yv = y[u];
    x[u] = xr;
    y[u] = yr;
    xr += xv;
    yr += yv;
  }
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

  // Tiles: maxima, sizes and masses; the row maximum m and Z.
  float Mv[kPerThread], zv[kPerThread];
  int sv[kPerThread];
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    const int b = kPerThread * t + u;
    const bool real = b < nblk;
    Mv[u] = real ? bs[b].y : INFINITY;
    zv[u] = real ? bz[b] : 0.0f;
    sv[u] = real ? static_cast<int>(min(static_cast<int64_t>(kScanTile), n - static_cast<int64_t>(b) * kScanTile)) : 0;
  }
  double mloc = -INFINITY;
#pragma unroll
  for (int u = 0; u < kPerThread; ++u)
    if (sv[u] > 0) mloc = fmax(mloc, static_cast<double>(Mv[u]));
  const float m = static_cast<float>(block_max(mloc, sh));
  double zloc = 0.0;
#pragma unroll
  for (int u = 0; u < kPerThread; ++u)
    if (sv[u] > 0) zloc += exp(static_cast<double>(Mv[u]) - m) * static_cast<double>(zv[u]);
  const double Z = block_sum(zloc, sh);
  const double budget = eps * Z;

  // Sort the tiles by maximum (bitonic, in LDS).
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    sh.M[kPerThread * t + u] = Mv[u];
    sh.sz[kPerThread * t + u] = sv[u];
  }
  int P = 1;
  while (P < nblk) P <<= 1;
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      __syncthreads();
      for (int i = t; i < P; i += kBoundThreads) {
        const int l = i ^ j;
        if (l > i) {
          const bool up = (i & k) == 0;
          const float a = sh.M[i], c = sh.M[l];
          if ((a > c) == up) {
            sh.M[i] = c;
            sh.M[l] = a;
            const int s = sh.sz[i];
            sh.sz[i] = sh.sz[l];
            sh.sz[l] = s;
          }
        }
      }
    }
  }
  __syncthreads();

  // A_j and c_j over the sorted tiles.
  double x[kPerThread];
  int y[kPerThread];
  int ctot = 0;
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    const int j = kPerThread * t + u;
    const int s = sh.sz[j];
    x[u] = s > 0 ? static_cast<double>(s) * exp(static_cast<double>(sh.M[j]) - m) : 0.0;
    y[u] = s > 0 ? s - 1 : 0;
  }
  block_scan(x, y, sh);
  // total sum of |B| - 1: the prefix past the last entry
  {
    int last = 0;
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int j = kPerThread * t + u;
      if (j == kBoundMaxTiles - 1) last = y[u] + (sh.sz[j] > 0 ? sh.sz[j] - 1 : 0);
    }
    __syncthreads();  // every thread has read the scan's wave totals
    if (t == kBoundThreads - 1) sh.wi[0] = last;
    __syncthreads();
    ctot = sh.wi[0];
    __syncthreads();
  }

  // The largest feasible threshold of each interval; the best over all.
  double best = -INFINITY;
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    const int j = kPerThread * t + u;
    if (j >= nblk) continue;
    const double lo = j > 0 ? static_cast<double>(sh.M[j - 1]) : -INFINITY;
    const double Aj = x[u];
    const double cj = static_cast<double>(ctot - y[u]);
    if (Aj > budget) continue;
    double tj;
    if (cj > 0.0) {
      const double room = budget - Aj;
      tj = room > 0.0 ? fmin(static_cast<double>(sh.M[j]), static_cast<double>(m) + log(room / cj))
                      : -INFINITY;
    } else {
      tj = static_cast<double>(sh.M[j]);
    }
    if (tj > lo) best = fmax(best, tj);
  }
  const double tstar = block_max(best, sh);

  // The fp32 threshold at or below t*, and U recomputed there from its
  // definition (U is non-decreasing, so U(f) <= U(t*) <= eps Z).
  float f = static_cast<float>(tstar);
  if (static_cast<double>(f) > tstar) f = nextafterf(f, -INFINITY);
  double uloc = 0.0;
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    const int j = kPerThread * t + u;
    const int s = sh.sz[j];
    if (s == 0) continue;
    const float Mj = sh.M[j];
    uloc += Mj < f ? static_cast<double>(s) * exp(static_cast<double>(Mj) - m)
                   : static_cast<double>(s - 1) * exp(static_cast<double>(f) - m);
  }
  const double U = block_sum(uloc, sh);

  // Keep every key scoring at or above f: count them (and write the mask).
  const float* sr = scores + static_cast<size_t>(row) * static_cast<size_t>(n);
  const int64_t nwords = ceil_div(n, 32);
  uint32_t* mrow = sel_mask ? sel_mask + static_cast<size_t>(row) * static_cast<size_t>(nwords) : nullptr;
  uint32_t cnt = 0u;
  for (int64_t base = static_cast<int64_t>(wave) * kWave; base < n;
       base += static_cast<int64_t>(kBoundWaves) * kWave) {
    const int64_t i = base + lane;
    const bool kept = i < n && ukey(sr[min(i, n - 1)]) >= ukey(f);  // the value stream's test
    const uint64_t bits = __ballot(kept);
    cnt += kept ? 1u : 0u;
    if (mrow != nullptr) {
      if (lane == 0) mrow[base / 32] = static_cast<uint32_t>(bits);
      if (lane == 1 && base / 32 + 1 < nwords) mrow[base / 32 + 1] = static_cast<uint32_t>(bits >> 32);
    }
  }
  const double k = block_sum(static_cast<double>(cnt), sh);

  if (t == 0) {
    rs[row].m = m;
    rs[row].lo = m;
    rs[row].Z = Z;
    rs[row].thr = static_cast<uint64_t>(ukey(f)) << 32;  // key64 >= this iff s >= f
    k_eps[row] = static_cast<int32_t>(k);
    tau[row] = U / Z;
    if (lse) lse[row] = static_cast<double>(m) + log(Z);
  }
}

}  // namespace

hipError_t launch_bound(const float* scores, int64_t n, int rows, const float2* blkstat,
                        const float* blkz, int nblk, double eps, RowSel* rs, int32_t* k_eps,
                        double* tau, double* lse, uint32_t* sel_mask, hipStream_t st) {
  if (nblk > kBoundMaxTiles) return hipErrorInvalidValue;
  return launch(bound_kernel, dim3(rows), dim3(kBoundThreads), 0, st, scores, n, blkstat, blkz,
                nblk, eps, rs, k_eps, tau, lse, sel_mask);
}

}  // namespace ctopk
