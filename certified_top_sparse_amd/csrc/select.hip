// Global log-sum-exp and the mass-weighted radix select.
//
// For one row of scores the select finds the cut key e: the largest key (in
// the key64 order of device_common.h) whose strictly-lower keys carry softmax
// mass <= eps * Z.  Then the head is { x : key64(x) >= key64(e) }, its size is
// the minimal k with discarded tail mass <= eps, and that tail mass is tau
// (Abstract of "A Mathematical Theory of Top-k Sparse Attention via Total
// Variation Distance", arXiv 2512.07647: TV(P, P_hat) equals the discarded
// tail mass and k_eps is the smallest k meeting the budget).
//
// The search runs digit by digit from the top of key64 (5 x 11 + 9 bits):
//   level 0  (hist0, many blocks per row): weights w = exp(s - m) with the row
//            maximum m, LDS histogram of (count, fp64 mass) per top digit,
//            merged across blocks with global atomics;
//   level >0 (resolve, one block per row): pick the cut bin b*, the largest
//            non-empty bin whose lower bins hold mass <= eps*Z - R (R = mass
//            already known to lie below), then histogram the next digit of the
//            keys inside b*.  Once b* holds <= kCandCap keys they are copied
//            into LDS and all further levels run there.  The search ends when
//            one key is left; since key64 is unique this takes <= 6 levels.
// Counts are exact integers, so k_eps is exact given the weights; masses are
// fp64 sums of fp32 weights.  tau = R / Z uses the same weights as Z.
#include "kernels.h"

namespace ctopk {
namespace {

constexpr int kRowMaxChunk = 4096;

// Row maxima of given logits, one value per kRowMaxChunk keys.
// grid = rows * nblk blocks, block b covers chunk b % nblk of row b / nblk.
__global__ __launch_bounds__(256) void rowmax_kernel(const float* __restrict__ x, int64_t n,
                                                     int nblk, float* __restrict__ blkmax,
                                                     void* zero_base, size_t zero_bytes) {
  __shared__ float s_red[4];
  zero_slice(zero_base, zero_bytes, blockIdx.x, gridDim.x);
  const int row = static_cast<int>(blockIdx.x / static_cast<unsigned>(nblk));
  const int cb = static_cast<int>(blockIdx.x % static_cast<unsigned>(nblk));
  const int64_t lo = static_cast<int64_t>(cb) * kRowMaxChunk;
  const int64_t hi = min(n, lo + kRowMaxChunk);
  const float* xr = x + static_cast<size_t>(row) * static_cast<size_t>(n);
  float v = -INFINITY;
  for (int64_t i = lo + threadIdx.x; i < hi; i += blockDim.x) v = fmaxf(v, xr[i]);
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    v = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    blkmax[static_cast<size_t>(row) * nblk + cb] = v;
  }
}

// Level 0 of the select.  grid = rows * nchunk blocks; block b covers chunk
// b % nchunk of row b / nchunk.
__global__ __launch_bounds__(256) void hist0_kernel(const float* __restrict__ scores, int64_t n,
                                                    int64_t chunk, int nchunk,
                                                    const float* __restrict__ blkmax, int nblk,
                                                    RowSel* __restrict__ rs,
                                                    uint32_t* __restrict__ hcnt,
                                                    double* __restrict__ hmass) {
  __shared__ uint32_t lc[kBins];
  __shared__ double lm[kBins];
  __shared__ float s_red[4];
  const int row = static_cast<int>(blockIdx.x / static_cast<unsigned>(nchunk));
  const int cb = static_cast<int>(blockIdx.x % static_cast<unsigned>(nchunk));
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  // Global maximum of the row from the per-tile maxima (wavefront reduction).
  float mx = -INFINITY;
  const float* bm = blkmax + static_cast<size_t>(row) * nblk;
  for (int b = threadIdx.x; b < nblk; b += blockDim.x) mx = fmaxf(mx, bm[b]);
  mx = wave_max(mx);
  if (lane == 0) s_red[wave] = mx;
  for (int b = threadIdx.x; b < kBins; b += blockDim.x) {
    lc[b] = 0u;
    lm[b] = 0.0;
  }
  __syncthreads();
  const float m = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  if (cb == 0 && threadIdx.x == 0) rs[row].m = m;

  const float* sr = scores + static_cast<size_t>(row) * static_cast<size_t>(n);
  const int64_t lo = static_cast<int64_t>(cb) * chunk;
  const int64_t hi = min(n, lo + chunk);
  for (int64_t i = lo + threadIdx.x; i < hi; i += blockDim.x) {
    const float s = sr[i];
    const uint32_t bin = ukey(s) >> (32 - kDigitBits);
    atomicAdd(&lc[bin], 1u);
    atomicAdd(&lm[bin], static_cast<double>(weight(s, m)));
  }
  __syncthreads();
  uint32_t* gc = hcnt + static_cast<size_t>(row) * kBins;
  double* gm = hmass + static_cast<size_t>(row) * kBins;
  for (int b = threadIdx.x; b < kBins; b += blockDim.x) {
    if (lc[b] != 0u) {
      atomicAdd(&gc[b], lc[b]);
      atomicAdd(&gm[b], lm[b]);
    }
  }
}

constexpr int kResolveThreads = 1024;
constexpr int kResolveWaves = kResolveThreads / 64;

struct ResolveShared {
  uint32_t hc[kBins];
  double hm[kBins];
  uint64_t cand[kCandCap];
  double wd[kResolveWaves];
  uint32_t wc[kResolveWaves];
  int best;
  uint32_t ncand;
  double selS;
  uint32_t selC;
  uint64_t thr;
};

// Block-wide choice of the cut bin among nb bins held in sh.hc / sh.hm.
// Returns b* and, through S and C, the mass and count of the bins below it.
__device__ int select_bin(ResolveShared& sh, int nb, double R, double epsZ, double& S,
                          uint32_t& C) {
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int b0 = 2 * t;
  const uint32_t c0 = b0 < nb ? sh.hc[b0] : 0u;
  const uint32_t c1 = b0 + 1 < nb ? sh.hc[b0 + 1] : 0u;
  const double m0 = b0 < nb ? sh.hm[b0] : 0.0;
  const double m1 = b0 + 1 < nb ? sh.hm[b0 + 1] : 0.0;
  const double tm = m0 + m1;
  const uint32_t tc = c0 + c1;
  const double im = wave_incl_scan(tm, lane);
  const uint32_t ic = wave_incl_scan_u32(tc, lane);
  if (lane == 63) {
    sh.wd[wave] = im;
    sh.wc[wave] = ic;
  }
  if (t == 0) sh.best = -1;
  __syncthreads();
  double off = 0.0;
  uint32_t offc = 0u;
  for (int w = 0; w < wave; ++w) {
    off += sh.wd[w];
    offc += sh.wc[w];
  }
  double em = __shfl_up(im, 1, 64);
  uint32_t ec = __shfl_up(ic, 1, 64);
  if (lane == 0) {
    em = 0.0;
    ec = 0u;
  }
  const double ex0 = off + em;
  const uint32_t exc0 = offc + ec;
  const double ex1 = ex0 + m0;
  int mine = -1;
  if (c0 != 0u && R + ex0 <= epsZ) mine = b0;
  if (c1 != 0u && R + ex1 <= epsZ) mine = b0 + 1;
  if (mine >= 0) atomicMax(&sh.best, mine);
  __syncthreads();
  const int bs = sh.best;
  if (bs >= 0 && (bs >> 1) == t) {
    if (bs == b0) {
      sh.selS = ex0;
      sh.selC = exc0;
    } else {
      sh.selS = ex1;
      sh.selC = exc0 + c0;
    }
  }
  __syncthreads();
  S = sh.selS;
  C = sh.selC;
  return bs;
}

__device__ __forceinline__ bool prefix_match(uint64_t k, uint64_t prefix, int plen) {
  return plen == 0 ? true : (plen >= 64 ? k == prefix : (k >> (64 - plen)) == prefix);
}

__global__ __launch_bounds__(kResolveThreads) void resolve_kernel(
    const float* __restrict__ scores, int64_t n, const uint32_t* __restrict__ hcnt0,
    const double* __restrict__ hmass0, double eps, RowSel* __restrict__ rs,
    int32_t* __restrict__ k_eps, double* __restrict__ tau, double* __restrict__ lse) {
  __shared__ ResolveShared sh;
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const float* sr = scores + static_cast<size_t>(row) * static_cast<size_t>(n);
  const float m = rs[row].m;

  for (int b = t; b < kBins; b += kResolveThreads) {
    sh.hc[b] = hcnt0[static_cast<size_t>(row) * kBins + b];
    sh.hm[b] = hmass0[static_cast<size_t>(row) * kBins + b];
  }
  if (t == 0) sh.ncand = 0u;
  __syncthreads();

  // Z = total weight, summed in a fixed order (pairs, wave tree, waves in order).
  double z = sh.hm[2 * t] + sh.hm[2 * t + 1];
  z = wave_sum(z);
  if (lane == 0) sh.wd[wave] = z;
  __syncthreads();
  double Z = 0.0;
  for (int w = 0; w < kResolveWaves; ++w) Z += sh.wd[w];
  __syncthreads();
  const double epsZ = eps * Z;

  uint64_t prefix = 0;
  int plen = 0;
  double R = 0.0;
  uint64_t below = 0;
  uint32_t cnt_in = 0;
  bool in_lds = false;
  uint32_t ncand = 0;

  for (int level = 0; level < kLevels; ++level) {
    const int wdt = digit_width(level);
    const int nb = 1 << wdt;
    if (level > 0) {
      for (int b = t; b < kBins; b += kResolveThreads) {
        sh.hc[b] = 0u;
        sh.hm[b] = 0.0;
      }
      __syncthreads();
      const int shift = 64 - plen - wdt;
      if (in_lds) {
        for (uint32_t c = t; c < ncand; c += kResolveThreads) {
          const uint64_t k = sh.cand[c];
          if (prefix_match(k, prefix, plen)) {
            const int b = static_cast<int>((k >> shift) & static_cast<uint64_t>(nb - 1));
            atomicAdd(&sh.hc[b], 1u);
            atomicAdd(&sh.hm[b], static_cast<double>(weight(key64_score(k), m)));
          }
        }
      } else {
        for (int64_t i = t; i < n; i += kResolveThreads) {
          const float s = sr[i];
          const uint64_t k = key64(s, static_cast<uint32_t>(i));
          if (prefix_match(k, prefix, plen)) {
            const int b = static_cast<int>((k >> shift) & static_cast<uint64_t>(nb - 1));
            atomicAdd(&sh.hc[b], 1u);
            atomicAdd(&sh.hm[b], static_cast<double>(weight(s, m)));
          }
        }
      }
      __syncthreads();
    }
    double S;
    uint32_t C;
    int bs = select_bin(sh, nb, R, epsZ, S, C);
    if (bs < 0) {  // only with non-finite scores (unspecified results)
      bs = 0;
      S = 0.0;
      C = 0u;
    }
    cnt_in = sh.hc[bs];
    R += S;
    below += C;
    prefix = (prefix << wdt) | static_cast<uint64_t>(bs);
    plen += wdt;
    __syncthreads();
    if (!in_lds && (cnt_in <= kCandCap || cnt_in == 1u)) {
      // Copy the keys of the cut bin into LDS (exactly cnt_in of them match).
      for (int64_t i = t; i < n; i += kResolveThreads) {
        const float s = sr[i];
        const uint64_t k = key64(s, static_cast<uint32_t>(i));
        if (prefix_match(k, prefix, plen)) {
          const uint32_t slot = atomicAdd(&sh.ncand, 1u);
          if (slot < kCandCap) sh.cand[slot] = k;
        }
      }
      __syncthreads();
      ncand = min(sh.ncand, static_cast<uint32_t>(kCandCap));
      in_lds = true;
    }
    if (cnt_in <= 1u || plen >= 64) break;
  }

  // The cut key is the one candidate matching the full prefix.
  if (t == 0) sh.thr = prefix;
  __syncthreads();
  if (plen < 64) {
    for (uint32_t c = t; c < ncand; c += kResolveThreads) {
      const uint64_t k = sh.cand[c];
      if (prefix_match(k, prefix, plen)) sh.thr = k;
    }
  }
  __syncthreads();
  if (t == 0) {
    const uint64_t thr = sh.thr;
    rs[row].Z = Z;
    rs[row].thr = thr;
    k_eps[row] = static_cast<int32_t>(static_cast<uint64_t>(n) - below);
    tau[row] = R / Z;
    if (lse) lse[row] = static_cast<double>(m) + log(Z);
  }
}

}  // namespace

hipError_t launch_rowmax(const float* logits, int64_t n, int rows, float* blkmax,
                         void* zero_base, size_t zero_bytes, hipStream_t st) {
  const int nblk = static_cast<int>(ceil_div(n, kRowMaxChunk));
  hipLaunchKernelGGL(rowmax_kernel, dim3(static_cast<unsigned>(nblk) * rows), dim3(256), 0, st,
                     logits, n, nblk, blkmax, zero_base, zero_bytes);
  return hipGetLastError();
}

int rowmax_nblk(int64_t n) { return static_cast<int>(ceil_div(n, kRowMaxChunk)); }

hipError_t launch_hist0(const float* scores, int64_t n, int rows, const float* blkmax, int nblk,
                        RowSel* rs, uint32_t* hcnt, double* hmass, hipStream_t st) {
  // Aim for a few thousand blocks in total: enough to fill 256 CUs while
  // keeping the number of global histogram merges small.
  const int64_t total = n * static_cast<int64_t>(rows);
  int64_t chunk = ceil_div(total, 4096);
  chunk = ceil_div(chunk, 4096) * 4096;
  if (chunk < kHistChunk) chunk = kHistChunk;
  if (chunk > n) chunk = n;
  const int nchunk = static_cast<int>(ceil_div(n, chunk));
  hipLaunchKernelGGL(hist0_kernel, dim3(static_cast<unsigned>(nchunk) * rows), dim3(256), 0, st,
                     scores, n, chunk, nchunk, blkmax, nblk, rs, hcnt, hmass);
  return hipGetLastError();
}

hipError_t launch_resolve(const float* scores, int64_t n, int rows, const uint32_t* hcnt,
                          const double* hmass, double eps, RowSel* rs, int32_t* k_eps,
                          double* tau, double* lse, hipStream_t st) {
  hipLaunchKernelGGL(resolve_kernel, dim3(rows), dim3(kResolveThreads), 0, st, scores, n, hcnt,
                     hmass, eps, rs, k_eps, tau, lse);
  return hipGetLastError();
}

}  // namespace ctopk
