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
// The search narrows a range of the key order that contains e, level by level,
// keeping R = mass and `below` = count of keys under the range:
//   level 0: row maximum m (the log-sum-exp reference) and minimum, from the
//            score scan's per-tile pairs or from a pass over given logits;
//            weights w = exp(s - m); (count, fp64 mass) per kBins equal-width
//            value bins on [min, max] -- built by many blocks per row
//            (hist0_kernel, per-chunk partial histograms, no atomics across
//            blocks) or inside the row's own block; Z = the bins' sum in a
//            fixed order; lse = m + log Z;
//   level >0 (resolve_kernel, one block per row): pick the cut bin b*, the
//            largest non-empty bin whose lower bins hold mass <= eps*Z - R;
//            then histogram the next 11 bits of key64 inside b*.  Once the
//            range holds <= kCandCap keys they are copied into LDS and the
//            radix continues from the first bit where they differ; once it
//            holds <= 64 keys one wave finishes by comparing every pair.  key64
//            is unique, so the search always ends on one key.
// Counts are exact integers, so k_eps is exact given the weights; masses are
// fp64 sums of fp32 weights.  tau = R / Z uses the same weights as Z.
#include "kernels.h"

namespace ctopk {
namespace {

constexpr int kResolveThreads = 1024;
constexpr int kResolveWaves = kResolveThreads / 64;
// Row scans keep kReadBatch loads in flight per thread.
constexpr int kReadBatch = 16;
// Candidate sets this small are finished by one wave.
constexpr int kSmallCand = 64;

// Row (min, max) from per-tile pairs, reduced identically by every block.
__device__ float2 row_minmax(const float2* __restrict__ bs, int nblk, float2* s_red) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  float vmax = -INFINITY, vmin = INFINITY;
  for (int b = threadIdx.x; b < nblk; b += blockDim.x) {
    const float2 v = bs[b];
    vmin = fminf(vmin, v.x);
    vmax = fmaxf(vmax, v.y);
  }
  vmax = wave_max_dpp(vmax);
  vmin = -wave_max_dpp(-vmin);
  if (lane == 0) s_red[wave] = make_float2(vmin, vmax);
  __syncthreads();
  float2 r = s_red[0];
  for (int w = 1; w < nwaves; ++w) {
    r.x = fminf(r.x, s_red[w].x);
    r.y = fmaxf(r.y, s_red[w].y);
  }
  return r;
}

// Level 0 for the decode path.  grid = rows * nchunk blocks; block b covers
// chunk b % nchunk of row b / nchunk and writes its own partial histogram.
__global__ __launch_bounds__(256) void hist0_kernel(const float* __restrict__ scores, int64_t n,
                                                    int64_t chunk, int nchunk,
                                                    const float2* __restrict__ blkstat, int nblk,
                                                    uint32_t* __restrict__ pcnt,
                                                    double* __restrict__ pmass) {
  __shared__ uint32_t lc[kBins];
  __shared__ double lm[kBins];
  __shared__ float2 s_red[4];
  const int row = static_cast<int>(blockIdx.x / static_cast<unsigned>(nchunk));
  const int cb = static_cast<int>(blockIdx.x % static_cast<unsigned>(nchunk));
  for (int b = threadIdx.x; b < kBins; b += blockDim.x) {
    lc[b] = 0u;
    lm[b] = 0.0;
  }
  const float2 mm = row_minmax(blkstat + static_cast<size_t>(row) * nblk, nblk, s_red);
  const float lo = mm.x;
  const float m = mm.y;
  const float inv = lin_scale(lo, m);

  const float* sr = scores + static_cast<size_t>(row) * static_cast<size_t>(n);
  const int64_t c0 = static_cast<int64_t>(cb) * chunk;
  const int64_t c1 = min(n, c0 + chunk);
  constexpr int U = 8;
  for (int64_t base = c0; base < c1; base += U * 256) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = sr[min(base + u * 256 + threadIdx.x, c1 - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (base + u * 256 + threadIdx.x < c1) {
        const int bin = lin_bin(v[u], lo, inv);
        atomicAdd(&lc[bin], 1u);
        atomicAdd(&lm[bin], static_cast<double>(weight(v[u], m)));
      }
    }
  }
  __syncthreads();
  const size_t off = (static_cast<size_t>(row) * nchunk + cb) * kBins;
  for (int b = threadIdx.x; b < kBins; b += blockDim.x) {
    pcnt[off + b] = lc[b];
    pmass[off + b] = lm[b];
  }
}

struct ResolveShared {
  uint32_t hc[kBins];
  double hm[kBins];
  uint64_t cand[kCandCap];
  uint64_t small[kSmallCand];
  double wd[kResolveWaves];
  uint32_t wc[kResolveWaves];
  float2 mm[kResolveWaves];
  int best;
  uint32_t ncand;
  uint32_t nsmall;
  double selS;
  uint32_t selC;
  uint64_t thr;
  double fin_R;
  uint32_t fin_below;
  unsigned long long kmin, kmax;
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

// Loads of positions base + u * kResolveThreads + t, clamped to the row (the
// clamped duplicates are skipped by the caller's bound test).
__device__ __forceinline__ void load_batch(const float* __restrict__ sr, int64_t n, int64_t base,
                                           int t, float* v) {
#pragma unroll
  for (int u = 0; u < kReadBatch; ++u) v[u] = sr[min(base + u * kResolveThreads + t, n - 1)];
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int j) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), j);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), j);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ double readlane_f64(double v, int j) {
  const uint64_t b = readlane_u64(static_cast<uint64_t>(__double_as_longlong(v)), j);
  return __longlong_as_double(static_cast<long long>(b));
}

// One wave ends the search over c <= 64 keys (all in the current range): the
// cut key is the largest whose lower candidates carry mass <= epsZ - R.
__device__ void finish_small(ResolveShared& sh, int c, float m, double R, double epsZ) {
  const int lane = threadIdx.x & 63;
  const uint64_t k = lane < c ? sh.small[lane] : 0ull;
  const double w = lane < c ? static_cast<double>(weight(key64_score(k), m)) : 0.0;
  double lower = 0.0;
  uint32_t nlower = 0u;
  for (int j = 0; j < c; ++j) {
    const uint64_t kj = readlane_u64(k, j);
    const double wj = readlane_f64(w, j);
    if (kj < k) {
      lower += wj;
      ++nlower;
    }
  }
  uint64_t best = (lane < c && R + lower <= epsZ) ? k : 0ull;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint64_t other = static_cast<uint64_t>(
        __shfl_xor(static_cast<long long>(best), o, kWave));
    best = other > best ? other : best;
  }
  if (lane < c && k == best) {
    sh.thr = k;
    sh.fin_R = R + lower;
    sh.fin_below = nlower;
  }
}

__global__ __launch_bounds__(kResolveThreads) void resolve_kernel(
    const float* __restrict__ scores, int64_t n, const float2* __restrict__ blkstat, int nblk,
    const uint32_t* __restrict__ pcnt, const double* __restrict__ pmass, int npart, double eps,
    RowSel* __restrict__ rs, int32_t* __restrict__ k_eps, double* __restrict__ tau,
    double* __restrict__ lse, uint32_t* __restrict__ sel_mask, void* zero_base,
    size_t zero_bytes) {
  __shared__ ResolveShared sh;
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const float* sr = scores + static_cast<size_t>(row) * static_cast<size_t>(n);
  zero_slice(zero_base, zero_bytes, blockIdx.x, gridDim.x);

  if (t == 0) {
    sh.ncand = 0u;
    sh.nsmall = 0u;
    sh.kmin = ~0ull;
    sh.kmax = 0ull;
  }

  // Row (min, max).
  float2 mm;
  if (blkstat != nullptr) {
    mm = row_minmax(blkstat + static_cast<size_t>(row) * nblk, nblk, sh.mm);
  } else {
    float vmax = -INFINITY, vmin = INFINITY;
    for (int64_t base = 0; base < n; base += kReadBatch * kResolveThreads) {
      float v[kReadBatch];
      load_batch(sr, n, base, t, v);
#pragma unroll
      for (int u = 0; u < kReadBatch; ++u) {
        vmax = fmaxf(vmax, v[u]);  // clamped duplicates are row values too
        vmin = fminf(vmin, v[u]);
      }
    }
    vmax = wave_max_dpp(vmax);
    vmin = -wave_max_dpp(-vmin);
    if (lane == 0) sh.mm[wave] = make_float2(vmin, vmax);
    __syncthreads();
    mm = sh.mm[0];
    for (int w = 1; w < kResolveWaves; ++w) {
      mm.x = fminf(mm.x, sh.mm[w].x);
      mm.y = fmaxf(mm.y, sh.mm[w].y);
    }
  }
  const float m = mm.y;
  const float lo = mm.x;
  const float inv = lin_scale(lo, m);

  // Level-0 histogram: sum of the partials in chunk order, or a pass over the row.
  if (npart > 0) {
    // Partials in chunk order; eight chunks' loads are issued before any add.
    const size_t base = static_cast<size_t>(row) * npart * kBins;
    for (int b = t; b < kBins; b += kResolveThreads) {
      uint32_t c = 0u;
      double ms = 0.0;
      for (int p0 = 0; p0 < npart; p0 += 8) {
        uint32_t cv[8];
        double mv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const size_t o = base + static_cast<size_t>(min(p0 + u, npart - 1)) * kBins + b;
          cv[u] = pcnt[o];
          mv[u] = pmass[o];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (p0 + u < npart) {
            c += cv[u];
            ms += mv[u];
          }
        }
      }
      sh.hc[b] = c;
      sh.hm[b] = ms;
    }
  } else {
    for (int b = t; b < kBins; b += kResolveThreads) {
      sh.hc[b] = 0u;
      sh.hm[b] = 0.0;
    }
    __syncthreads();
    for (int64_t base = 0; base < n; base += kReadBatch * kResolveThreads) {
      float v[kReadBatch];
      load_batch(sr, n, base, t, v);
#pragma unroll
      for (int u = 0; u < kReadBatch; ++u) {
        if (base + u * kResolveThreads + t < n) {
          const int bin = lin_bin(v[u], lo, inv);
          atomicAdd(&sh.hc[bin], 1u);
          atomicAdd(&sh.hm[bin], static_cast<double>(weight(v[u], m)));
        }
      }
    }
  }
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

  // Level 0: the value bin holding the cut.
  double S;
  uint32_t C;
  int b0 = select_bin(sh, kBins, 0.0, epsZ, S, C);
  if (b0 < 0) {  // only with non-finite scores (unspecified results)
    b0 = 0;
    S = 0.0;
    C = 0u;
  }
  double R = S;
  uint64_t below = C;
  uint32_t cnt_in = sh.hc[b0];
  uint64_t prefix = 0;
  int plen = 0;
  bool in_lds = false;
  bool done = false;
  uint32_t ncand = 0;
  __syncthreads();

  // Each pass either copies the range into LDS, finishes it with one wave, or
  // narrows it by one 11-bit digit; at most ~8 passes are needed for 64-bit
  // keys, the bound only guards against non-finite scores.
  for (int guard = 0; guard < 16 && !done; ++guard) {
    if (!in_lds && cnt_in <= static_cast<uint32_t>(kCandCap)) {
      // Copy the keys of the current range into LDS (exactly cnt_in match).
      for (int64_t base = 0; base < n; base += kReadBatch * kResolveThreads) {
        float v[kReadBatch];
        load_batch(sr, n, base, t, v);
#pragma unroll
        for (int u = 0; u < kReadBatch; ++u) {
          const int64_t i = base + u * kResolveThreads + t;
          if (i < n && lin_bin(v[u], lo, inv) == b0) {
            const uint64_t k = key64(v[u], static_cast<uint32_t>(i));
            if (prefix_match(k, prefix, plen)) {
              const uint32_t slot = atomicAdd(&sh.ncand, 1u);
              if (slot < static_cast<uint32_t>(kCandCap)) sh.cand[slot] = k;
              atomicMin(&sh.kmin, static_cast<unsigned long long>(k));
              atomicMax(&sh.kmax, static_cast<unsigned long long>(k));
            }
          }
        }
      }
      __syncthreads();
      ncand = min(sh.ncand, static_cast<uint32_t>(kCandCap));
      in_lds = true;
      // Skip the leading bits all candidates share.
      const uint64_t diff = static_cast<uint64_t>(sh.kmin) ^ static_cast<uint64_t>(sh.kmax);
      const int common = diff == 0 ? 64 : __clzll(static_cast<long long>(diff));
      if (common > plen) {
        plen = common;
        prefix = plen >= 64 ? static_cast<uint64_t>(sh.kmin)
                            : (static_cast<uint64_t>(sh.kmin) >> (64 - plen));
      }
    }
    if (in_lds && cnt_in <= static_cast<uint32_t>(kSmallCand)) {
      // Gather the range's keys and let wave 0 finish.
      if (t == 0) sh.nsmall = 0u;
      __syncthreads();
      for (uint32_t c = t; c < ncand; c += kResolveThreads) {
        const uint64_t k = sh.cand[c];
        if (prefix_match(k, prefix, plen)) {
          const uint32_t slot = atomicAdd(&sh.nsmall, 1u);
          if (slot < static_cast<uint32_t>(kSmallCand)) sh.small[slot] = k;
        }
      }
      __syncthreads();
      if (wave == 0) finish_small(sh, static_cast<int>(min(sh.nsmall, static_cast<uint32_t>(kSmallCand))), m, R, epsZ);
      __syncthreads();
      R = sh.fin_R;
      below += sh.fin_below;
      done = true;
      break;
    }

    const int wdt = min(kDigitBits, 64 - plen);
    const int nb = 1 << wdt;
    const int shift = 64 - plen - wdt;
    for (int b = t; b < kBins; b += kResolveThreads) {
      sh.hc[b] = 0u;
      sh.hm[b] = 0.0;
    }
    __syncthreads();
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
      for (int64_t base = 0; base < n; base += kReadBatch * kResolveThreads) {
        float v[kReadBatch];
        load_batch(sr, n, base, t, v);
#pragma unroll
        for (int u = 0; u < kReadBatch; ++u) {
          const int64_t i = base + u * kResolveThreads + t;
          if (i < n && lin_bin(v[u], lo, inv) == b0) {
            const uint64_t k = key64(v[u], static_cast<uint32_t>(i));
            if (prefix_match(k, prefix, plen)) {
              const int b = static_cast<int>((k >> shift) & static_cast<uint64_t>(nb - 1));
              atomicAdd(&sh.hc[b], 1u);
              atomicAdd(&sh.hm[b], static_cast<double>(weight(v[u], m)));
            }
          }
        }
      }
    }
    __syncthreads();
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
  }
  if (!done) {
    // Ended by the pass bound (non-finite scores): report the range's top.
    if (t == 0) sh.thr = prefix;
    __syncthreads();
  }
  const uint64_t thr = sh.thr;

  if (t == 0) {
    rs[row].m = m;
    rs[row].lo = lo;
    rs[row].Z = Z;
    rs[row].thr = thr;
    k_eps[row] = static_cast<int32_t>(static_cast<uint64_t>(n) - below);
    tau[row] = R / Z;
    if (lse) lse[row] = static_cast<double>(m) + log(Z);
  }
  if (sel_mask != nullptr) {
    // Bit i % 32 of word i / 32: key i is in the head.  Each wave covers 64
    // consecutive keys per step.
    const int64_t nwords = ceil_div(n, 32);
    uint32_t* mrow = sel_mask + static_cast<size_t>(row) * static_cast<size_t>(nwords);
    for (int64_t base = static_cast<int64_t>(wave) * 64; base < n;
         base += static_cast<int64_t>(kResolveWaves) * 64) {
      const int64_t i = base + lane;
      const bool kept = i < n && key64(sr[min(i, n - 1)], static_cast<uint32_t>(i)) >= thr;
      const uint64_t bits = __ballot(kept);
      if (lane == 0) mrow[base / 32] = static_cast<uint32_t>(bits);
      if (lane == 1 && base / 32 + 1 < nwords) mrow[base / 32 + 1] = static_cast<uint32_t>(bits >> 32);
    }
  }
}

}  // namespace

int hist_nchunk(int64_t n, int rows) {
  // About two blocks per CU in total and at least 4096 keys per block.
  const int64_t total = n * static_cast<int64_t>(rows);
  int64_t chunk = ceil_div(total, 2 * kNumCUs);
  chunk = ceil_div(chunk, 4096) * 4096;
  if (chunk > n) chunk = n;
  return static_cast<int>(ceil_div(n, chunk));
}

hipError_t launch_hist0(const float* scores, int64_t n, int rows, const float2* blkstat,
                        int nblk, int nchunk, uint32_t* pcnt, double* pmass, hipStream_t st) {
  const int64_t chunk = ceil_div(n, nchunk);
  return launch(hist0_kernel, dim3(static_cast<unsigned>(nchunk) * rows), dim3(256), 0, st,
                scores, n, chunk, nchunk, blkstat, nblk, pcnt, pmass);
}

hipError_t launch_resolve(const float* scores, int64_t n, int rows, const float2* blkstat,
                          int nblk, const uint32_t* pcnt, const double* pmass, int npart,
                          double eps, RowSel* rs, int32_t* k_eps, double* tau, double* lse,
                          uint32_t* sel_mask, void* zero_base, size_t zero_bytes,
                          hipStream_t st) {
  return launch(resolve_kernel, dim3(rows), dim3(kResolveThreads), 0, st, scores, n, blkstat,
                nblk, pcnt, pmass, npart, eps, rs, k_eps, tau, lse, sel_mask, zero_base,
                zero_bytes);
}

}  // namespace ctopk
