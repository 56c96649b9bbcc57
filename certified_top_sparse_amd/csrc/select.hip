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
//            weights w = exp(s - m); an fp64 mass histogram over kBins
//            equal-width value bins on [min, max] -- built by many blocks per
//            row for long rows (hist0_kernel, per-chunk partials, no atomics
//            across blocks) or inside the row's own block, which then holds
//            the row in registers; Z = the bins' sum in a fixed order;
//            lse = m + log Z.  The cut bin b* is the largest bin of positive
//            mass whose lower bins hold mass <= eps*Z; one pass then counts
//            the keys of lower bins and copies b*'s keys into LDS;
//   level >0 (resolve_kernel, one block per row): histogram (count, mass) of
//            the next 11 bits of key64 inside the range and keep the bin
//            holding the cut.  Once the range holds <= kCandCap keys they are
//            in LDS and the radix continues from the first bit where they
//            differ; once it holds <= 64 keys one wave finishes by comparing
//            every pair.  key64 is unique, so the search always ends on one key.
// Counts are exact integers, so k_eps is exact given the weights; masses are
// fp64 sums of fp32 weights.  tau = R / Z uses the same weights as Z.
#include <type_traits>

#include "kernels.h"
#include "vsum_body.h"

namespace ctopk {
namespace {

constexpr int kResolveThreads = 1024;
constexpr int kResolveWaves = kResolveThreads / 64;
// Row scans keep kReadBatch loads in flight per thread.
constexpr int kReadBatch = 16;
// Candidate sets this small are finished by one wave.
constexpr int kSmallCand = 64;
// Rows up to this length are held in registers by their block (32 per thread).
constexpr int kResolveRegRow = 32 * kResolveThreads;

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
                                                    double* __restrict__ pmass) {
  __shared__ double lm[kBins];
  __shared__ float2 s_red[4];
  const int row = static_cast<int>(blockIdx.x / static_cast<unsigned>(nchunk));
  const int cb = static_cast<int>(blockIdx.x % static_cast<unsigned>(nchunk));
  for (int b = threadIdx.x; b < kBins; b += blockDim.x) lm[b] = 0.0;
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
        atomicAdd(&lm[lin_bin(v[u], lo, inv)], static_cast<double>(weight(v[u], m)));
      }
    }
  }
  __syncthreads();
  const size_t off = (static_cast<size_t>(row) * nchunk + cb) * kBins;
  for (int b = threadIdx.x; b < kBins; b += blockDim.x) pmass[off + b] = lm[b];
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
  float f0, f1;  // bin b0 of level 0 is the score range [f0, f1)
};

// Wave totals of the current histogram (nb <= kBins bins in sh.hc / sh.hm):
// thread t holds bins 2t and 2t + 1, so wave w covers bins [128 w, 128 w + 128).
// Every lane of a wave gets the same fixed-tree sum; sh.wd / sh.wc hold them.
// With by_mass the histogram holds masses only and a bin counts as non-empty
// when its mass is positive (bins of weight-0 keys, which underflowed, lie
// below every positive bin and never hold the cut).
__device__ __forceinline__ uint32_t bin_count(const ResolveShared& sh, int b, int nb, bool by_mass) {
  if (b >= nb) return 0u;
  return by_mass ? (sh.hm[b] > 0.0 ? 1u : 0u) : sh.hc[b];
}

__device__ void hist_wave_totals(ResolveShared& sh, int nb, bool by_mass) {
  const int t = threadIdx.x;
  const int b0 = 2 * t;
  const double m = (b0 < nb ? sh.hm[b0] : 0.0) + (b0 + 1 < nb ? sh.hm[b0 + 1] : 0.0);
  const uint32_t c = bin_count(sh, b0, nb, by_mass) + bin_count(sh, b0 + 1, nb, by_mass);
  const double wm = wave_sum_f64(m);
  const uint32_t wc = wave_sum_u32_dpp(c);
  if ((t & 63) == 0) {
    sh.wd[t >> 6] = wm;
    sh.wc[t >> 6] = wc;
  }
  __syncthreads();
}

// Block-wide choice of the cut bin among nb bins held in sh.hc / sh.hm, after
// hist_wave_totals: the largest non-empty bin whose lower bins hold mass
// R + S <= epsZ.  Every thread scans the 16 wave totals to find the wave that
// holds it; only that wave scans its own 128 bins.  Returns b* and, through S
// and C, the mass and count of the bins below it (-1 if no bin qualifies; C
// is meaningless with by_mass).
__device__ int select_bin(ResolveShared& sh, int nb, bool by_mass, double R, double epsZ,
                          double& S, uint32_t& C) {
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  double P = 0.0, Pw = 0.0;
  uint32_t PC = 0u, PCw = 0u;
  int ws = -1;
  for (int w = 0; w < kResolveWaves; ++w) {
    const uint32_t c = sh.wc[w];
    if (c != 0u && R + P <= epsZ) {
      ws = w;
      Pw = P;
      PCw = PC;
    }
    P += sh.wd[w];
    PC += c;
  }
  if (wave == ws) {
    const int b0 = 2 * t;
    const uint32_t c0 = bin_count(sh, b0, nb, by_mass);
    const uint32_t c1 = bin_count(sh, b0 + 1, nb, by_mass);
    const double m0 = b0 < nb ? sh.hm[b0] : 0.0;
    const double m1 = b0 + 1 < nb ? sh.hm[b0 + 1] : 0.0;
    const double im = wave_incl_scan_f64_dpp(m0 + m1);
    const uint32_t ic = wave_incl_scan_u32_dpp(c0 + c1);
    double em = __shfl_up(im, 1, kWave);
    uint32_t ec = __shfl_up(ic, 1, kWave);
    if (lane == 0) {
      em = 0.0;
      ec = 0u;
    }
    const double ex0 = Pw + em;
    const double ex1 = ex0 + m0;
    const uint32_t exc0 = PCw + ec;
    int mine = -1;
    if (c0 != 0u && R + ex0 <= epsZ) mine = b0;
    if (c1 != 0u && R + ex1 <= epsZ) mine = b0 + 1;
    // The wave's first non-empty bin qualifies (its prefix is Pw), so the
    // ballot is never empty; the highest qualifying lane holds the answer.
    const uint64_t bal = __ballot(mine >= 0);
    const int L = 63 - __clzll(static_cast<long long>(bal));
    if (lane == L) {
      sh.best = mine;
      sh.selS = mine == b0 ? ex0 : ex1;
      sh.selC = mine == b0 ? exc0 : exc0 + c0;
    }
  } else if (ws < 0 && t == 0) {
    sh.best = -1;
  }
  __syncthreads();
  S = sh.selS;
  C = sh.selC;
  return sh.best;
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
__device__ void finish_small(ResolveShared& sh, const uint64_t* keys, int c, float m, double R,
                             double epsZ) {
  const int lane = threadIdx.x & 63;
  const uint64_t k = lane < c ? keys[lane] : 0ull;
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
  const uint64_t best = wave_pick_u64<true>((lane < c && R + lower <= epsZ) ? k : 0ull);
  if (lane < c && k == best) {
    sh.thr = k;
    sh.fin_R = R + lower;
    sh.fin_below = nlower;
  }
}

// The smallest score s >= lo with lin_bin(s, lo, inv) >= b, for a whole wave
// (every lane returns it); -inf for b <= 0 and +inf past the last bin.  The
// bin is non-decreasing in s, so s lies in bins [b, b') iff
// bin_floor(b) <= s < bin_floor(b'): membership by two compares instead of
// recomputing the bin.  A 64-ary search over the order-preserving integer
// encoding of the scores: lin_bin(lo) = 0 < b and lin_bin(+inf) = kBins - 1
// >= b keep the answer in (L, H]; each round tests the points L + step * j,
// j = 1..64, step = ceil((H - L) / 64), and keeps one step.
__device__ float bin_floor(int b, float lo, float inv) {
  if (b <= 0) return -INFINITY;
  if (b >= kBins) return INFINITY;
  const uint32_t lane = threadIdx.x & (kWave - 1);
  uint32_t L = ukey(lo), H = ukey(INFINITY);
  // Start from a bracket of 512 representable values around lo + b / inv when
  // it holds the answer (lin_bin is monotone, so checking its two ends is
  // enough; only extreme fp32 rounding would miss): two rounds instead of
  // about six.  Every lane takes the same branch.
  if (inv > 0.0f) {
    const float g = lo + static_cast<float>(b) / inv;
    if (isfinite(g)) {
      const uint32_t ug = ukey(g);
      const uint32_t gl = ug > L + 256u ? ug - 256u : L;
      const uint32_t gh = ug < H - 256u ? ug + 256u : H;
      const bool okl = gl == L || lin_bin(ukey_to_float(gl), lo, inv) < b;
      const bool okh = gh == H || lin_bin(ukey_to_float(gh), lo, inv) >= b;
      if (okl && okh) {
        L = gl;
        H = gh;
      }
    }
  }
  while (H - L > 1u) {
    const uint32_t step = (H - L + 63u) >> 6;
    const uint32_t off = step * (lane + 1u);  // at most (H - L) + 63 * 64 < 2^32
    const uint32_t p = off < H - L ? L + off : H;
    const bool ge = p == H || lin_bin(ukey_to_float(p), lo, inv) >= b;
    const uint64_t bal = __ballot(ge);  // lane 63 tests H, so never empty
    const int j = __ffsll(static_cast<long long>(bal)) - 1;  // first point at or past
    // j is wave-uniform: scalar lane reads
    H = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(p), j));
    L = j > 0 ? static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(p), j - 1)) : L;
  }
  return ukey_to_float(H);
}

// The elements of one row as seen by one thread of its block: element
// i = u * kResolveThreads + t.  With PT > 0 the thread holds its PT elements
// in registers, all loaded when the block starts (rows of n <= PT * 1024);
// with PT == 0 every pass streams them from global memory in batches.
template <int PT>
struct RowElems {
  float v[PT > 0 ? PT : 1];
  const float* sr;
  int64_t n;

  __device__ __forceinline__ void load(const float* __restrict__ row, int64_t len) {
    sr = row;
    n = len;
    if constexpr (PT > 0) {  // n <= PT * kResolveThreads: 32-bit indices
      const int last = static_cast<int>(len) - 1;
#pragma unroll
      for (int u = 0; u < PT; ++u)
        v[u] = row[min(u * kResolveThreads + static_cast<int>(threadIdx.x), last)];
    }
  }

  // As for_each, but every slot of a register row is visited without a
  // branch: f(i, s, valid), where slots past n (valid false) hold a copy of
  // the row's last element and must contribute nothing.
  template <typename F>
  __device__ __forceinline__ void for_each_all(F&& f) {
    if constexpr (PT > 0) {
      int t = threadIdx.x;
      asm volatile("" : "+v"(t));
#pragma unroll
      for (int u = 0; u < PT; ++u) asm volatile("" : "+v"(v[u]));
      const int nn = static_cast<int>(n);
#pragma unroll
      for (int u = 0; u < PT; ++u) {
        const int i = u * kResolveThreads + t;
        f(static_cast<int64_t>(i), v[u], i < nn);
        if ((u & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      for_each([&](int64_t i, float s) { f(i, s, true); });
    }
  }

  // Each pass recomputes what it derives from an element (bin, weight, key):
  // the empty asm makes the values opaque, so the compiler cannot keep such
  // per-element results live from one pass to the next (PT registers each).
  template <typename F>
  __device__ __forceinline__ void for_each(F&& f) {
    int t = threadIdx.x;
    if constexpr (PT > 0) {
      asm volatile("" : "+v"(t));  // indices are recomputed per pass, not kept
#pragma unroll
      for (int u = 0; u < PT; ++u) asm volatile("" : "+v"(v[u]));
      const int nn = static_cast<int>(n);
#pragma unroll
      for (int u = 0; u < PT; ++u) {
        const int i = u * kResolveThreads + t;
        if (i < nn) f(static_cast<int64_t>(i), v[u]);
        // bound the scheduler's window: it would otherwise evaluate many
        // elements ahead and run out of registers
        if ((u & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      for (int64_t base = 0; base < n; base += kReadBatch * kResolveThreads) {
        float vv[kReadBatch];
        load_batch(sr, n, base, t, vv);
#pragma unroll
        for (int u = 0; u < kReadBatch; ++u) {
          const int64_t i = base + u * kResolveThreads + t;
          if (i < n) f(i, vv[u]);
        }
      }
    }
  }
};

// The select of one row by one workgroup of kResolveThreads threads.
template <int PT>
__device__ __forceinline__ void resolve_row(
    ResolveShared& sh, int row, const float* __restrict__ scores, int64_t n,
    const float2* __restrict__ blkstat, int nblk, const double* __restrict__ pmass, int npart,
    double eps, RowSel* __restrict__ rs, int32_t* __restrict__ k_eps, double* __restrict__ tau,
    double* __restrict__ lse, uint32_t* __restrict__ sel_mask, void* zero_base,
    size_t zero_bytes) {
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const float* sr = scores + static_cast<size_t>(row) * static_cast<size_t>(n);
  RowElems<PT> E;
  E.load(sr, n);  // register rows: every load of the row is in flight from here
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
    E.for_each([&](int64_t, float s) {
      vmax = fmaxf(vmax, s);
      vmin = fminf(vmin, s);
    });
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

  // Level-0 histogram of masses: sum of the partials in chunk order, or a
  // pass over the row (one LDS atomic per key; counts come from the pass
  // that collects the cut bin's keys).
  if (PT == 0 && npart > 0) {
    // Partials in chunk order; eight chunks' loads are issued before any add.
    const size_t base = static_cast<size_t>(row) * npart * kBins;
    for (int b = t; b < kBins; b += kResolveThreads) {
      double ms = 0.0;
      for (int p0 = 0; p0 < npart; p0 += 8) {
        double mv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          mv[u] = pmass[base + static_cast<size_t>(min(p0 + u, npart - 1)) * kBins + b];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (p0 + u < npart) ms += mv[u];
      }
      sh.hm[b] = ms;
    }
  } else {
    for (int b = t; b < kBins; b += kResolveThreads) sh.hm[b] = 0.0;
    __syncthreads();
    E.for_each_all([&](int64_t, float s, bool valid) {
      atomicAdd(&sh.hm[lin_bin(s, lo, inv)], valid ? static_cast<double>(weight(s, m)) : 0.0);
    });
  }
  __syncthreads();

  // Z = total weight: wave totals (fixed DPP trees) added in wave order.
  hist_wave_totals(sh, kBins, true);
  double Z = 0.0;
  for (int w = 0; w < kResolveWaves; ++w) Z += sh.wd[w];
  const double epsZ = eps * Z;

  // Level 0: the value bin holding the cut.
  double S;
  uint32_t C;
  int b0 = select_bin(sh, kBins, true, 0.0, epsZ, S, C);
  if (b0 < 0) {  // only with non-finite scores (unspecified results)
    b0 = 0;
    S = 0.0;
  }
  double R = S;
  uint64_t below = 0;
  uint64_t prefix = 0;
  int plen = 0;
  bool done = false;

  // Copies the keys of the current range (bin b0 and the prefix) into LDS,
  // up to kCandCap of them, with one LDS atomic per wave and step; returns
  // how many there are.  With count_below it also adds the number of keys in
  // lower bins to `below`.
  // Bin b0 is the score range [f0, f1) (two waves search in parallel).
  if (wave < 2) {
    const float f = bin_floor(b0 + wave, lo, inv);
    if (lane == 0) (wave == 0 ? sh.f0 : sh.f1) = f;
  }
  auto collect = [&](bool count_below, auto with_prefix) -> uint32_t {
    // Only passes after the first (plen > 0) match the key prefix; the first
    // builds key64 only in waves that hold a candidate.
    constexpr bool kPrefix = decltype(with_prefix)::value;
    if (t == 0) {
      sh.ncand = 0u;
      sh.kmin = ~0ull;
      sh.kmax = 0ull;
    }
    __syncthreads();
    const float f0 = sh.f0, f1 = sh.f1;
    uint32_t nbelow = 0u;  // counted from lane masks; lane 0 holds the wave's count
    unsigned long long kmn = ~0ull, kmx = 0ull;
    E.for_each_all([&](int64_t i, float s, bool valid) {
      // One lane mask per comparison (each a single vector compare), combined
      // on the scalar unit; bitwise, not short-circuit: no branch per key.
      const uint64_t mv = __builtin_amdgcn_ballot_w64(valid);
      const uint64_t mge = __builtin_amdgcn_ballot_w64(s >= f0);
      nbelow += static_cast<uint32_t>(__popcll(mv & __builtin_amdgcn_ballot_w64(s < f0)));
      uint64_t bal = mv & mge & __builtin_amdgcn_ballot_w64(s < f1);
      bool in = valid & (s >= f0) & (s < f1);
      uint64_t k = 0ull;
      if constexpr (kPrefix) {
        k = key64(s, static_cast<uint32_t>(i));
        const bool pm = prefix_match(k, prefix, plen);
        in = in & pm;
        bal &= __builtin_amdgcn_ballot_w64(pm);
      }
      if (bal != 0ull) {
        if constexpr (!kPrefix) k = key64(s, static_cast<uint32_t>(i));
        const int leader = __ffsll(static_cast<long long>(bal)) - 1;
        uint32_t base = 0u;
        if (lane == leader) base = atomicAdd(&sh.ncand, static_cast<uint32_t>(__popcll(bal)));
        base = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(base), leader));
        if (in) {
          const uint32_t slot =
              base + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal >> 32),
                                               __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0u));
          if (slot < static_cast<uint32_t>(kCandCap)) sh.cand[slot] = k;
          kmn = k < kmn ? k : kmn;
          kmx = k > kmx ? k : kmx;
        }
      }
    });
    kmn = wave_pick_u64<false>(kmn);
    kmx = wave_pick_u64<true>(kmx);
    if (count_below && lane == 0) sh.wc[wave] = nbelow;
    if (lane == 0 && kmn <= kmx) {
      atomicMin(&sh.kmin, kmn);
      atomicMax(&sh.kmax, kmx);
    }
    __syncthreads();
    if (count_below) {
      uint64_t bsum = 0;
      for (int w = 0; w < kResolveWaves; ++w) bsum += sh.wc[w];
      below += bsum;
    }
    return sh.ncand;
  };

  uint32_t cnt_in = collect(true, std::false_type{});
  uint32_t ncand = min(cnt_in, static_cast<uint32_t>(kCandCap));
  bool in_lds = cnt_in <= static_cast<uint32_t>(kCandCap);
  // The LDS list holds exactly the keys of the current range (every key of it
  // matches the prefix) until a digit level narrows the range.
  bool cand_exact = in_lds;
  if (in_lds) {  // skip the leading bits all candidates share
    const uint64_t diff = static_cast<uint64_t>(sh.kmin) ^ static_cast<uint64_t>(sh.kmax);
    plen = diff == 0 ? 64 : __clzll(static_cast<long long>(diff));
    // (a shift by 64 is undefined, so plen == 0 keeps the empty prefix)
    prefix = plen == 0 ? 0ull
                       : (plen >= 64 ? static_cast<uint64_t>(sh.kmin)
                                     : (static_cast<uint64_t>(sh.kmin) >> (64 - plen)));
  }
  __syncthreads();

  // Each pass either copies the range into LDS, finishes it with one wave, or
  // narrows it by one 11-bit digit; at most ~8 passes are needed for 64-bit
  // keys, the bound only guards against non-finite scores.
  for (int guard = 0; guard < 16 && !done; ++guard) {
    if (!in_lds && cnt_in <= static_cast<uint32_t>(kCandCap)) {
      cnt_in = collect(false, std::true_type{});
      ncand = min(cnt_in, static_cast<uint32_t>(kCandCap));
      in_lds = true;
      cand_exact = true;
      // Skip the leading bits all candidates share.
      const uint64_t diff = static_cast<uint64_t>(sh.kmin) ^ static_cast<uint64_t>(sh.kmax);
      const int common = diff == 0 ? 64 : __clzll(static_cast<long long>(diff));
      if (common > plen) {
        plen = common;
        prefix = plen >= 64 ? static_cast<uint64_t>(sh.kmin)
                            : (static_cast<uint64_t>(sh.kmin) >> (64 - plen));
      }
      __syncthreads();
    }
    if (in_lds && cnt_in <= static_cast<uint32_t>(kSmallCand)) {
      if (cand_exact) {  // the list is exactly the range: wave 0 finishes from it
        if (wave == 0) finish_small(sh, sh.cand, static_cast<int>(ncand), m, R, epsZ);
      } else {  // gather the range's keys from the list, then wave 0 finishes
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
        if (wave == 0)
          finish_small(sh, sh.small,
                       static_cast<int>(min(sh.nsmall, static_cast<uint32_t>(kSmallCand))), m, R,
                       epsZ);
      }
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
      const float f0 = sh.f0, f1 = sh.f1;
      E.for_each([&](int64_t i, float s) {
        if (s >= f0 && s < f1) {
          const uint64_t k = key64(s, static_cast<uint32_t>(i));
          if (prefix_match(k, prefix, plen)) {
            const int b = static_cast<int>((k >> shift) & static_cast<uint64_t>(nb - 1));
            atomicAdd(&sh.hc[b], 1u);
            atomicAdd(&sh.hm[b], static_cast<double>(weight(s, m)));
          }
        }
      });
    }
    __syncthreads();
    hist_wave_totals(sh, nb, false);
    int bs = select_bin(sh, nb, false, R, epsZ, S, C);
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
    cand_exact = false;  // the list may now hold keys outside the narrowed range
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

template <int PT>
__global__ __launch_bounds__(kResolveThreads) void resolve_kernel(
    const float* __restrict__ scores, int64_t n, const float2* __restrict__ blkstat, int nblk,
    const double* __restrict__ pmass, int npart, double eps, RowSel* __restrict__ rs,
    int32_t* __restrict__ k_eps, double* __restrict__ tau, double* __restrict__ lse,
    uint32_t* __restrict__ sel_mask, void* zero_base, size_t zero_bytes) {
  __shared__ ResolveShared sh;
  resolve_row<PT>(sh, static_cast<int>(blockIdx.x), scores, n, blkstat, nblk, pmass, npart, eps,
                  rs, k_eps, tau, lse, sel_mask, zero_base, zero_bytes);
}

// The select of every row and, on the compute units it leaves idle, the
// dense value stream: workgroups [0, rows) each select one row; the others
// each sum w v over one chunk of keys for GB query heads of one V head, with
// weights exp(s - m) from the row maximum alone (no cut needed).  One launch
// places both, so they run side by side.
template <typename T, int D, int GB>
union SelectDenseSmem {
  ResolveShared r;
  StreamSmem<T, D, GB, kStreamDense, kResolveWaves> v;
};

template <typename T, int D, int GB>
__global__ __launch_bounds__(kResolveThreads) void select_dense_kernel(
    const float* __restrict__ scores, int64_t n, const float2* __restrict__ blkstat, int nblk,
    double eps, RowSel* __restrict__ rs, int32_t* __restrict__ k_eps, double* __restrict__ tau,
    double* __restrict__ lse, uint32_t* __restrict__ sel_mask, int rows, int G,
    const T* __restrict__ V, float* __restrict__ dpart, int nchunk, int tpb, int nz) {
  __shared__ SelectDenseSmem<T, D, GB> sm;
  const int b = static_cast<int>(blockIdx.x);
  if (b < rows) {
    resolve_row<kResolveRegRow / kResolveThreads>(sm.r, b, scores, n, blkstat, nblk, nullptr, 0,
                                                  eps, rs, k_eps, tau, lse, sel_mask, nullptr, 0);
    return;
  }
  const int db = b - rows;
  const int grp = db / nchunk;
  value_stream_block<T, D, GB, kStreamDense, kResolveWaves>(sm.v, scores, n, G, V, nullptr,
                                                            blkstat, nblk, dpart, nchunk, tpb,
                                                            db % nchunk, grp / nz, grp % nz);
}

template <typename T, int D, int GB>
hipError_t select_dense_t(const float* scores, int64_t n, int rows, const float2* blkstat,
                          int nblk, double eps, RowSel* rs, int32_t* k_eps, double* tau,
                          double* lse, uint32_t* sel_mask, int n_v, const void* V, float* dpart,
                          int nchunk, hipStream_t st) {
  const int G = rows / n_v;
  const int nz = static_cast<int>(ceil_div(G, GB));
  const int tpb = static_cast<int>(ceil_div(ceil_div(n, kVsumTile), nchunk));
  const unsigned grid = static_cast<unsigned>(rows + n_v * nz * nchunk);
  return launch(select_dense_kernel<T, D, GB>, dim3(grid), dim3(kResolveThreads), 0, st, scores,
                n, blkstat, nblk, eps, rs, k_eps, tau, lse, sel_mask, rows, G,
                static_cast<const T*>(V), dpart, nchunk, tpb, nz);
}

template <typename T, int D>
hipError_t select_dense_d(const float* scores, int64_t n, int rows, const float2* blkstat,
                          int nblk, double eps, RowSel* rs, int32_t* k_eps, double* tau,
                          double* lse, uint32_t* sel_mask, int n_v, const void* V, float* dpart,
                          int nchunk, hipStream_t st) {
  const int G = rows / n_v;
#define CTOPK_SD(GB)                                                                            \
  select_dense_t<T, D, GB>(scores, n, rows, blkstat, nblk, eps, rs, k_eps, tau, lse, sel_mask, \
                           n_v, V, dpart, nchunk, st)
  if (G == 1) return CTOPK_SD(1);
  if (G == 2) return CTOPK_SD(2);
  if constexpr (kGroupMax<T, D> == 4) {
    return CTOPK_SD(4);
  } else {
    if (G <= 4) return CTOPK_SD(4);
    return CTOPK_SD(8);
  }
#undef CTOPK_SD
}

}  // namespace

int select_dense_nchunk(int64_t n, int rows, int n_v, int v_dtype, int dv) {
  // Rows held in registers by the widest register-row select, and at least
  // half the compute units left beside the select's workgroups: the dense
  // stream then takes at most about twice as long as a stream over the whole
  // chip, which the select's own time covers.
  if (n <= 16 * kResolveThreads || n > kResolveRegRow) return 0;
  const int spare = kNumCUs - rows;
  if (spare < kNumCUs / 2) return 0;
  const int groups = vsum_groups(rows, n_v, v_dtype, dv);
  const int64_t tiles = ceil_div(n, kVsumTile);
  int64_t want = spare / groups;  // at most `spare` workgroups in total
  if (want > tiles) want = tiles;
  if (want < 1) return 0;
  const int64_t tpb = ceil_div(tiles, want);
  if (tpb * kVsumTile > kFixKeys) return 0;  // the tail pass lists a chunk in LDS
  return static_cast<int>(ceil_div(tiles, tpb));
}

hipError_t launch_select_dense(const float* scores, int64_t n, int rows, const float2* blkstat,
                               int nblk, double eps, RowSel* rs, int32_t* k_eps, double* tau,
                               double* lse, uint32_t* sel_mask, int n_v, const void* V,
                               int v_dtype, int dv, float* dpart, int nchunk, hipStream_t st) {
  if (v_dtype == 1) {
    if (dv == 128)
      return select_dense_d<uint16_t, 128>(scores, n, rows, blkstat, nblk, eps, rs, k_eps, tau,
                                           lse, sel_mask, n_v, V, dpart, nchunk, st);
    return select_dense_d<uint16_t, 64>(scores, n, rows, blkstat, nblk, eps, rs, k_eps, tau, lse,
                                        sel_mask, n_v, V, dpart, nchunk, st);
  }
  if (dv == 128)
    return select_dense_d<float, 128>(scores, n, rows, blkstat, nblk, eps, rs, k_eps, tau, lse,
                                      sel_mask, n_v, V, dpart, nchunk, st);
  return select_dense_d<float, 64>(scores, n, rows, blkstat, nblk, eps, rs, k_eps, tau, lse,
                                   sel_mask, n_v, V, dpart, nchunk, st);
}

int resolve_register_row() { return kResolveRegRow; }

int hist_nchunk(int64_t n, int rows) {
  // About two blocks per CU in total and at least 4096 keys per block.
  const int64_t total = n * static_cast<int64_t>(rows);
  int64_t chunk = ceil_div(total, 2 * kNumCUs);
  chunk = ceil_div(chunk, 4096) * 4096;
  if (chunk > n) chunk = n;
  return static_cast<int>(ceil_div(n, chunk));
}

hipError_t launch_hist0(const float* scores, int64_t n, int rows, const float2* blkstat,
                        int nblk, int nchunk, double* pmass, hipStream_t st) {
  const int64_t chunk = ceil_div(n, nchunk);
  return launch(hist0_kernel, dim3(static_cast<unsigned>(nchunk) * rows), dim3(256), 0, st,
                scores, n, chunk, nchunk, blkstat, nblk, pmass);
}

hipError_t launch_resolve(const float* scores, int64_t n, int rows, const float2* blkstat,
                          int nblk, const double* pmass, int npart,
                          double eps, RowSel* rs, int32_t* k_eps, double* tau, double* lse,
                          uint32_t* sel_mask, void* zero_base, size_t zero_bytes,
                          hipStream_t st) {
#define CTOPK_RESOLVE(PT)                                                                    \
  launch(resolve_kernel<PT>, dim3(rows), dim3(kResolveThreads), 0, st, scores, n, blkstat, nblk, \
         pmass, npart, eps, rs, k_eps, tau, lse, sel_mask, zero_base, zero_bytes)
  if (npart == 0 && n <= 8 * kResolveThreads) return CTOPK_RESOLVE(8);
  if (npart == 0 && n <= 16 * kResolveThreads) return CTOPK_RESOLVE(16);
  if (npart == 0 && n <= kResolveRegRow) return CTOPK_RESOLVE(kResolveRegRow / kResolveThreads);
  return CTOPK_RESOLVE(0);
#undef CTOPK_RESOLVE
}

}  // namespace ctopk
