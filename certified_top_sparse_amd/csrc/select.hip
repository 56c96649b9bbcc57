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
//            score scan's per-tile pairs or from a pass over a register row
//            (given logits streamed from memory take a sampled range and
//            reference instead, checked against the row's true maximum);
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
// A sampled weight reference may lie this far below the row maximum: fp32
// weights stay below e^80 and their fp64 sums far from overflow.
constexpr float kSampledHeadroom = 80.0f;

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
  constexpr int U = 16;
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

// The workgroup ends the search over c <= 64 keys (all in the current range):
// the cut key is the largest whose lower candidates carry mass <= epsZ - R.
// Lane i of every wave holds candidate i; wave w sums, for each i, the
// weights of candidates j of its slice [w per, w per + per) below key i, and
// wave 0 adds the slices in wave order (sh.hm and sh.hc, free by now, hold
// the partial masses and counts).  Called by every thread of the block.
__device__ void finish_small(ResolveShared& sh, const uint64_t* keys, int c, float m, double R,
                             double epsZ) {
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  static_assert(kResolveWaves * kSmallCand <= kBins, "slice partials fit the histogram");
  const uint64_t k = lane < c ? keys[lane] : 0ull;
  const int per = (c + kResolveWaves - 1) / kResolveWaves;
  const int j0 = wave * per, j1 = min(c, j0 + per);
  double lower = 0.0;
  uint32_t nlower = 0u;
  for (int j = j0; j < j1; ++j) {  // wave-uniform: LDS broadcast reads
    const uint64_t kj = keys[j];
    const double wj = static_cast<double>(weight(key64_score(kj), m));
    if (kj < k) {
      lower += wj;
      ++nlower;
    }
  }
  sh.hm[wave * kSmallCand + lane] = lower;
  sh.hc[wave * kSmallCand + lane] = nlower;
  __syncthreads();
  if (wave == 0) {
    double L = 0.0;
    uint32_t N = 0u;
    for (int g = 0; g < kResolveWaves; ++g) {
      L += sh.hm[g * kSmallCand + lane];
      N += sh.hc[g * kSmallCand + lane];
    }
    const uint64_t best = wave_pick_u64<true>((lane < c && R + L <= epsZ) ? k : 0ull);
    if (lane < c && k == best) {
      sh.thr = k;
      sh.fin_R = R + L;
      sh.fin_below = N;
    }
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
      // Slots past n hold a copy of element i mod P, P the largest power of
      // two <= n: their zero contributions then fall into bins spread like
      // the row's own instead of queueing on one bin's atomics.
      const int nn = static_cast<int>(len);
      if (nn == PT * kResolveThreads) {
#pragma unroll
        for (int u = 0; u < PT; ++u) v[u] = row[u * kResolveThreads + static_cast<int>(threadIdx.x)];
      } else {
        const int pmask = (1 << (31 - __clz(nn))) - 1;
#pragma unroll
        for (int u = 0; u < PT; ++u) {
          const int i = u * kResolveThreads + static_cast<int>(threadIdx.x);
          v[u] = row[i < nn ? i : (i & pmask)];
        }
      }
    }
  }

  // As for_each, but every slot of a register row is visited without a
  // branch: f(i, s, valid), where slots past n (valid false) hold a copy of
  // an element of the row and must contribute nothing.
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
    size_t zero_bytes, CutPub* publish = nullptr) {
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

  // The level-0 range [lo, hi] and the weight reference m.  From the scan's
  // tile pairs or a pass over a register row these are the row's minimum and
  // maximum.  A row streamed from memory without tile pairs takes them from
  // a strided sample of one key per thread, widened by half the sample's
  // span on each side (keys outside fall into the end bins), so that level 0
  // is its first pass over the row; that pass also finds the row's true
  // maximum and minimum, and is redone over them if the maximum lies so far
  // above the reference that weights could overflow.
  auto block_minmax = [&](float vmin, float vmax) -> float2 {
    vmax = wave_max_dpp(vmax);
    vmin = -wave_max_dpp(-vmin);
    if (lane == 0) sh.mm[wave] = make_float2(vmin, vmax);
    __syncthreads();
    float2 r = sh.mm[0];
    for (int w = 1; w < kResolveWaves; ++w) {
      r.x = fminf(r.x, sh.mm[w].x);
      r.y = fmaxf(r.y, sh.mm[w].y);
    }
    __syncthreads();  // sh.mm is free again
    return r;
  };
  const bool sampled = PT == 0 && blkstat == nullptr && npart == 0;
  float2 mm;
  float m;
  if (blkstat != nullptr) {
    mm = row_minmax(blkstat + static_cast<size_t>(row) * nblk, nblk, sh.mm);
    m = mm.y;
  } else if (sampled) {
    const int64_t stride = n > kResolveThreads ? n / kResolveThreads : 1;
    const float sv = sr[min(static_cast<int64_t>(t) * stride, n - 1)];
    mm = block_minmax(sv, sv);
    m = mm.y;
    const float half = 0.5f * (mm.y - mm.x);
    mm.x -= half;
    mm.y += half;
  } else {
    float vmax = -INFINITY, vmin = INFINITY;
    E.for_each([&](int64_t, float s) {
      vmax = fmaxf(vmax, s);
      vmin = fminf(vmin, s);
    });
    mm = block_minmax(vmin, vmax);
    m = mm.y;
  }
  float lo = mm.x;
  float inv = lin_scale(lo, mm.y);

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
  } else if (sampled) {
    for (int pass = 0; pass < 2; ++pass) {
      for (int b = t; b < kBins; b += kResolveThreads) sh.hm[b] = 0.0;
      __syncthreads();
      float vmax = -INFINITY, vmin = INFINITY;
      E.for_each([&](int64_t, float s) {
        vmax = fmaxf(vmax, s);
        vmin = fminf(vmin, s);
        atomicAdd(&sh.hm[lin_bin_clamped(s, lo, inv)], static_cast<double>(weight(s, m)));
      });
      const float2 tr = block_minmax(vmin, vmax);
      if (pass == 1 || tr.y - m <= kSampledHeadroom) break;
      // every thread saw the same tr: the redo is uniform over the block
      lo = tr.x;
      m = tr.y;
      inv = lin_scale(lo, m);
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
  // Bin b0 is the score range [f0, f1) (two waves search in parallel).
  if (wave < 2) {
    const float f = bin_floor(b0 + wave, lo, inv);
    if (lane == 0) (wave == 0 ? sh.f0 : sh.f1) = f;
  }
  // Other workgroups of the launch may use the bin before the cut is known:
  // (ukey(f0), ukey(f1)) in one word, non-zero since ukey of a float is.
  if (publish != nullptr) {
    __syncthreads();
    if (t == 0)
      __hip_atomic_store(&publish->bin,
                         (static_cast<uint64_t>(ukey(sh.f0)) << 32) | ukey(sh.f1),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  uint64_t prefix = 0;
  int plen = 0;
  bool done = false;

  // Copies the keys of the current range (the score range [f0, f1) and the
  // prefix) into LDS, up to kCandCap of them, with one LDS atomic per wave
  // and step; returns how many there are.  With count_below it also adds the
  // number of keys below f0 to `below`.
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
    uint32_t nbelow = 0u;  // lane 0 holds the wave's count
    unsigned long long kmn = ~0ull, kmx = 0ull;
    if constexpr (!kPrefix && PT > 0) {
      // A register row's first pass in vector code only: per lane, the count
      // of its keys below f0 and one bit per slot in [f0, f1); only the few
      // lanes with such a slot then append their keys (one LDS atomic each).
      int tt = t;
      asm volatile("" : "+v"(tt));
#pragma unroll
      for (int u = 0; u < PT; ++u) asm volatile("" : "+v"(E.v[u]));
      static_assert(PT <= 32, "one bit per slot");
      const int nn = static_cast<int>(n);
      uint32_t cnt = 0u, inm = 0u;
#pragma unroll
      for (int u = 0; u < PT; ++u) {
        const float sv = E.v[u];
        const bool valid = u * kResolveThreads + tt < nn;
        cnt += (valid & (sv < f0)) ? 1u : 0u;
        inm |= (valid & (sv >= f0) & (sv < f1)) ? (1u << u) : 0u;
      }
      nbelow = wave_sum_u32_dpp(cnt);
      if (inm != 0u) {
#pragma unroll
        for (int u = 0; u < PT; ++u) {
          if (inm & (1u << u)) {
            const uint64_t k = key64(E.v[u], static_cast<uint32_t>(u * kResolveThreads + tt));
            const uint32_t slot = atomicAdd(&sh.ncand, 1u);
            if (slot < static_cast<uint32_t>(kCandCap)) sh.cand[slot] = k;
            kmn = k < kmn ? k : kmn;
            kmx = k > kmx ? k : kmx;
          }
        }
      }
    } else if constexpr (!kPrefix && PT == 0) {
      // A streamed row's first pass, batch by batch, in the same vector form:
      // per lane the count of its keys below f0 and one bit per slot of the
      // batch in [f0, f1); the few lanes with a set bit append their keys.
      static_assert(kReadBatch <= 32, "one bit per slot");
      uint32_t cnt = 0u;
      for (int64_t base = 0; base < n; base += static_cast<int64_t>(kReadBatch) * kResolveThreads) {
        float vv[kReadBatch];
        load_batch(sr, n, base, t, vv);
        uint32_t inm = 0u;
#pragma unroll
        for (int u = 0; u < kReadBatch; ++u) {
          const bool valid = base + u * kResolveThreads + t < n;
          cnt += (valid & (vv[u] < f0)) ? 1u : 0u;
          inm |= (valid & (vv[u] >= f0) & (vv[u] < f1)) ? (1u << u) : 0u;
        }
        if (inm != 0u) {
#pragma unroll
          for (int u = 0; u < kReadBatch; ++u) {
            if (inm & (1u << u)) {
              const uint64_t k =
                  key64(vv[u], static_cast<uint32_t>(base + u * kResolveThreads + t));
              const uint32_t slot = atomicAdd(&sh.ncand, 1u);
              if (slot < static_cast<uint32_t>(kCandCap)) sh.cand[slot] = k;
              kmn = k < kmn ? k : kmn;
              kmx = k > kmx ? k : kmx;
            }
          }
        }
      }
      nbelow = wave_sum_u32_dpp(cnt);
    } else {
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
    }
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
      if (cand_exact) {  // the list is exactly the range: finish from it
        finish_small(sh, sh.cand, static_cast<int>(ncand), m, R, epsZ);
      } else {  // gather the range's keys from the list, then finish
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
  // Other workgroups of the launch may wait for the cut: the head's mass and
  // the cut, with device-scope stores.  Both words are zero before and
  // non-zero after (the head holds the row maximum, and every finite score's
  // key64 has a non-zero upper word), and each has this one writer, so a
  // reader that sees both non-zero has both final values, in either order.
  if (publish != nullptr && t == 0) {
    const double den = Z - R;
    __hip_atomic_store(&publish->den, den > 0.0 ? den : 1.0, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&publish->cut, thr != 0ull ? thr : 1ull, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }

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
// value stream, in one launch.  Workgroups [0, rows) each select one row and
// publish its head's mass and cut (pub[row]).  The others each own one chunk
// of keys of GB query heads of one V head and:
//   1. guess each head's cut from 512 of its scores (64 evenly spaced runs of
//      8 consecutive keys; one wave per head bisects the sample's score range
//      for the value below which the sample's softmax mass first exceeds eps
//      of its total) -- a provisional head {key64 >= spec};
//   2. stream V over the chunk summing w v for the provisional head
//      (w = exp(s - m), m the row maximum from the scan's tile pairs, the same
//      m and weights the select uses), keeping the chunk's scores in LDS,
//      while the select runs;
//   3. wait for the level-0 bin [f0, f1) that holds the cut, which the
//      select publishes as soon as it has it; list every key whose
//      membership may differ from the guess's (kept by it and below f1, or
//      left out and at or above f0; in key order in LDS, packed into as few
//      waves as possible) and load their V rows;
//   4. wait for the published mass and cut (bounded spins on pub[]; the
//      select workgroups have the lowest ids, so they were dispatched first,
//      and they wait on nothing), add, signed, w v of the listed keys the cut
//      decides against the guess (+ for head keys the guess left out, - for
//      the others) to the lane sums, reduce them over the workgroup (fp64
//      per head and V element) and add num / den into out with device-scope
//      float atomics (out is zeroed before the launch).
// out is thus a sum of one term per chunk in arrival order: reproducible to
// fp32 rounding of those terms, not bit for bit.  A timed-out wait adds NaN.
// pub[] and out must be zero at launch (the score scan zeroes both).
constexpr int kSpecRuns = 64;       // sample runs per head (one per lane)
constexpr int kSpecRunKeys = 8;     // consecutive keys per run
constexpr int kSpecRounds = 10;     // bisection rounds of the guess
constexpr int kSpinLimit = 1 << 21;  // polls of about a microsecond: ~2 s, never reached

template <typename T, int D, int GB>
struct SpecSmem {
  union {
    StreamSmem<T, D, GB, kStreamGiven, kResolveWaves> v;
    struct {
      int idx[kFixKeys];
      float w[kFixKeys][GB];
      __attribute__((aligned(16))) uint32_t cnt[kFixKeys / kResolveThreads][kResolveWaves];
    } band;
  };
  float stash[GB * kFixKeys];  // the chunk's scores, [head][key in chunk]
  float mx[GB][kResolveWaves];
  uint64_t spec[GB];
  uint64_t exact[GB];
  double den[GB];
  float f0[GB], f1[GB];  // the level-0 bin [f0, f1) that holds each head's cut
};

// Steps 3 and 4 above, run by value_stream_block after the stream with every
// lane's sums (acc[j][e]: head j, V elements seg * EPL + e of the rows the
// lane handles).
template <typename T, int D, int GB>
struct SpecFinish {
  SpecSmem<T, D, GB>* sm;
  const T* V;
  const CutPub* pub;
  const float* m;
  float* out;
  int64_t c0;
  int len, h0, nh;

  template <typename L>
  __device__ __forceinline__ void operator()(L& ln) const {
    using Acc = typename AccOf<T>::type;
    constexpr int NT = kResolveThreads, NW = kResolveWaves;
    constexpr int KPT = kFixKeys / NT;
    constexpr int EPL = VSlice<T>::kElems, LPR = D / EPL, RPW = kWave / LPR;
    static_assert(kFixKeys % NT == 0, "whole keys per thread");
    const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
    const int seg = lane % LPR, rg = lane / LPR;
    __syncthreads();  // every wave is past its stream loop: the staging LDS is free
    // The level-0 bin [f0, f1) of each head's cut, published by its select
    // as soon as it is known (well before the cut itself).  Keys below the
    // bin are outside the head and keys above it inside, whatever the cut;
    // only the bin's own keys wait for it.  Without the word (a timed-out
    // wait) every key is treated as undecided.
    if (t < nh) {
      uint64_t b = 0ull;
      for (int it = 0; it < kSpinLimit; ++it) {
        b = __hip_atomic_load(&pub[h0 + t].bin, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (b != 0ull) break;
        __builtin_amdgcn_s_sleep(2);
      }
      sm->f0[t] = b != 0ull ? ukey_to_float(static_cast<uint32_t>(b >> 32)) : -INFINITY;
      sm->f1[t] = b != 0ull ? ukey_to_float(static_cast<uint32_t>(b)) : INFINITY;
    }
    __syncthreads();

    // Lists the keys whose signed weight for some head is non-zero, in key
    // order (sm->band.idx, sm->band.w); returns how many.  wfun(i, j)
    // gives key i's signed weight for head j (i < len, j < nh).
    auto compact = [&](auto wfun) -> int {
      float wv[KPT][GB];
      bool sel[KPT];
      uint64_t bal[KPT];
#pragma unroll
      for (int u = 0; u < KPT; ++u) {
        const int i = t + u * NT;
        bool any = false;
#pragma unroll
        for (int j = 0; j < GB; ++j) {
          const float w = (j < nh && i < len) ? wfun(i, j) : 0.0f;
          wv[u][j] = w;
          any = any || w != 0.0f;
        }
        sel[u] = any;
        bal[u] = __ballot(any);
        if (lane == 0) sm->band.cnt[u][wave] = static_cast<uint32_t>(__popcll(bal[u]));
      }
      __syncthreads();
      uint32_t base = 0u;
      static_assert(NW % 4 == 0, "counts read as 16-byte vectors");
#pragma unroll
      for (int u = 0; u < KPT; ++u) {
        uint32_t before = 0u, all = 0u;
        uint4 c4[NW / 4];
#pragma unroll
        for (int q = 0; q < NW / 4; ++q) c4[q] = reinterpret_cast<const uint4*>(sm->band.cnt[u])[q];
#pragma unroll
        for (int q = 0; q < NW / 4; ++q) {
          const uint32_t c[4] = {c4[q].x, c4[q].y, c4[q].z, c4[q].w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            before += 4 * q + r < wave ? c[r] : 0u;
            all += c[r];
          }
        }
        if (sel[u]) {
          const uint32_t slot =
              base + before +
              __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal[u] >> 32),
                                        __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal[u]), 0u));
          sm->band.idx[slot] = t + u * NT;
#pragma unroll
          for (int j = 0; j < GB; ++j) sm->band.w[slot][j] = wv[u][j];
        }
        base += all;
      }
      __syncthreads();
      return static_cast<int>(base);
    };
    // Listed entry e goes to wave (e / PER) % NW, load it = (e % PER) / RPW
    // of a round, row group e % RPW, so a short list occupies few waves.
    constexpr int ITB = 4;
    constexpr int PER = ITB * RPW;
    // Adds the listed rows' signed w v to the lane sums (which hold the
    // provisional head's), the V rows of the first round having been loaded
    // into u0 already when `preloaded`.
    auto accumulate = [&](int nb, uint4 (&u0)[ITB], bool preloaded) {
      bool first = true;
      for (int k0 = wave * PER; k0 < nb; k0 += NW * PER) {
        uint4 u[ITB];
#pragma unroll
        for (int it = 0; it < ITB; ++it) {
          if (first && preloaded) {
            u[it] = u0[it];
          } else {
            const int e = min(k0 + it * RPW + rg, nb - 1);
            const int64_t r = c0 + sm->band.idx[e];
            u[it] = *reinterpret_cast<const uint4*>(V + r * D + seg * EPL);
          }
        }
        first = false;
#pragma unroll
        for (int it = 0; it < ITB; ++it) {
          const int e = k0 + it * RPW + rg;
          const bool valid = e < nb;
          const int ec = min(e, nb - 1);
          float v[EPL];
          VSlice<T>::load(u[it], v);
#pragma unroll
          for (int j = 0; j < GB; ++j) {
            const Acc w = valid ? static_cast<Acc>(sm->band.w[ec][j]) : Acc(0);
#pragma unroll
            for (int e2 = 0; e2 < EPL; ++e2) ln.acc[j][e2] += w * static_cast<Acc>(v[e2]);
          }
        }
      }
    };
    // The lane sums over the workgroup: the row groups of a wave by
    // cross-lane adds, then the waves in order through LDS in fp64; each
    // column's num / den into out.
    auto finish_out = [&]() {
#pragma unroll
      for (int j = 0; j < GB; ++j)
#pragma unroll
        for (int e = 0; e < EPL; ++e) ln.acc[j][e] = stride_sum<LPR>(ln.acc[j][e]);
      __syncthreads();  // the list is read: its LDS takes the reduction
      if (rg == 0) {
#pragma unroll
        for (int j = 0; j < GB; ++j)
#pragma unroll
          for (int e = 0; e < EPL; ++e) sm->v.red[0][wave][j * D + seg * EPL + e] = ln.acc[j][e];
      }
      __syncthreads();
      for (int col = t; col < nh * D; col += NT) {
        const int j = col / D;
        double sum = 0.0;
#pragma unroll
        for (int g = 0; g < NW; ++g) sum += static_cast<double>(sm->v.red[0][g][col]);
        unsafeAtomicAdd(out + static_cast<size_t>(h0 + j) * D + (col - j * D),
                        static_cast<float>(sum / sm->den[j]));
      }
    };
    auto score_of = [&](int i, int j) { return sm->stash[j * kFixKeys + i]; };

    // Every key whose membership may differ from the guess's: kept by the
    // guess and below f1 (the cut may leave it out: marked -1), or left out
    // and at or above f0 (the cut may take it: +1); weights are computed
    // for listed keys only, once the cut is known.  Their first round of V
    // rows is loaded before the wait for the cut.
    uint4 u0[ITB];
    int nb;
    {
      // thresholds and this thread's scores in registers first: the list's
      // own LDS stores would otherwise force a reload per test
      uint64_t sp[GB];
      float lo_f[GB], hi_f[GB], sc[KPT][GB];
#pragma unroll
      for (int j = 0; j < GB; ++j) {
        sp[j] = sm->spec[j];
        lo_f[j] = sm->f0[j];
        hi_f[j] = sm->f1[j];
#pragma unroll
        for (int u = 0; u < KPT; ++u) sc[u][j] = score_of(min(t + u * NT, kFixKeys - 1), j);
      }
      nb = compact([&](int i, int j) -> float {
        const float s = sc[(i - t) / NT][j];
        const bool in_spec = key64(s, static_cast<uint32_t>(c0 + i)) >= sp[j];
        return in_spec ? (s < hi_f[j] ? -1.0f : 0.0f) : (s >= lo_f[j] ? 1.0f : 0.0f);
      });
    }
    if (nb > 0) {
      const int k0 = wave * PER;
#pragma unroll
      for (int it = 0; it < ITB; ++it) {
        const int e = min(k0 + it * RPW + rg, nb - 1);
        const int64_t r = c0 + sm->band.idx[e];
        u0[it] = *reinterpret_cast<const uint4*>(V + r * D + seg * EPL);
      }
    }
    if (t < nh) {
      // Both words non-zero: both stores have landed (each word has one
      // writer, and zero is only its value before that store).
      uint64_t c = 0ull;
      double dn = 0.0;
      for (int it = 0; it < kSpinLimit; ++it) {
        c = __hip_atomic_load(&pub[h0 + t].cut, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        dn = __hip_atomic_load(&pub[h0 + t].den, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (c != 0ull && dn != 0.0) break;
        __builtin_amdgcn_s_sleep(2);
      }
      const bool got = c != 0ull && dn != 0.0;
      sm->exact[t] = got ? c : ~0ull;
      sm->den[t] = got ? dn : __longlong_as_double(0x7FF8000000000000LL);  // NaN: no cut arrived
    }
    __syncthreads();
    if (nb > 0) {
      // Each listed (key, head) gets its signed weight where the cut decides
      // against the guess (the bin decides every key outside it), else 0.
      for (int p = t; p < nb * GB; p += NT) {
        const int e = p / GB, j = p % GB;
        const float mark = sm->band.w[e][j];
        float w = 0.0f;
        if (mark != 0.0f) {
          const int i = sm->band.idx[e];
          const float s = score_of(i, j);
          const bool in_head =
              s >= sm->f1[j] ||
              (s >= sm->f0[j] && key64(s, static_cast<uint32_t>(c0 + i)) >= sm->exact[j]);
          const bool in_spec = mark < 0.0f;
          if (in_head != in_spec) w = in_spec ? -weight(s, m[j]) : weight(s, m[j]);
        }
        sm->band.w[e][j] = w;
      }
      __syncthreads();
      accumulate(nb, u0, true);
    }
    finish_out();
  }
};

template <typename T, int D, int GB>
__device__ __forceinline__ void spec_stream_block(
    SpecSmem<T, D, GB>& sm, const float* __restrict__ scores, int64_t n, int G,
    const T* __restrict__ V, const float2* __restrict__ blkstat, int nblk, double eps, int tpb,
    int chunk, int vh, int hz, const CutPub* __restrict__ pub, float* __restrict__ out) {
  constexpr int NT = kResolveThreads, NW = kResolveWaves;
  static_assert(kSpecRuns == kWave, "one sample run per lane");
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int h0 = vh * G + hz * GB;
  const int nh = min(GB, G - hz * GB);

  // Wave j < nh loads head j's sample (run of lane l at l (n - 8) / 63, or
  // keys l + 64 u of short rows); every thread loads its share of the scan's
  // tile maxima.  Both are issued before any arithmetic.
  float sv[kSpecRunKeys];
  const bool sampler = wave < nh;
  if (sampler) {
    const float* srow = scores + static_cast<size_t>(h0 + wave) * static_cast<size_t>(n);
    if (n >= kSpecRuns * kSpecRunKeys) {
      const int64_t p = static_cast<int64_t>(lane) * (n - kSpecRunKeys) / (kSpecRuns - 1);
#pragma unroll
      for (int u = 0; u < kSpecRunKeys; ++u) sv[u] = srow[p + u];
    } else {
#pragma unroll
      for (int u = 0; u < kSpecRunKeys; ++u) {
        const int64_t i = lane + static_cast<int64_t>(kWave) * u;
        sv[u] = i < n ? srow[i] : -INFINITY;  // -inf: weight 0, never below a finite t
      }
    }
  }
#pragma unroll
  for (int j = 0; j < GB; ++j) {
    const float2* bs = blkstat + static_cast<size_t>(h0 + min(j, nh - 1)) * nblk;
    float vmax = -INFINITY;
    for (int b = t; b < nblk; b += NT) vmax = fmaxf(vmax, bs[b].y);
    vmax = wave_max_dpp(vmax);
    if (lane == 0) sm.mx[j][wave] = vmax;
  }
  if (sampler) {
    // Bisection over the sample's range for the largest value t with the
    // sample's mass below t at most eps of its total (fp32; only a guess).
    float smax = -INFINITY, smin = INFINITY;
#pragma unroll
    for (int u = 0; u < kSpecRunKeys; ++u) {
      smax = fmaxf(smax, sv[u]);
      smin = sv[u] > -INFINITY ? fminf(smin, sv[u]) : smin;
    }
    smax = wave_max_dpp(smax);
    smin = -wave_max_dpp(-smin);
    float wsv[kSpecRunKeys];
    float tot = 0.0f;
#pragma unroll
    for (int u = 0; u < kSpecRunKeys; ++u) {
      wsv[u] = sv[u] > -INFINITY ? weight(sv[u], smax) : 0.0f;
      tot += wsv[u];
    }
    const float lim = static_cast<float>(eps) * group_sum<kWave>(tot);
    float lo = smin, hi = smax;
    for (int r = 0; r < kSpecRounds; ++r) {
      const float mid = 0.5f * (lo + hi);
      float below = 0.0f;
#pragma unroll
      for (int u = 0; u < kSpecRunKeys; ++u) below += sv[u] < mid ? wsv[u] : 0.0f;
      if (group_sum<kWave>(below) > lim) {
        hi = mid;
      } else {
        lo = mid;
      }
    }
    if (lane == 0) {
      const uint64_t spec = lo > smin ? static_cast<uint64_t>(ukey(lo)) << 32 : 0ull;
      sm.spec[wave] = spec;
      sm.v.thr[wave] = spec;
    }
  } else if (wave == nh && lane < GB - nh) {  // unused head slots keep nothing
    sm.spec[nh + lane] = ~0ull;
    sm.v.thr[nh + lane] = ~0ull;
  }
  __syncthreads();
  float mx[GB];
#pragma unroll
  for (int j = 0; j < GB; ++j) {
    float b = sm.mx[j][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) b = fmaxf(b, sm.mx[j][w]);
    mx[j] = b;
  }
  if (t < GB) sm.v.m[t] = mx[t];
  __syncthreads();

  const int64_t c0 = static_cast<int64_t>(chunk) * tpb * kVsumTile;
  const int len = static_cast<int>(min(n - c0, static_cast<int64_t>(tpb) * kVsumTile));
  const T* Vb = V + static_cast<size_t>(vh) * static_cast<size_t>(n) * D;
  SpecFinish<T, D, GB> fin{&sm, Vb, pub, mx, out, c0, len, h0, nh};
  value_stream_block<T, D, GB, kStreamGiven, NW>(sm.v, scores, n, G, V, nullptr, nullptr, 0, tpb,
                                                 chunk, vh, hz, fin, sm.stash);
}

template <typename T, int D, int GB>
union SelectSpecSmem {
  ResolveShared r;
  SpecSmem<T, D, GB> s;
};

template <typename T, int D, int GB>
__global__ __launch_bounds__(kResolveThreads) void select_spec_kernel(
    const float* __restrict__ scores, int64_t n, const float2* __restrict__ blkstat, int nblk,
    double eps, RowSel* __restrict__ rs, int32_t* __restrict__ k_eps, double* __restrict__ tau,
    double* __restrict__ lse, uint32_t* __restrict__ sel_mask, int rows, int G,
    const T* __restrict__ V, int nchunk, int tpb, int nz, CutPub* pub, float* __restrict__ out) {
  __shared__ SelectSpecSmem<T, D, GB> sm;
  const int b = static_cast<int>(blockIdx.x);
  if (b < rows) {
    resolve_row<kResolveRegRow / kResolveThreads>(sm.r, b, scores, n, blkstat, nblk, nullptr, 0,
                                                  eps, rs, k_eps, tau, lse, sel_mask, nullptr, 0,
                                                  pub + b);
    return;
  }
  const int db = b - rows;
  const int grp = db / nchunk;
  spec_stream_block<T, D, GB>(sm.s, scores, n, G, V, blkstat, nblk, eps, tpb, db % nchunk,
                              grp / nz, grp % nz, pub, out);
}

template <typename T, int D, int GB>
hipError_t select_spec_t(const float* scores, int64_t n, int rows, const float2* blkstat,
                         int nblk, double eps, RowSel* rs, int32_t* k_eps, double* tau,
                         double* lse, uint32_t* sel_mask, int n_v, const void* V, int nchunk,
                         CutPub* pub, float* out, hipStream_t st) {
  const int G = rows / n_v;
  const int nz = static_cast<int>(ceil_div(G, GB));
  const int tpb = static_cast<int>(ceil_div(ceil_div(n, kVsumTile), nchunk));
  const unsigned grid = static_cast<unsigned>(rows + n_v * nz * nchunk);
  return launch(select_spec_kernel<T, D, GB>, dim3(grid), dim3(kResolveThreads), 0, st, scores,
                n, blkstat, nblk, eps, rs, k_eps, tau, lse, sel_mask, rows, G,
                static_cast<const T*>(V), nchunk, tpb, nz, pub, out);
}

template <typename T, int D>
hipError_t select_spec_d(const float* scores, int64_t n, int rows, const float2* blkstat,
                         int nblk, double eps, RowSel* rs, int32_t* k_eps, double* tau,
                         double* lse, uint32_t* sel_mask, int n_v, const void* V, int nchunk,
                         CutPub* pub, float* out, hipStream_t st) {
  const int G = rows / n_v;
#define CTOPK_SS(GB)                                                                           \
  select_spec_t<T, D, GB>(scores, n, rows, blkstat, nblk, eps, rs, k_eps, tau, lse, sel_mask, \
                          n_v, V, nchunk, pub, out, st)
  if (G == 1) return CTOPK_SS(1);
  if (G == 2) return CTOPK_SS(2);
  if constexpr (kGroupMax<T, D> == 4) {
    return CTOPK_SS(4);
  } else {
    if (G <= 4) return CTOPK_SS(4);
    return CTOPK_SS(8);
  }
#undef CTOPK_SS
}

}  // namespace

int select_spec_nchunk(int64_t n, int rows, int n_v, int v_dtype, int dv) {
  // Rows held in registers by the widest register-row select, and at least
  // half the compute units left beside the select's workgroups: the stream
  // then takes at most about twice as long as a stream over the whole chip,
  // which the select's own time covers.  At most one workgroup per compute
  // unit in total, so the whole launch is resident at once.
  if (n <= 16 * kResolveThreads || n > kResolveRegRow) return 0;
  const int spare = kNumCUs - rows;
  if (spare < kNumCUs / 2) return 0;
  const int groups = vsum_groups(rows, n_v, v_dtype, dv);
  const int64_t tiles = ceil_div(n, kVsumTile);
  int64_t want = spare / groups;  // at most `spare` workgroups in total
  if (want > tiles) want = tiles;
  if (want < 1) return 0;
  const int64_t tpb = ceil_div(tiles, want);
  if (tpb * kVsumTile > kFixKeys) return 0;  // a chunk's correction list lives in LDS
  return static_cast<int>(ceil_div(tiles, tpb));
}

hipError_t launch_select_spec(const float* scores, int64_t n, int rows, const float2* blkstat,
                              int nblk, double eps, RowSel* rs, int32_t* k_eps, double* tau,
                              double* lse, uint32_t* sel_mask, int n_v, const void* V,
                              int v_dtype, int dv, int nchunk, CutPub* pub, float* out,
                              hipStream_t st) {
  if (v_dtype == 1) {
    if (dv == 128)
      return select_spec_d<uint16_t, 128>(scores, n, rows, blkstat, nblk, eps, rs, k_eps, tau,
                                           lse, sel_mask, n_v, V, nchunk, pub, out, st);
    return select_spec_d<uint16_t, 64>(scores, n, rows, blkstat, nblk, eps, rs, k_eps, tau, lse,
                                        sel_mask, n_v, V, nchunk, pub, out, st);
  }
  if (dv == 128)
    return select_spec_d<float, 128>(scores, n, rows, blkstat, nblk, eps, rs, k_eps, tau, lse,
                                      sel_mask, n_v, V, nchunk, pub, out, st);
  return select_spec_d<float, 64>(scores, n, rows, blkstat, nblk, eps, rs, k_eps, tau, lse,
                                   sel_mask, n_v, V, nchunk, pub, out, st);
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
