// Fused decode for short rows (n <= kShortRowMaxN keys): one workgroup per
// query row computes the row's scores, selects its certified head and writes
// the head-only output, in a single launch.
//
// What is computed is the same as on the other decode plans (the Abstract of
// "A Mathematical Theory of Top-k Sparse Attention via Total Variation
// Distance", arXiv 2512.07647): P = softmax of the scores s_i = scale * <q, k_i>,
// the head = the k largest-score keys (ties broken toward the lower index),
// with k_eps the least k whose discarded tail mass TV = P(tail) is at most
// eps, tau = that TV, and out = the head-only attention output
// sum_{i in head} P_i v_i / P(head).
//
// Why a separate kernel: for a row of a few hundred keys the general path is
// four launches whose every phase is a short dependent step (its select alone
// is ~9 us for 1024 keys, almost all of it fixed per-phase latency).  Here the
// whole row lives in one workgroup of sixteen waves, one key per thread:
//   1. scores: the score scan's lane layout and arithmetic (Slice<T>::dot and
//      group_sum over the LPR lanes of a row, then * scale), so every score is
//      bitwise the scan's; staged in LDS;
//   2. lo, m = row minimum and maximum, w_i = weight(s_i, m) (the library's
//      one fp32 weight), Z = sum of w_i in fp64 in a fixed order;
//   3. the cut key by a mass-weighted descent: a (count, fp64 mass) histogram
//      of the keys in the current range, and the highest non-empty bin whose
//      lower bins leave the mass below the range, R, at most eps * Z.  Level 0
//      has 256 equal-width value bins over [lo, m] (each a contiguous range of
//      the key order); further levels, needed only when the range holds more
//      than kShortFin keys, take 8-bit digits of key64 = (order-preserving
//      score bits << 32) | ~i below the bits the range's keys share.  The last
//      range is finished by comparing every pair: the cut is the largest key
//      whose lower keys carry mass <= eps * Z - R;
//   4. the head-only output: the rows of the head keys' V, 16-byte loads in
//      the scan's lane layout (tail rows are never read), w v summed per lane
//      in fp32, lanes of a wave and then the waves added in a fixed order in
//      fp64, divided by the head's mass Z - R.
// One workgroup reads the row's K and V at what one compute unit can pull
// (about 90 GB/s measured on MI355X): 256 KiB of K takes ~2.8 us, and each
// row-level step of the select ~1 us of LDS and cross-lane latency; a call
// at n = 1024 takes ~10.4 us against ~17.7 us for the general path's four
// launches.  Four waves with four keys per thread measured slower (~15 us:
// a quarter of the loads in flight).

#include "kernels.h"
#include "scan_dot.h"

namespace ctopk {
namespace {

// Sixteen waves: with a whole row's K (or V) slices in flight at once each
// pass costs one memory round trip.
constexpr int kShortThreads = 1024;
constexpr int kShortWaves = kShortThreads / kWave;
// Keys per thread: key i is held by thread i % kShortThreads, slot i / kShortThreads.
constexpr int kShortPT = kShortRowMaxN / kShortThreads;
static_assert(kShortPT * kShortThreads == kShortRowMaxN, "whole slots");
constexpr int kShortDigit = 8;
constexpr int kShortBins = 1 << kShortDigit;
static_assert(kShortBins == 4 * kWave, "one wave scans the bins, four per lane");
static_assert(kShortBins <= kShortThreads, "one thread clears each bin");
// Ranges of at most this many keys are finished by comparing every pair.
constexpr int kShortFin = 64;
// 16-byte loads in flight per lane in the K and V passes.
constexpr int kShortBatch = 16;

template <int D>
struct ShortShared {
  float s[kShortRowMaxN];   // scores
  float wh[kShortRowMaxN];  // weights of head keys, 0 for the tail
  double hm[kShortBins];    // histogram of the current level: mass
  uint32_t hc[kShortBins];  // and count
  uint64_t cand[kShortFin];
  union {
    struct {
      double m[kShortWaves][kShortFin];
      uint32_t c[kShortWaves][kShortFin];
    } fin;                        // per-wave partial masses and counts of the pair finish
    float red[kShortWaves][D];    // per-wave output partials
  } u;
  float2 wmm[kShortWaves];
  double wz[kShortWaves];
  double selS;
  double finR;
  uint64_t thr;
  unsigned long long kmin, kmax;
  int best;
  uint32_t selC, selN, finN, ncand;
};

__device__ __forceinline__ bool prefix_is(uint64_t k, uint64_t prefix, int plen) {
  return plen == 0 ? true : (plen >= 64 ? k == prefix : (k >> (64 - plen)) == prefix);
}

template <typename T, int D>
__global__ __launch_bounds__(kShortThreads) void short_row_kernel(
    const T* __restrict__ q, const T* __restrict__ K, const T* __restrict__ V,
    const float* __restrict__ head_scale, float default_scale, int n, int G, double eps,
    float* __restrict__ out, int32_t* __restrict__ k_eps, double* __restrict__ tau,
    double* __restrict__ lse, uint32_t* __restrict__ sel_mask, float* __restrict__ scores) {
  constexpr int EPL = Slice<T>::kElems;     // elements per 16-byte slice
  constexpr int LPR = D / EPL;              // lanes per K or V row
  constexpr int RPW = kWave / LPR;          // rows per wave and load instruction
  constexpr int RPB = RPW * kShortWaves;    // rows per block and load instruction
  static_assert(LPR == 8 || LPR == 16 || LPR == 32, "lane stride of the output sums");
  // V slices in flight per lane (bf16 unpacks to twice the registers).
  constexpr int kVBatch = EPL == 8 ? kShortBatch / 2 : kShortBatch;
  __shared__ ShortShared<D> sh;

  const int row = static_cast<int>(blockIdx.x);
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = t / kWave;
  const int seg = lane % LPR;
  const int rg = lane / LPR;
  const size_t kv_base = static_cast<size_t>(row / G) * static_cast<size_t>(n) * D;
  const int iters = (n + RPB - 1) / RPB;

  // 1. Scores.  Row r of load step it is it * RPB + wave * RPW + rg; loads of
  // rows past n re-read row n - 1 and are never used.
  {
    const uint4 qv = *reinterpret_cast<const uint4*>(q + static_cast<size_t>(row) * D + seg * EPL);
    const float scale = head_scale != nullptr ? head_scale[row] : default_scale;
    for (int it0 = 0; it0 < iters; it0 += kShortBatch) {
      uint4 kv[kShortBatch];
#pragma unroll
      for (int u = 0; u < kShortBatch; ++u) {
        const int r = min((it0 + u) * RPB + wave * RPW + rg, n - 1);
        kv[u] = load_stream16(K + kv_base + static_cast<size_t>(r) * D + seg * EPL);
      }
#pragma unroll
      for (int u = 0; u < kShortBatch; ++u) {
        const int r = (it0 + u) * RPB + wave * RPW + rg;
        const float acc = group_sum<LPR>(Slice<T>::dot(kv[u], qv));
        if (seg == 0 && r < n) sh.s[r] = acc * scale;
      }
    }
  }
  __syncthreads();

  // 2. Row minimum and maximum, weights and Z (per thread in slot order, wave
  // trees, then the waves in order).
  float s[kShortPT], w[kShortPT];
  uint64_t key[kShortPT];
  bool valid[kShortPT];
  float vmin = INFINITY, vmax = -INFINITY;
#pragma unroll
  for (int u = 0; u < kShortPT; ++u) {
    const int i = u * kShortThreads + t;
    valid[u] = i < n;
    s[u] = valid[u] ? sh.s[i] : 0.0f;
    if (valid[u]) {
      vmin = fminf(vmin, s[u]);
      vmax = fmaxf(vmax, s[u]);
      if (scores != nullptr) scores[static_cast<size_t>(row) * n + i] = s[u];
    }
    key[u] = valid[u] ? key64(s[u], static_cast<uint32_t>(i)) : 0ull;
  }
  {
    const float wmx = wave_max_dpp(vmax);
    const float wmn = -wave_max_dpp(-vmin);
    if (lane == 0) sh.wmm[wave] = make_float2(wmn, wmx);
  }
  __syncthreads();
  float lo = sh.wmm[0].x, m = sh.wmm[0].y;
  for (int i = 1; i < kShortWaves; ++i) {
    lo = fminf(lo, sh.wmm[i].x);
    m = fmaxf(m, sh.wmm[i].y);
  }
  double zt = 0.0;
#pragma unroll
  for (int u = 0; u < kShortPT; ++u) {
    w[u] = valid[u] ? weight(s[u], m) : 0.0f;
    zt += static_cast<double>(w[u]);
  }
  {
    const double zw = wave_sum_f64(zt);
    if (lane == 0) sh.wz[wave] = zw;
  }
  __syncthreads();
  double Z = 0.0;
  for (int i = 0; i < kShortWaves; ++i) Z += sh.wz[i];
  const double epsZ = eps * Z;

  // 3. The cut's range.  Level 0: kShortBins equal-width value bins over
  // [lo, m] (a bin is a contiguous range of the key order, so the descent
  // stays exact); then, while the range holds more than kShortFin keys, 8-bit
  // digits of key64 below the bits its keys share.  R and below are the mass
  // and count of the keys under the range.
  const float inv = lin_scale(lo, m) * (static_cast<float>(kShortBins) / static_cast<float>(kBins));
  int vb[kShortPT];
#pragma unroll
  for (int u = 0; u < kShortPT; ++u) {
    const float x = (s[u] - lo) * inv;
    vb[u] = x < static_cast<float>(kShortBins) ? static_cast<int>(x) : kShortBins - 1;
  }
  int b0 = -1;          // the level-0 bin of the range
  uint64_t prefix = 0ull;
  int plen = -1;        // key64 bits fixed below level 0 (-1: level 0 not done)
  double R = 0.0;
  uint32_t below = 0u;
  uint32_t cnt = static_cast<uint32_t>(n);
  auto in_range = [&](int u) -> bool {
    return valid[u] && (b0 < 0 || (vb[u] == b0 && prefix_is(key[u], prefix, plen)));
  };
  for (int guard = 0; guard < 10 && cnt > static_cast<uint32_t>(kShortFin); ++guard) {
    // One level: a (count, mass) histogram of the range, then the highest
    // non-empty bin whose lower bins keep R + mass <= epsZ.
    if (b0 >= 0) {
      // Skip the key bits the range's keys share.
      unsigned long long kmn = ~0ull, kmx = 0ull;
#pragma unroll
      for (int u = 0; u < kShortPT; ++u) {
        if (in_range(u)) {
          kmn = key[u] < kmn ? key[u] : kmn;
          kmx = key[u] > kmx ? key[u] : kmx;
        }
      }
      kmn = wave_pick_u64<false>(kmn);
      kmx = wave_pick_u64<true>(kmx);
      if (t == 0) {
        sh.kmin = ~0ull;
        sh.kmax = 0ull;
      }
      __syncthreads();
      if (lane == 0) {
        atomicMin(&sh.kmin, kmn);
        atomicMax(&sh.kmax, kmx);
      }
      __syncthreads();
      const uint64_t diff = static_cast<uint64_t>(sh.kmin) ^ static_cast<uint64_t>(sh.kmax);
      const int common = diff == 0ull ? 64 : __clzll(static_cast<long long>(diff));
      if (common > plen) {
        plen = min(common, 64 - kShortDigit);
        prefix = static_cast<uint64_t>(sh.kmin) >> (64 - plen);
      }
    }
    const int shift = 64 - plen - kShortDigit;
    if (t < kShortBins) {
      sh.hm[t] = 0.0;
      sh.hc[t] = 0u;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kShortPT; ++u) {
      if (in_range(u)) {
        const int b = b0 < 0 ? vb[u]
                             : static_cast<int>((key[u] >> shift) &
                                                static_cast<uint64_t>(kShortBins - 1));
        atomicAdd(&sh.hc[b], 1u);
        atomicAdd(&sh.hm[b], static_cast<double>(w[u]));
      }
    }
    __syncthreads();
    if (wave == 0) {
      double mb[4];
      uint32_t cb[4];
      double ms = 0.0;
      uint32_t cs = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        mb[j] = sh.hm[4 * lane + j];
        cb[j] = sh.hc[4 * lane + j];
        ms += mb[j];
        cs += cb[j];
      }
      const double im = wave_incl_scan_f64_dpp(ms);
      const uint32_t ic = wave_incl_scan_u32_dpp(cs);
      double e = __shfl_up(im, 1, kWave);
      uint32_t ec = __shfl_up(ic, 1, kWave);
      if (lane == 0) {
        e = 0.0;
        ec = 0u;
      }
      int mine = -1;
      double mS = 0.0;
      uint32_t mC = 0u, mN = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (cb[j] != 0u && R + e <= epsZ) {
          mine = 4 * lane + j;
          mS = e;
          mC = ec;
          mN = cb[j];
        }
        e += mb[j];
        ec += cb[j];
      }
      const uint64_t bal = __ballot(mine >= 0);
      if (bal == 0ull) {
        if (lane == 0) sh.best = -1;  // only with non-finite scores
      } else if (lane == 63 - __clzll(static_cast<long long>(bal))) {
        sh.best = mine;
        sh.selS = mS;
        sh.selC = mC;
        sh.selN = mN;
      }
    }
    __syncthreads();
    const int b = sh.best;
    if (b < 0) break;
    R += sh.selS;
    below += sh.selC;
    cnt = sh.selN;
    if (b0 < 0) {
      b0 = b;
      plen = 0;
    } else {
      prefix = (prefix << kShortDigit) | static_cast<uint64_t>(b);
      plen += kShortDigit;
    }
  }

  // 4. Finish: the range's keys in LDS; lane i of every wave holds candidate
  // i, wave g sums the weights of the candidates of its slice below it, and
  // wave 0 adds the slices in wave order.
  if (t == 0) {
    sh.ncand = 0u;
    sh.thr = 0ull;  // kept only if no candidate qualifies (non-finite scores)
    sh.finR = R;
    sh.finN = 0u;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kShortPT; ++u) {
    if (in_range(u)) {
      const uint32_t slot = atomicAdd(&sh.ncand, 1u);
      if (slot < static_cast<uint32_t>(kShortFin)) sh.cand[slot] = key[u];
    }
  }
  __syncthreads();
  const int c = static_cast<int>(min(sh.ncand, static_cast<uint32_t>(kShortFin)));
  const uint64_t ck = lane < c ? sh.cand[lane] : 0ull;
  {
    const int per = (c + kShortWaves - 1) / kShortWaves;
    const int j0 = wave * per, j1 = min(c, j0 + per);
    double lower = 0.0;
    uint32_t nlower = 0u;
    for (int j = j0; j < j1; ++j) {  // wave-uniform: LDS broadcast reads
      const uint64_t kj = sh.cand[j];
      if (kj < ck) {
        lower += static_cast<double>(weight(key64_score(kj), m));
        ++nlower;
      }
    }
    sh.u.fin.m[wave][lane] = lower;
    sh.u.fin.c[wave][lane] = nlower;
  }
  __syncthreads();
  if (wave == 0) {
    double L = 0.0;
    uint32_t N = 0u;
#pragma unroll
    for (int g = 0; g < kShortWaves; ++g) {
      L += sh.u.fin.m[g][lane];
      N += sh.u.fin.c[g][lane];
    }
    const bool ok = lane < c && R + L <= epsZ;
    const uint64_t best = wave_pick_u64<true>(ok ? ck : 0ull);
    if (ok && ck == best) {
      sh.thr = ck;
      sh.finR = R + L;
      sh.finN = N;
    }
  }
  __syncthreads();
  const uint64_t thr = sh.thr;
  const double Rf = sh.finR;
  below += sh.finN;
  const int nwords = (n + 31) / 32;
  uint32_t* mrow = sel_mask != nullptr ? sel_mask + static_cast<size_t>(row) * nwords : nullptr;
#pragma unroll
  for (int u = 0; u < kShortPT; ++u) {
    const int i = u * kShortThreads + t;
    const bool head = valid[u] && key[u] >= thr;
    sh.wh[i] = head ? w[u] : 0.0f;
    if (mrow != nullptr) {
      // Bit i % 32 of word i / 32: key i is in the head; wave w holds keys
      // u * kShortThreads + 64 w .. + 63 of slot u.
      const uint64_t bits = __ballot(head);
      const int w0 = (u * kShortThreads + wave * kWave) / 32;
      if (lane == 0 && w0 < nwords) mrow[w0] = static_cast<uint32_t>(bits);
      if (lane == 1 && w0 + 1 < nwords) mrow[w0 + 1] = static_cast<uint32_t>(bits >> 32);
    }
  }
  if (t == 0) {
    k_eps[row] = static_cast<int32_t>(static_cast<uint32_t>(n) - below);
    tau[row] = Rf / Z;
    if (lse != nullptr) lse[row] = static_cast<double>(m) + log(Z);
  }
  __syncthreads();

  // 5. Head-only output.  Lane (rg, seg) sums w v over its rows for the
  // columns seg * EPL .. seg * EPL + EPL - 1; only head rows are loaded.
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
  for (int it0 = 0; it0 < iters; it0 += kVBatch) {
    uint4 vv[kVBatch];
    float ww[kVBatch];
#pragma unroll
    for (int u = 0; u < kVBatch; ++u) {
      const int r = (it0 + u) * RPB + wave * RPW + rg;
      ww[u] = r < n ? sh.wh[r] : 0.0f;
      vv[u] = make_uint4(0u, 0u, 0u, 0u);
      if (ww[u] != 0.0f)
        vv[u] = load_stream16(V + kv_base + static_cast<size_t>(r) * D + seg * EPL);
    }
#pragma unroll
    for (int u = 0; u < kVBatch; ++u) {
      float x[EPL];
      Slice<T>::unpack(vv[u], x);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(ww[u], x[e], acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = stride_sum<LPR>(acc[e]);
  if (rg == 0) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) sh.u.red[wave][seg * EPL + e] = acc[e];
  }
  __syncthreads();
  if (t < D) {
    double num = 0.0;
#pragma unroll
    for (int g = 0; g < kShortWaves; ++g) num += static_cast<double>(sh.u.red[g][t]);
    const double den = Z - Rf;
    out[static_cast<size_t>(row) * D + t] = static_cast<float>(num / (den > 0.0 ? den : 1.0));
  }
}

template <typename T, int D>
hipError_t launch_t(const void* q, const void* K, const void* V, const float* head_scale,
                    float default_scale, int n, int n_q, int n_kv, double eps, float* out,
                    int32_t* k_eps, double* tau, double* lse, uint32_t* sel_mask, float* scores,
                    hipStream_t st) {
  return launch(short_row_kernel<T, D>, dim3(n_q), dim3(kShortThreads), 0, st,
                static_cast<const T*>(q), static_cast<const T*>(K), static_cast<const T*>(V),
                head_scale, default_scale, n, n_q / n_kv, eps, out, k_eps, tau, lse, sel_mask,
                scores);
}

}  // namespace

hipError_t launch_short_row(const void* q, const void* K, const void* V, int dtype, int d,
                            const float* head_scale, float default_scale, int64_t n, int n_q,
                            int n_kv, double eps, float* out, int32_t* k_eps, double* tau,
                            double* lse, uint32_t* sel_mask, float* scores, hipStream_t st) {
  if (n < 1 || n > kShortRowMaxN) return hipErrorInvalidValue;
  const int nn = static_cast<int>(n);
  if (dtype == 1) {
    if (d == 128)
      return launch_t<uint16_t, 128>(q, K, V, head_scale, default_scale, nn, n_q, n_kv, eps, out,
                                     k_eps, tau, lse, sel_mask, scores, st);
    return launch_t<uint16_t, 64>(q, K, V, head_scale, default_scale, nn, n_q, n_kv, eps, out,
                                  k_eps, tau, lse, sel_mask, scores, st);
  }
  if (d == 128)
    return launch_t<float, 128>(q, K, V, head_scale, default_scale, nn, n_q, n_kv, eps, out,
                                k_eps, tau, lse, sel_mask, scores, st);
  return launch_t<float, 64>(q, K, V, head_scale, default_scale, nn, n_q, n_kv, eps, out, k_eps,
                             tau, lse, sel_mask, scores, st);
}

}  // namespace ctopk
