// 4-bit key copy with deterministic score bounds, shared across a GQA group,
// and exact candidate generation from it ("Certified Sparse Attention via
// Perturbed Retrieval", arXiv 2610.24991, Abstract: the scan generates the
// candidates exactly while reading every key; the paperfoot.com page on it,
// "Limitations and Discussion": the 4-bit scan is a fixed share of the bytes
// of dense attention).  The pages print no formula; this library's reading:
//
//   copy     per key: a = amax / 7 and codes c = clamp(rint(k / a), -7, 7) in
//            fp32 (two's-complement nibbles, element 2j in the low half of
//            byte j), and rho >= ||k - a c||_2 (rounded up);
//   bounds   s = scale (q . k) lies within R of shat = scale a (q . c), with
//            R = |scale| ||q||_2 rho (Cauchy-Schwarz on the residual) plus the
//            rounding of both fp32 dot products (the 4-bit one here and the
//            exact one of the score scan);
//   exact    for per-head thresholds T the candidates are {i : s_i >= T},
//            with s the library's fp32 score: keys whose interval lies at or
//            above T are in, keys whose interval lies below T are out, and
//            only the keys whose interval straddles T have their full-width
//            row read and scored (the score scan's arithmetic, so the set
//            matches a threshold on the score scan's scores bit for bit).
//
// Bytes per key of the scan: d / 2 code bytes plus 8 (scale and residual
// bound), against 2d for bf16 keys: 72 of 256 at d = 128.
#include <cfloat>

#include "kernels.h"
#include "scan_dot.h"

namespace ctopk {
namespace {

constexpr int kLevel = 7;

template <int L>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (L >= 2) v = fmaxf(v, dpp<kDppXor1>(v));
  if constexpr (L >= 4) v = fmaxf(v, dpp<kDppXor2>(v));
  if constexpr (L >= 8) v = fmaxf(v, dpp<kDppHalfMirror>(v));
  if constexpr (L >= 16) v = fmaxf(v, dpp<kDppMirror>(v));
  if constexpr (L >= 32) v = fmaxf(v, __shfl_xor(v, 16, 64));
  if constexpr (L >= 64) v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

// ---------------------------------------------------------------------------
// The copy: LPR lanes per key row, one 16-byte slice each; 4 waves per block.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void quantize_k4_kernel(const T* __restrict__ K, int64_t rows,
                                                          uint8_t* __restrict__ K4,
                                                          float* __restrict__ kscale,
                                                          float* __restrict__ kres) {
  constexpr int EPL = Slice<T>::kElems;
  constexpr int LPR = D / EPL;
  constexpr int RPW = kWave / LPR;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int seg = lane % LPR;
  const int64_t r = (static_cast<int64_t>(blockIdx.x) * 4 + wave) * RPW + lane / LPR;
  const bool live = r < rows;
  const int64_t rr = live ? r : rows - 1;
  float x[EPL];
  Slice<T>::unpack(*reinterpret_cast<const uint4*>(K + rr * D + seg * EPL), x);
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(x[e]));
  amax = group_max<LPR>(amax);
  const float a = __fdiv_rn(amax, static_cast<float>(kLevel));
  uint32_t packed = 0u;
  float ss = 0.0f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    float c = 0.0f;
    if (a > 0.0f) c = fminf(fmaxf(rintf(__fdiv_rn(x[e], a)), -static_cast<float>(kLevel)), static_cast<float>(kLevel));
    packed |= (static_cast<uint32_t>(static_cast<int>(c)) & 0xFu) << (4 * e);
    const float res = fmaf(-a, c, x[e]);  // one rounding of the exact residual
    ss = fmaf(res, res, ss);
  }
  ss = group_sum<LPR>(ss);
  if (live) {
    uint8_t* dst = K4 + r * (D / 2) + seg * (EPL / 2);
    if constexpr (EPL == 8) {
      *reinterpret_cast<uint32_t*>(dst) = packed;
    } else {
      *reinterpret_cast<uint16_t*>(dst) = static_cast<uint16_t>(packed);
    }
    if (seg == 0) {
      kscale[r] = a;
      // an upper bound: the fp32 sum of squares and the root are within a few
      // units in the last place, far inside the 1e-5 margin
      kres[r] = nextafterf(sqrtf(ss) * 1.00001f, INFINITY);
    }
  }
}

template <typename T, int D>
hipError_t launch_quantize_d(const void* K, int64_t rows, uint8_t* K4, float* ks, float* kr,
                             hipStream_t st) {
  constexpr int RPB = 4 * (kWave / (D / Slice<T>::kElems));
  return launch(quantize_k4_kernel<T, D>, dim3(static_cast<unsigned>(ceil_div(rows, RPB))),
                dim3(256), 0, st, static_cast<const T*>(K), rows, K4, ks, kr);
}

// ---------------------------------------------------------------------------
// The scan: one block per (64-key tile, KV head, up to GB query heads).
// D / 8 lanes per key, each with 8 codes (4 bytes) and the matching 8 fp32
// elements of every q_h of the block.
// ---------------------------------------------------------------------------
template <typename T, int D, int GB>
__global__ __launch_bounds__(256) void k4_scan_kernel(
    const T* __restrict__ q, const uint8_t* __restrict__ K4, const float* __restrict__ kscale,
    const float* __restrict__ kres, const float* __restrict__ head_scale, float default_scale,
    const float* __restrict__ thr, int64_t n, int G, int nblk, int nzb,
    uint32_t* __restrict__ mask, unsigned long long* __restrict__ smask,
    float2* __restrict__ bounds) {
  constexpr int CPL = 8;              // codes per lane
  constexpr int LPR = D / CPL;        // lanes per key
  constexpr int RPW = kWave / LPR;    // keys per wave and step
  constexpr int WAVES = 4;
  constexpr int ITER = kScanTile / (WAVES * RPW);
  static_assert(GB <= LPR, "one lane per head within a key's lanes");
  static_assert(kScanTile == kWave, "one key per lane in the classification");
  __shared__ float s_dot[GB][kScanTile];
  __shared__ float s_a[kScanTile], s_rho[kScanTile];
  __shared__ uint32_t s_str[GB][2];

  const int tile = blockIdx.x;
  const int kvh = blockIdx.y;
  const int z = blockIdx.z;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int seg = lane % LPR;
  const int rg = lane / LPR;
  const int h0 = kvh * G + z * GB;
  const int nh = min(GB, G - z * GB);
  const int64_t tile0 = static_cast<int64_t>(tile) * kScanTile;
  const int lbase = wave * (ITER * RPW);
  const size_t kbase = static_cast<size_t>(kvh) * static_cast<size_t>(n);

  // Codes first (rows past n re-read row n - 1 and are never classified).
  uint32_t cw[ITER];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int64_t r = min(tile0 + lbase + it * RPW + rg, n - 1);
    cw[it] = *reinterpret_cast<const uint32_t*>(K4 + (kbase + r) * (D / 2) + seg * (CPL / 2));
  }
  if (wave == 0) {
    const int64_t r = min(tile0 + lane, n - 1);
    s_a[lane] = kscale[kbase + r];
    s_rho[lane] = kres[kbase + r];
  }
  // q slices in fp32, and per head |scale| ||q||_2 and the dot products'
  // rounding allowance.
  float qv[GB][CPL];
  float sc[GB], b2[GB], b1[GB];
#pragma unroll
  for (int j = 0; j < GB; ++j) {
    const int hj = h0 + min(j, nh - 1);
    const T* qs = q + static_cast<size_t>(hj) * D + seg * CPL;
    float n1 = 0.0f, n2 = 0.0f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      float v;
      if constexpr (sizeof(T) == 2) {
        v = __uint_as_float(static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(qs)[e]) << 16);
      } else {
        v = reinterpret_cast<const float*>(qs)[e];
      }
      qv[j][e] = v;
      n1 += fabsf(v);
      n2 = fmaf(v, v, n2);
    }
    n1 = group_sum<LPR>(n1);
    n2 = group_sum<LPR>(n2);
    sc[j] = head_scale != nullptr ? head_scale[hj] : default_scale;
    const float as = fabsf(sc[j]);
    b2[j] = as * sqrtf(n2) * 1.00001f;
    // |fl(dot) - dot| <= (steps) 2^-24 sum |q_e c_e| <= (D + 4) 2^-24 * 7 ||q||_1 * a,
    // once for the 4-bit dot and once for the full-width one (amax = 7 a)
    b1[j] = as * n1 * (2.0f * kLevel * static_cast<float>(D + 4) * 5.9604645e-8f) * 1.00001f;
  }

#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    float c[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e)
      c[e] = static_cast<float>(static_cast<int>(cw[it] << (28 - 4 * e)) >> 28);  // nibble e, signed
    const int lr = lbase + it * RPW + rg;
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      float acc = 0.0f;
#pragma unroll
      for (int e = 0; e < CPL; ++e) acc = fmaf(qv[j][e], c[e], acc);
      acc = group_sum<LPR>(acc);
      if (seg == j) s_dot[j][lr] = acc;
    }
  }
  __syncthreads();

  // Wave w classifies heads w, w + 4, ...: one key per lane.
  const int64_t i = tile0 + lane;
  const bool real = i < n;
  const int64_t nwords = ceil_div(n, 32);
  for (int j = wave; j < nh; j += WAVES) {
    const float a = s_a[lane];
    const float shat = (sc[j] * s_dot[j][lane]) * a;
    // plus the roundings of the two products and of R itself
    const float R = (b2[j] * s_rho[lane] + b1[j] * a + fabsf(shat) * 4.7683716e-7f) * 1.000001f;
    const float lo = shat - R, hi = shat + R;
    const float th = thr[h0 + j];
    const bool in = real && lo >= th;
    const bool straddle = real && !(lo >= th) && !(hi < th);
    const uint64_t bin = __ballot(in);
    const uint64_t bst = __ballot(straddle);
    uint32_t* mrow = mask + static_cast<size_t>(h0 + j) * static_cast<size_t>(nwords);
    if (lane == 0) mrow[2 * tile] = static_cast<uint32_t>(bin);
    if (lane == 1 && 2 * tile + 1 < nwords) mrow[2 * tile + 1] = static_cast<uint32_t>(bin >> 32);
    if (lane == 0) {
      s_str[j][0] = static_cast<uint32_t>(bst);
      s_str[j][1] = static_cast<uint32_t>(bst >> 32);
    }
    if (bounds != nullptr && real)
      bounds[static_cast<size_t>(h0 + j) * static_cast<size_t>(n) + i] = make_float2(lo, hi);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t any = 0ull;
    for (int j = 0; j < nh; ++j)
      any |= static_cast<uint64_t>(s_str[j][0]) | (static_cast<uint64_t>(s_str[j][1]) << 32);
    smask[(static_cast<size_t>(kvh) * nzb + z) * nblk + tile] = any;
  }
}

// ---------------------------------------------------------------------------
// The rescoring: one block per (chunk of kRescoreTiles tiles, KV head, head
// block).  The straddling keys of the chunk are listed in key order, their
// full-width rows read (the score scan's lane layout and arithmetic), and
// each head's bit set where s >= T.
// ---------------------------------------------------------------------------
constexpr int kRescoreTiles = 8;

template <typename T, int D, int GB>
__global__ __launch_bounds__(256) void k4_rescore_kernel(
    const T* __restrict__ q, const T* __restrict__ K, const float* __restrict__ head_scale,
    float default_scale, const float* __restrict__ thr, int64_t n, int G, int nblk, int nzb,
    const unsigned long long* __restrict__ smask, uint32_t* __restrict__ mask) {
  constexpr int EPL = Slice<T>::kElems;
  constexpr int LPR = D / EPL;
  constexpr int RPW = kWave / LPR;
  constexpr int WAVES = 4;
  constexpr int CAP = kRescoreTiles * kScanTile;
  static_assert(GB <= LPR, "one lane per head within a key's lanes");
  __shared__ int s_keys[CAP];
  __shared__ uint32_t s_bits[GB][2 * kRescoreTiles];
  __shared__ unsigned long long s_tm[kRescoreTiles];
  __shared__ int s_off[kRescoreTiles + 1];

  const int chunk = blockIdx.x;
  const int kvh = blockIdx.y;
  const int z = blockIdx.z;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int t = threadIdx.x;
  const int h0 = kvh * G + z * GB;
  const int nh = min(GB, G - z * GB);
  const int tile0 = chunk * kRescoreTiles;
  const int ntiles = min(kRescoreTiles, nblk - tile0);

  // The chunk's straddle masks and their key lists, in key order.
  if (t < kRescoreTiles) {
    s_tm[t] = t < ntiles ? smask[(static_cast<size_t>(kvh) * nzb + z) * nblk + tile0 + t] : 0ull;
  }
  if (t < GB * 2 * kRescoreTiles) s_bits[t / (2 * kRescoreTiles)][t % (2 * kRescoreTiles)] = 0u;
  __syncthreads();
  if (t == 0) {
    int o = 0;
    for (int u = 0; u < kRescoreTiles; ++u) {
      s_off[u] = o;
      o += __popcll(s_tm[u]);
    }
    s_off[kRescoreTiles] = o;
  }
  __syncthreads();
  const int nkeys = s_off[kRescoreTiles];
  if (nkeys == 0) return;  // uniform: nothing straddles in this chunk
  if (wave < kRescoreTiles / 2) {
    // wave w lists tiles 2w and 2w + 1: lane l of tile u writes its key if set
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int u = 2 * wave + h;
      const uint64_t m = s_tm[u];
      if ((m >> lane) & 1ull) {
        const int rank = __popcll(m & ((1ull << lane) - 1ull));
        s_keys[s_off[u] + rank] = (tile0 + u) * kScanTile + lane;
      }
    }
  }
  // q slices (the score scan's layout) and scales.
  uint4 qv[GB];
  float sc[GB], th[GB];
  const int seg = lane % LPR;
  const int rg = lane / LPR;
#pragma unroll
  for (int j = 0; j < GB; ++j) {
    const int hj = h0 + min(j, nh - 1);
    qv[j] = *reinterpret_cast<const uint4*>(q + static_cast<size_t>(hj) * D + seg * EPL);
    sc[j] = head_scale != nullptr ? head_scale[hj] : default_scale;
    th[j] = thr[hj];
  }
  __syncthreads();

  const T* Kb = K + static_cast<size_t>(kvh) * static_cast<size_t>(n) * D;
  for (int base = wave * RPW; base < nkeys; base += WAVES * RPW) {
    const int e = base + rg;
    const bool live = e < nkeys;
    const int key = s_keys[live ? e : nkeys - 1];
    const uint4 kv = load_stream16(Kb + static_cast<size_t>(key) * D + seg * EPL);
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      const float acc = group_sum<LPR>(Slice<T>::dot(kv, qv[j]));
      const float s = acc * sc[j];
      if (live && seg == j && j < nh && s >= th[j]) {
        const int local = key - tile0 * kScanTile;
        atomicOr(&s_bits[j][local >> 5], 1u << (local & 31));
      }
    }
  }
  __syncthreads();
  // Merge into the mask words of the tiles that had straddling keys (this
  // block owns those words for its heads).
  const int64_t nwords = ceil_div(n, 32);
  if (t < nh * 2 * kRescoreTiles) {
    const int j = t / (2 * kRescoreTiles);
    const int w = t % (2 * kRescoreTiles);
    const int u = w / 2;
    const int64_t word = static_cast<int64_t>(tile0) * 2 + w;
    if (u < ntiles && s_tm[u] != 0ull && word < nwords) {
      uint32_t* p = mask + static_cast<size_t>(h0 + j) * static_cast<size_t>(nwords) + word;
      *p = *p | s_bits[j][w];
    }
  }
}

// ---------------------------------------------------------------------------
// Counts: blocks [0, n_q) popcount a head's mask row; blocks [n_q, n_q + n_kv)
// count a KV head's rescored keys (over its head blocks).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k4_count_kernel(const uint32_t* __restrict__ mask,
                                                       const unsigned long long* __restrict__ smask,
                                                       int64_t nwords, int n_q, int nblk, int nzb,
                                                       int32_t* __restrict__ count,
                                                       int32_t* __restrict__ rescored) {
  __shared__ int s_w[4];
  const int b = blockIdx.x;
  int c = 0;
  if (b < n_q) {
    const uint32_t* row = mask + static_cast<size_t>(b) * static_cast<size_t>(nwords);
    for (int64_t w = threadIdx.x; w < nwords; w += 256) c += __popc(row[w]);
  } else {
    const unsigned long long* row = smask + static_cast<size_t>(b - n_q) * nzb * nblk;
    for (int64_t w = threadIdx.x; w < static_cast<int64_t>(nzb) * nblk; w += 256) c += __popcll(row[w]);
  }
  c = static_cast<int>(wave_sum_u32(static_cast<uint32_t>(c)));
  if ((threadIdx.x & (kWave - 1)) == 0) s_w[threadIdx.x / kWave] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int tot = s_w[0] + s_w[1] + s_w[2] + s_w[3];
    if (b < n_q) {
      count[b] = tot;
    } else if (rescored != nullptr) {
      rescored[b - n_q] = tot;
    }
  }
}

template <typename T, int D, int GB>
hipError_t launch_k4_t(const void* q, const void* K, const uint8_t* K4, const float* ks,
                       const float* kr, const float* hs, float ds, const float* thr, int64_t n,
                       int n_q, int n_kv, uint32_t* mask, int32_t* count, int32_t* rescored,
                       float2* bounds, unsigned long long* smask, hipStream_t st) {
  const int G = n_q / n_kv;
  const int nblk = static_cast<int>(ceil_div(n, kScanTile));
  const int nzb = static_cast<int>(ceil_div(G, GB));
  hipError_t e = launch(k4_scan_kernel<T, D, GB>, dim3(nblk, n_kv, nzb), dim3(256), 0, st,
                        static_cast<const T*>(q), K4, ks, kr, hs, ds, thr, n, G, nblk, nzb, mask,
                        smask, bounds);
  if (e != hipSuccess) return e;
  e = launch(k4_rescore_kernel<T, D, GB>,
             dim3(static_cast<unsigned>(ceil_div(nblk, kRescoreTiles)), n_kv, nzb), dim3(256), 0,
             st, static_cast<const T*>(q), static_cast<const T*>(K), hs, ds, thr, n, G, nblk, nzb,
             static_cast<const unsigned long long*>(smask), mask);
  if (e != hipSuccess) return e;
  return launch(k4_count_kernel, dim3(n_q + n_kv), dim3(256), 0, st,
                static_cast<const uint32_t*>(mask), static_cast<const unsigned long long*>(smask),
                ceil_div(n, 32), n_q, nblk, nzb, count, rescored);
}

template <typename T, int D>
hipError_t launch_k4_d(const void* q, const void* K, const uint8_t* K4, const float* ks,
                       const float* kr, const float* hs, float ds, const float* thr, int64_t n,
                       int n_q, int n_kv, uint32_t* mask, int32_t* count, int32_t* rescored,
                       float2* bounds, unsigned long long* smask, hipStream_t st) {
  const int G = n_q / n_kv;
#define CTOPK_K4(GB)                                                                            \
  launch_k4_t<T, D, GB>(q, K, K4, ks, kr, hs, ds, thr, n, n_q, n_kv, mask, count, rescored, bounds, \
                        smask, st)
  if (G == 1) return CTOPK_K4(1);
  if (G == 2) return CTOPK_K4(2);
  if (G <= 4) return CTOPK_K4(4);
  return CTOPK_K4(8);
#undef CTOPK_K4
}

}  // namespace

int k4_head_blocks(int group) { return group <= 8 ? 1 : static_cast<int>(ceil_div(group, 8)); }

hipError_t launch_quantize_k4(const void* K, int dtype, int d, int64_t rows, uint8_t* K4,
                              float* kscale, float* kres, hipStream_t st) {
  if (dtype == 1)
    return d == 128 ? launch_quantize_d<uint16_t, 128>(K, rows, K4, kscale, kres, st)
                    : launch_quantize_d<uint16_t, 64>(K, rows, K4, kscale, kres, st);
  return d == 128 ? launch_quantize_d<float, 128>(K, rows, K4, kscale, kres, st)
                  : launch_quantize_d<float, 64>(K, rows, K4, kscale, kres, st);
}

hipError_t launch_candidates_k4(const void* q, const void* K, int dtype, int d, const uint8_t* K4,
                                const float* kscale, const float* kres, const float* head_scale,
                                float default_scale, const float* thr, int64_t n, int n_q,
                                int n_kv, uint32_t* mask, int32_t* count, int32_t* rescored,
                                float2* bounds, void* straddle, hipStream_t st) {
  auto* sm = static_cast<unsigned long long*>(straddle);
  if (dtype == 1)
    return d == 128 ? launch_k4_d<uint16_t, 128>(q, K, K4, kscale, kres, head_scale, default_scale,
                                                 thr, n, n_q, n_kv, mask, count, rescored, bounds, sm, st)
                    : launch_k4_d<uint16_t, 64>(q, K, K4, kscale, kres, head_scale, default_scale,
                                                thr, n, n_q, n_kv, mask, count, rescored, bounds, sm, st);
  return d == 128 ? launch_k4_d<float, 128>(q, K, K4, kscale, kres, head_scale, default_scale, thr,
                                            n, n_q, n_kv, mask, count, rescored, bounds, sm, st)
                  : launch_k4_d<float, 64>(q, K, K4, kscale, kres, head_scale, default_scale, thr, n,
                                           n_q, n_kv, mask, count, rescored, bounds, sm, st);
}

}  // namespace ctopk
