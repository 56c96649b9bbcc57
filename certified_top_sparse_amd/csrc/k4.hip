// 4-bit key copy and exact candidate generation from it.  Source: the page
// "Certified Sparse Attention via Perturbed Retrieval" (arXiv 2610.24991),
// Abstract -- its method passes over every key once in a 4-bit form whose
// score error is bounded deterministically, one pass serving all query heads
// of a grouped-query group, and recovers the exact candidate set; the
// paperfoot.com page on it ("Limitations and Discussion") gives that pass as a
// fixed fraction of dense attention's bytes.  Neither page prints a formula;
// this library's reading:
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
constexpr int kK4TilesPerWave = 1;  // 64-key tiles per wave of the 4-bit scan

template <int L>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (L >= 2) v = fmaxf(v, dpp<kDppXor1>(v));
  if constexpr (L >= 4) v = fmaxf(v, dpp<kDppXor2>(v));
  if constexpr (L >= 8) v = fmaxf(v, dpp<kDppHalfMirror>(v));
  if constexpr (L >= 16) v = fmaxf(v, dpp<kDppMirror>(v));
  if constexpr (L >= 32) v = fmaxf(v, xor_lane<16>(v));
  if constexpr (L >= 64) v = fmaxf(v, xor_lane<32>(v));
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
// The scan on MFMA: scores of up to 8 query heads against 16 keys per
// v_mfma_f32_16x16x32_bf16 group, rows = heads, columns = keys, k over d in
// blocks of 32 (A[i][k] in lane i + 16 (k / 8), B[k][j] in lane j + 16 (k / 8),
// D[i][j] in lane j + 16 (i / 4), element i % 4).  The order of k inside the
// product is free as long as both operands share it: in block kb, lane group
// g holds elements 8 KB g + 8 kb + t (t < 8), so one load of 4 KB bytes gives
// a lane its key's codes for every block.  A code c enters the product as
// the bf16 number 136 + c (0x4300 | (c + 8): exact, and made from the nibble
// with two bit operations), so the product is sum q (136 + c) and the dot is
// that minus 136 sum q.  One wave per 64-key tile; no LDS, no barrier.
// ---------------------------------------------------------------------------
typedef __bf16 k4_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float k4_f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

template <typename T, int D, int GB>
__global__ __launch_bounds__(256) void k4_scan_kernel(
    const T* __restrict__ q, const uint8_t* __restrict__ K4, const float* __restrict__ kscale,
    const float* __restrict__ kres, const float* __restrict__ head_scale, float default_scale,
    const float* __restrict__ thr, int64_t n, int G, int nblk, int nzb,
    uint32_t* __restrict__ mask, unsigned long long* __restrict__ smask,
    float2* __restrict__ bounds, int32_t* __restrict__ count, int32_t* __restrict__ rescored) {
  constexpr int KB = D / 32;           // k blocks
  constexpr int BPL = 4 * KB;          // code bytes per lane and key
  constexpr int GROUPS = kScanTile / 16;
  constexpr bool kSplit = sizeof(T) == 4;  // fp32 q: a high and a low bf16 part
  static_assert(GB <= 8, "heads are MFMA rows 0..7");
  static_assert(kScanTile == 64, "four 16-key groups per wave");
  __shared__ float s_dot[4][kScanTile * GB];  // wave-private
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int tile_first = (blockIdx.x * 4 + wave) * kK4TilesPerWave;
  if (tile_first >= nblk) return;  // whole wave; nothing below synchronises the block
  const int kvh = blockIdx.y;
  const int z = blockIdx.z;
  const int h0 = kvh * G + z * GB;
  const int nh = min(GB, G - z * GB);
  const int j = lane & 15;
  const int g = lane >> 4;
  const size_t kbase = static_cast<size_t>(kvh) * static_cast<size_t>(n);
  if (tile_first == 0) {  // the totals the rescoring adds to
    if (lane < nh) count[h0 + lane] = 0;
    if (lane == 0 && z == 0 && rescored != nullptr) rescored[kvh] = 0;
  }

  // All loads first: codes of group u's key tile0 + 16 u + j (bytes BPL g ..
  // BPL g + BPL - 1) and each key's scale and residual bound, per tile.
  uint32_t cw[kK4TilesPerWave][GROUPS][KB];
  float a_key[kK4TilesPerWave], rho_key[kK4TilesPerWave];
#pragma unroll
  for (int tt = 0; tt < kK4TilesPerWave; ++tt) {
    const int64_t tile0 = static_cast<int64_t>(tile_first + tt) * kScanTile;
#pragma unroll
    for (int u = 0; u < GROUPS; ++u) {
      const int64_t r = min(tile0 + 16 * u + j, n - 1);
      const uint8_t* src = K4 + (kbase + r) * (D / 2) + BPL * g;
      if constexpr (KB == 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(src);
        cw[tt][u][0] = v.x;
        cw[tt][u][1] = v.y;
        cw[tt][u][2] = v.z;
        cw[tt][u][3] = v.w;
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(src);
        cw[tt][u][0] = v.x;
        cw[tt][u][1] = v.y;
      }
    }
    const int64_t r = min(tile0 + lane, n - 1);
    a_key[tt] = kscale[kbase + r];
    rho_key[tt] = kres[kbase + r];
  }

  // Each head's scale and threshold (uniform loads, issued with the rest).
  float sc_h[GB], th_h[GB];
#pragma unroll
  for (int i = 0; i < GB; ++i) {
    const int hi = h0 + min(i, nh - 1);
    sc_h[i] = head_scale != nullptr ? head_scale[hi] : default_scale;
    th_h[i] = thr[hi];
  }

  // A operands: row i = lane & 15 is head h0 + i (zero past nh), its elements
  // 8 KB g + 8 kb .. + 7 for block kb; per-row sums for the offset and norms.
  const int i_row = lane & 15;
  const bool row_live = i_row < nh;
  uint4 ah[KB], al[KB];
  float qs = 0.0f, q1 = 0.0f, q2 = 0.0f;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const T* src = q + static_cast<size_t>(h0 + min(i_row, nh - 1)) * D + 8 * KB * g + 8 * kb;
    float x[8];
    if constexpr (kSplit) {
      const uint4 v0 = *reinterpret_cast<const uint4*>(src);
      const uint4 v1 = *reinterpret_cast<const uint4*>(src + 4);
      const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int t = 0; t < 8; ++t) x[t] = row_live ? __uint_as_float(w[t]) : 0.0f;
      uint32_t hw[4] = {0u, 0u, 0u, 0u}, lw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t bh = bf16_rne_bits(x[t]);
        const float xh = __uint_as_float(bh << 16);
        const uint32_t bl = bf16_rne_bits(x[t] - xh);
        hw[t / 2] |= bh << (16 * (t & 1));
        lw[t / 2] |= bl << (16 * (t & 1));
        qs += xh + __uint_as_float(bl << 16);
      }
      ah[kb] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      al[kb] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    } else {
      uint4 v = *reinterpret_cast<const uint4*>(src);
      if (!row_live) v = make_uint4(0u, 0u, 0u, 0u);
      Slice<uint16_t>::unpack(v, x);
      ah[kb] = v;
      al[kb] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int t = 0; t < 8; ++t) qs += x[t];
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      q1 += fabsf(x[t]);
      q2 = fmaf(x[t], x[t], q2);
    }
  }
  // row totals over the four lane groups (lanes i, i + 16, i + 32, i + 48)
  qs = xrow32_sum(xrow16_sum(qs));
  q1 = xrow32_sum(xrow16_sum(q1));
  q2 = xrow32_sum(xrow16_sum(q2));

#pragma unroll
  for (int tt = 0; tt < kK4TilesPerWave; ++tt) {
    const int tile = tile_first + tt;
    if (tile >= nblk) break;  // uniform
    const int64_t tile0 = static_cast<int64_t>(tile) * kScanTile;
    k4_f32x4_t acc[GROUPS];
#pragma unroll
    for (int u = 0; u < GROUPS; ++u) {
      acc[u] = k4_f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const uint32_t w = cw[tt][u][kb] ^ 0x88888888u;  // nibbles c + 8
        const uint32_t lo = w & 0x0F0F0F0Fu;                // elements 0, 2, 4, 6 (one a byte)
        const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;         // elements 1, 3, 5, 7
        uint32_t b[4];
#pragma unroll
        for (int p = 0; p < 4; ++p)  // bytes [lo_p, 0, hi_p, 0], then the bf16 exponent byte
          b[p] = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u + 0x00010001u * p) | 0x43004300u;
        const k4_bf16x8_t bv = __builtin_bit_cast(k4_bf16x8_t, make_uint4(b[0], b[1], b[2], b[3]));
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(k4_bf16x8_t, ah[kb]), bv,
                                                         acc[u], 0, 0, 0);
        if constexpr (kSplit)
          acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(k4_bf16x8_t, al[kb]), bv,
                                                           acc[u], 0, 0, 0);
      }
    }

    // The dots to one key per lane: lane j + 16 hq holds heads 4 hq + e of keys
    // 16 u + j; through wave-private LDS each lane takes key `lane`, all heads.
    float* sd = s_dot[wave];
#pragma unroll
    for (int u = 0; u < GROUPS; ++u) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * (lane >> 4) + e;
        if (i < GB) sd[(16 * u + j) * GB + i] = acc[u][e];
      }
    }
    __builtin_amdgcn_wave_barrier();  // LDS operations of one wave complete in order
    const int64_t key = tile0 + lane;
    const bool real = key < n;
    const float a = a_key[tt];
    const float rho = rho_key[tt];
    const int64_t nwords = ceil_div(n, 32);
    uint64_t any_str = 0ull;
#pragma unroll
    for (int i = 0; i < GB; ++i) {
      if (i < nh) {  // uniform
        // head i's constants, from row lane i (uniform values)
        const float Si = readlane_f(qs, i);
        const float n1 = readlane_f(q1, i);
        const float n2 = readlane_f(q2, i);
        const float sci = sc_h[i];
        const float as = fabsf(sci);
        const float b2 = as * sqrtf(n2) * 1.00001f;
        // rounding of the 4-bit product (terms q (136 + c) and 136 sum q) and of
        // the full-width dot (|k| <= 7 a); fp32 q: its low part's own rounding
        const float b1 = as * n1 *
                         ((429.0f * static_cast<float>(D + 4)) * 5.9604645e-8f +
                          (kSplit ? 7.0f * 7.6293945e-6f : 0.0f)) * 1.00001f;
        const float th = th_h[i];
        const float dot = sd[lane * GB + i] - 136.0f * Si;
        const float shat = (sci * dot) * a;
        const float R = (b2 * rho + b1 * a + fabsf(shat) * 4.7683716e-7f) * 1.000001f;
        const float lo = shat - R, hi = shat + R;
        const bool in = real && lo >= th;
        const bool strad = real && !(lo >= th) && !(hi < th);
        const uint64_t bi = __ballot(in);
        any_str |= __ballot(strad);
        uint32_t* mrow = mask + static_cast<size_t>(h0 + i) * static_cast<size_t>(nwords);
        if (lane == 0) mrow[2 * tile] = static_cast<uint32_t>(bi);
        if (lane == 1 && 2 * tile + 1 < nwords) mrow[2 * tile + 1] = static_cast<uint32_t>(bi >> 32);
        if (bounds != nullptr && real)
          bounds[static_cast<size_t>(h0 + i) * static_cast<size_t>(n) + key] = make_float2(lo, hi);
      }
    }
    if (lane == 0) smask[(static_cast<size_t>(kvh) * nzb + z) * nblk + tile] = any_str;
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
    const unsigned long long* __restrict__ smask, uint32_t* __restrict__ mask,
    int32_t* __restrict__ count, int32_t* __restrict__ rescored) {
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
  if (nkeys > 0 && wave < kRescoreTiles / 2) {
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
  constexpr int UNROLL = 8;  // rows in flight per lane
  for (int base = wave * RPW; base < nkeys; base += WAVES * RPW * UNROLL) {  // none when nothing straddles
    uint4 kv[UNROLL];
    int key[UNROLL];
#pragma unroll
    for (int it = 0; it < UNROLL; ++it) {
      const int e = base + it * WAVES * RPW + rg;
      key[it] = e < nkeys ? s_keys[e] : -1;
      kv[it] = load_stream16(Kb + static_cast<size_t>(max(key[it], 0)) * D + seg * EPL);
    }
#pragma unroll
    for (int it = 0; it < UNROLL; ++it) {
#pragma unroll
      for (int j = 0; j < GB; ++j) {
        const float acc = group_sum<LPR>(Slice<T>::dot(kv[it], qv[j]));
        const float s = acc * sc[j];
        if (key[it] >= 0 && seg == j && j < nh && s >= th[j]) {
          const int local = key[it] - tile0 * kScanTile;
          atomicOr(&s_bits[j][local >> 5], 1u << (local & 31));
        }
      }
    }
  }
  __syncthreads();
  // Merge into the mask words of the tiles that had straddling keys (this
  // block owns those words for its heads), and count the chunk's candidates
  // per head and its rescored keys (integer atomics onto totals the scan
  // zeroed, so the sums are exact whatever the order).
  const int64_t nwords = ceil_div(n, 32);
  uint32_t c = 0u;
  if (t < nh * 2 * kRescoreTiles) {
    const int j = t / (2 * kRescoreTiles);
    const int w = t % (2 * kRescoreTiles);
    const int u = w / 2;
    const int64_t word = static_cast<int64_t>(tile0) * 2 + w;
    if (u < ntiles && word < nwords) {
      uint32_t* p = mask + static_cast<size_t>(h0 + j) * static_cast<size_t>(nwords) + word;
      uint32_t v = *p;
      if (s_tm[u] != 0ull) {
        v |= s_bits[j][w];
        *p = v;
      }
      c = static_cast<uint32_t>(__popc(v));
    }
  }
  static_assert(2 * kRescoreTiles == 16, "one head's words fill a 16-lane row");
  c = static_cast<uint32_t>(group_sum<16>(static_cast<float>(c)));  // <= 512: exact in fp32
  if (t < nh * 2 * kRescoreTiles && (t & 15) == 0) atomicAdd(&count[h0 + t / 16], static_cast<int32_t>(c));
  if (t == 0 && rescored != nullptr && nkeys > 0) atomicAdd(&rescored[kvh], nkeys);
}

template <typename T, int D, int GB>
hipError_t launch_k4_t(const void* q, const void* K, const uint8_t* K4, const float* ks,
                       const float* kr, const float* hs, float ds, const float* thr, int64_t n,
                       int n_q, int n_kv, uint32_t* mask, int32_t* count, int32_t* rescored,
                       float2* bounds, unsigned long long* smask, hipStream_t st) {
  const int G = n_q / n_kv;
  const int nblk = static_cast<int>(ceil_div(n, kScanTile));
  const int nzb = static_cast<int>(ceil_div(G, GB));
  hipError_t e = launch(k4_scan_kernel<T, D, GB>,
                        dim3(static_cast<unsigned>(ceil_div(nblk, 4 * kK4TilesPerWave)), n_kv, nzb),
                        dim3(256), 0, st,
                        static_cast<const T*>(q), K4, ks, kr, hs, ds, thr, n, G, nblk, nzb, mask,
                        smask, bounds, count, rescored);
  if (e != hipSuccess) return e;
  e = launch(k4_rescore_kernel<T, D, GB>,
             dim3(static_cast<unsigned>(ceil_div(nblk, kRescoreTiles)), n_kv, nzb), dim3(256), 0,
             st, static_cast<const T*>(q), static_cast<const T*>(K), hs, ds, thr, n, G, nblk, nzb,
             static_cast<const unsigned long long*>(smask), mask, count, rescored);
  return e;
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
