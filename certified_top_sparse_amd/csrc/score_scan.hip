// K1 -- GQA-shared score scan.
//
// Computes s_i = scale_h * <q_h, k_i> for every key i of a KV head and every
// query head h of its group (the scores whose softmax is P in the Abstract of
// "A Mathematical Theory of Top-k Sparse Attention via Total Variation
// Distance", arXiv 2512.07647), and the (minimum, maximum) score of each tile
// of kScanTile keys.
//
// Memory plan (HBM-bound: one K row of d*esize bytes feeds G dot products):
//   * every K row is read from HBM exactly once per group of up to 8 query
//     heads, with 16-byte loads; LPR = d*esize/16 consecutive lanes cover one
//     row, so a wave64 load instruction reads 64/LPR whole rows (1 KiB,
//     fully coalesced);
//   * each lane keeps the matching 16-byte slice of every q_h in registers;
//     bf16 pairs use v_dot2_f32_bf16 (products exact in fp32, fp32 sum);
//   * one short block per tile (thousands of blocks, all loads of a wave
//     issued before any arithmetic, no branch around a load), so blocks in
//     different phases keep HBM busy;
//   * K of at most kScanCachedMax bytes is read with ordinary loads, larger K
//     with non-temporal ones (measured: at 64 MiB of K the ordinary loads take
//     the scan from 14.7 to 13.7 us; at 1 GiB they make it 180 -> 200 us and
//     slow the next kernel's reads of the scores, which they evict);
//   * the LPR partial dots are combined by DPP butterflies (full-rate VALU,
//     no LDS round trips), the scores are staged in LDS and written out
//     coalesced ([n_q_heads, n] fp32, 4*G bytes per key against d*esize bytes
//     of K read);

#include "kernels.h"
#include "scan_dot.h"

namespace ctopk {
namespace {

// One block per tile of kScanTile keys of one KV head and up to GB query
// heads: 4 waves, each covering kScanTile / 4 keys with all of its K loads
// issued before any arithmetic.
constexpr size_t kScanCachedMax = size_t(128) << 20;

template <typename T, int D, int GB, bool HS, bool NT>
__global__ __launch_bounds__(256) void score_scan_kernel(
    const T* __restrict__ q, const T* __restrict__ K, const float* __restrict__ head_scale,
    float default_scale, int64_t n, int G, int nblk, float* __restrict__ scores,
    float2* __restrict__ blkstat, float* __restrict__ blkz, void* zero_base, size_t zero_bytes,
    void* zero_base2, size_t zero_bytes2) {
  constexpr int EPL = Slice<T>::kElems;
  constexpr int LPR = D / EPL;
  constexpr int RPW = kWave / LPR;
  constexpr int WAVES = 4;
  constexpr int ITER = kScanTile / (WAVES * RPW);
  static_assert(GB <= LPR, "one lane per head within a row group");
  static_assert(kScanTile % kWave == 0, "tile is a whole number of waves");
  __shared__ float s_sc[GB][kScanTile];

  const int tile = blockIdx.x;
  const int kvh = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int seg = lane % LPR;
  const int rg = lane / LPR;
  const int h0 = kvh * G + blockIdx.z * GB;
  const int nh = min(GB, G - static_cast<int>(blockIdx.z) * GB);
  const int64_t tile0 = static_cast<int64_t>(tile) * kScanTile;
  const int lbase = wave * (ITER * RPW);

  // K rows first: they carry the block's HBM latency.  Rows past n re-read
  // row n-1 (their scores are never written), so the loads are unconditional.
  const T* Kb = K + static_cast<size_t>(kvh) * static_cast<size_t>(n) * D;
  uint4 kv[ITER];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int64_t r = min(tile0 + lbase + it * RPW + rg, n - 1);
    if constexpr (NT) {
      kv[it] = load_stream16(Kb + r * D + seg * EPL);
    } else {
      kv[it] = *reinterpret_cast<const uint4*>(Kb + r * D + seg * EPL);
    }
  }
  // q slices (head slots past nh repeat the last head and are never written).
  uint4 qv[GB];
  float sc[GB];
#pragma unroll
  for (int j = 0; j < GB; ++j) {
    const int hj = h0 + min(j, nh - 1);
    qv[j] = *reinterpret_cast<const uint4*>(q + static_cast<size_t>(hj) * D + seg * EPL);
    if constexpr (HS) {
      sc[j] = head_scale[hj];
    } else {
      sc[j] = default_scale;
    }
  }
  {
    const size_t bl = (static_cast<size_t>(blockIdx.z) * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
    const size_t nb = static_cast<size_t>(gridDim.x) * gridDim.y * gridDim.z;
    zero_slice(zero_base, zero_bytes, bl, nb);
    zero_slice(zero_base2, zero_bytes2, bl, nb);
  }

#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int lr = lbase + it * RPW + rg;
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      const float acc = group_sum<LPR>(Slice<T>::dot(kv[it], qv[j]));
      if (seg == j) s_sc[j][lr] = acc * sc[j];
    }
  }
  __syncthreads();

  // Wave w writes heads w, w + 4, ...: coalesced score stores and the tile's
  // (min, max) for that head.
  for (int j = wave; j < nh; j += WAVES) {
    float vmax = -INFINITY, vmin = INFINITY;
    float* srow = scores + static_cast<size_t>(h0 + j) * static_cast<size_t>(n);
#pragma unroll
    for (int k = lane; k < kScanTile; k += kWave) {
      const int64_t i = tile0 + k;
      if (i < n) {
        const float v = s_sc[j][k];
        srow[i] = v;
        vmax = fmaxf(vmax, v);
        vmin = fminf(vmin, v);
      }
    }
    vmax = wave_max_dpp(vmax);
    vmin = -wave_max_dpp(-vmin);
    if (lane == 0) blkstat[static_cast<size_t>(h0 + j) * nblk + tile] = make_float2(vmin, vmax);
    if (blkz != nullptr) {  // the tile's softmax mass relative to its maximum
      static_assert(kScanTile == kWave, "one key per lane");
      const int64_t i = tile0 + lane;
      const float z = group_sum<kWave>(i < n ? weight(s_sc[j][lane], vmax) : 0.0f);
      if (lane == 0) blkz[static_cast<size_t>(h0 + j) * nblk + tile] = z;
    }
  }
}

template <typename T, int D, int GB>
hipError_t launch_t(const void* q, const void* K, const float* head_scale, float default_scale,
                    int64_t n, int n_q, int n_kv, float* scores, float2* blkstat, float* blkz,
                    void* zb, size_t zbytes, void* zb2, size_t zbytes2, hipStream_t st) {
  const int G = n_q / n_kv;
  const int nblk = static_cast<int>(ceil_div(n, kScanTile));
  dim3 grid(nblk, n_kv, static_cast<unsigned>(ceil_div(G, GB)));
  const bool nt = static_cast<size_t>(n_kv) * static_cast<size_t>(n) * D * sizeof(T) >
                  kScanCachedMax;
#define CTOPK_SCAN_LAUNCH(HS, NT)                                                              \
  launch(score_scan_kernel<T, D, GB, HS, NT>, grid, dim3(256), 0, st,                       \
         static_cast<const T*>(q), static_cast<const T*>(K), head_scale, default_scale, n, G, \
         nblk, scores, blkstat, blkz, zb, zbytes, zb2, zbytes2)
  if (head_scale != nullptr)
    return nt ? CTOPK_SCAN_LAUNCH(true, true) : CTOPK_SCAN_LAUNCH(true, false);
  return nt ? CTOPK_SCAN_LAUNCH(false, true) : CTOPK_SCAN_LAUNCH(false, false);
#undef CTOPK_SCAN_LAUNCH
}

template <typename T, int D>
hipError_t launch_d(const void* q, const void* K, const float* hs, float ds, int64_t n, int n_q,
                    int n_kv, float* scores, float2* bs, float* bz, void* zb, size_t zbytes,
                    void* zb2, size_t zbytes2, hipStream_t st) {
  const int G = n_q / n_kv;
#define CTOPK_SCAN(GB) \
  launch_t<T, D, GB>(q, K, hs, ds, n, n_q, n_kv, scores, bs, bz, zb, zbytes, zb2, zbytes2, st)
  if (G == 1) return CTOPK_SCAN(1);
  if (G == 2) return CTOPK_SCAN(2);
  if (G <= 4) return CTOPK_SCAN(4);
  return CTOPK_SCAN(8);
#undef CTOPK_SCAN
}

}  // namespace

hipError_t launch_score_scan(const void* q, const void* K, int dtype, int d,
                             const float* head_scale, float default_scale, int64_t n, int n_q,
                             int n_kv, float* scores, float2* blkstat, float* blkz,
                             void* zero_base, size_t zero_bytes, void* zero_base2,
                             size_t zero_bytes2, hipStream_t st) {
  if (dtype == 1) {
    if (d == 128)
      return launch_d<uint16_t, 128>(q, K, head_scale, default_scale, n, n_q, n_kv, scores,
                                     blkstat, blkz, zero_base, zero_bytes, zero_base2, zero_bytes2, st);
    return launch_d<uint16_t, 64>(q, K, head_scale, default_scale, n, n_q, n_kv, scores, blkstat,
                                  blkz, zero_base, zero_bytes, zero_base2, zero_bytes2, st);
  }
  if (d == 128)
    return launch_d<float, 128>(q, K, head_scale, default_scale, n, n_q, n_kv, scores, blkstat,
                                blkz, zero_base, zero_bytes, zero_base2, zero_bytes2, st);
  return launch_d<float, 64>(q, K, head_scale, default_scale, n, n_q, n_kv, scores, blkstat, blkz,
                             zero_base, zero_bytes, zero_base2, zero_bytes2, st);
}

}  // namespace ctopk
