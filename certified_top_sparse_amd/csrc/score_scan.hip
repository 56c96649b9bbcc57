// K1 -- GQA-shared score scan.
//
// Computes s_i = scale_h * <q_h, k_i> for every key i of a KV head and every
// query head h of its group (the scores whose softmax is P in the Abstract of
// "A Mathematical Theory of Top-k Sparse Attention via Total Variation
// Distance", arXiv 2512.07647), and the maximum score of each tile of
// kScanTile keys.
//
// Memory plan (HBM-bound: one K row of d*esize bytes feeds G dot products):
//   * every K row is read from HBM exactly once per group of up to 8 query
//     heads, with 16-byte loads; LPR = d*esize/16 consecutive lanes cover one
//     row, so a wave64 load instruction reads 64/LPR whole rows (1 KiB,
//     fully coalesced);
//   * each lane keeps the matching 16-byte slice of every q_h in registers;
//     bf16 pairs use v_dot2_f32_bf16 (products exact in fp32, fp32 sum);
//   * the LPR partial dots are combined by an xor butterfly, the scores are
//     staged in LDS and written out coalesced ([n_q_heads, n] fp32, 4*G bytes
//     per key against d*esize bytes of K read).
#include "kernels.h"

namespace ctopk {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <typename T>
struct Slice;

// bf16: 8 elements per 16-byte slice, dot2 on packed pairs.
template <>
struct Slice<uint16_t> {
  static constexpr int kElems = 8;
  __device__ static __forceinline__ float dot(const uint4& k, const uint4& q) {
    float a = 0.0f;
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.x),
                                        __builtin_bit_cast(bf16x2_t, q.x), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.y),
                                        __builtin_bit_cast(bf16x2_t, q.y), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.z),
                                        __builtin_bit_cast(bf16x2_t, q.z), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.w),
                                        __builtin_bit_cast(bf16x2_t, q.w), a, false);
    return a;
  }
};

// fp32: 4 elements per 16-byte slice.
template <>
struct Slice<float> {
  static constexpr int kElems = 4;
  __device__ static __forceinline__ float dot(const uint4& k, const uint4& q) {
    float a = __uint_as_float(k.x) * __uint_as_float(q.x);
    a = fmaf(__uint_as_float(k.y), __uint_as_float(q.y), a);
    a = fmaf(__uint_as_float(k.z), __uint_as_float(q.z), a);
    a = fmaf(__uint_as_float(k.w), __uint_as_float(q.w), a);
    return a;
  }
};

template <typename T, int D, int GB>
__global__ __launch_bounds__(256) void score_scan_kernel(
    const T* __restrict__ q, const T* __restrict__ K, const float* __restrict__ head_scale,
    float default_scale, int64_t n, int G, int nblk, float* __restrict__ scores,
    float* __restrict__ blkmax, void* zero_base, size_t zero_bytes) {
  constexpr int EPL = Slice<T>::kElems;
  constexpr int LPR = D / EPL;
  constexpr int RPW = kWave / LPR;
  constexpr int WAVES = 4;
  constexpr int ITER = kScanTile / (WAVES * RPW);
  static_assert(GB <= LPR, "one lane per head within a row group");
  __shared__ float s_sc[GB][kScanTile];
  __shared__ float s_red[GB][WAVES];

  const size_t nblocks = static_cast<size_t>(gridDim.x) * gridDim.y * gridDim.z;
  const size_t blin =
      (static_cast<size_t>(blockIdx.z) * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
  zero_slice(zero_base, zero_bytes, blin, nblocks);

  const int tile = blockIdx.x;
  const int kvh = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int seg = lane % LPR;
  const int rg = lane / LPR;
  const int h0 = kvh * G + blockIdx.z * GB;
  const int nh = min(GB, G - static_cast<int>(blockIdx.z) * GB);

  uint4 qv[GB];
  float sc[GB];
#pragma unroll
  for (int j = 0; j < GB; ++j) {
    if (j < nh) {
      qv[j] = *reinterpret_cast<const uint4*>(q + static_cast<size_t>(h0 + j) * D + seg * EPL);
      sc[j] = head_scale ? head_scale[h0 + j] : default_scale;
    } else {
      qv[j] = make_uint4(0, 0, 0, 0);
      sc[j] = 0.0f;
    }
  }

  const T* Kb = K + static_cast<size_t>(kvh) * static_cast<size_t>(n) * D;
  const int64_t tile0 = static_cast<int64_t>(tile) * kScanTile;
  const int lbase = wave * (ITER * RPW);

  uint4 kv[ITER];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int64_t r = tile0 + lbase + it * RPW + rg;
    kv[it] = make_uint4(0, 0, 0, 0);
    if (r < n) kv[it] = *reinterpret_cast<const uint4*>(Kb + r * D + seg * EPL);
  }
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    float acc[GB];
#pragma unroll
    for (int j = 0; j < GB; ++j) acc[j] = Slice<T>::dot(kv[it], qv[j]);
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) {
#pragma unroll
      for (int j = 0; j < GB; ++j) acc[j] += __shfl_xor(acc[j], o, kWave);
    }
    const int lr = lbase + it * RPW + rg;
#pragma unroll
    for (int j = 0; j < GB; ++j)
      if (seg == j) s_sc[j][lr] = acc[j] * sc[j];
  }
  __syncthreads();

  const int64_t i = tile0 + threadIdx.x;
#pragma unroll
  for (int j = 0; j < GB; ++j) {
    float v = -INFINITY;
    if (j < nh && i < n) {
      v = s_sc[j][threadIdx.x];
      scores[static_cast<size_t>(h0 + j) * static_cast<size_t>(n) + i] = v;
    }
    v = wave_max(v);
    if (lane == 0) s_red[j][wave] = v;
  }
  __syncthreads();
  if (threadIdx.x < nh) {
    const int j = threadIdx.x;
    float v = s_red[j][0];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) v = fmaxf(v, s_red[j][w]);
    blkmax[static_cast<size_t>(h0 + j) * nblk + tile] = v;
  }
}

template <typename T, int D, int GB>
hipError_t launch_t(const void* q, const void* K, const float* head_scale, float default_scale,
                    int64_t n, int n_q, int n_kv, float* scores, float* blkmax, void* zb,
                    size_t zbytes, hipStream_t st) {
  const int G = n_q / n_kv;
  const int nblk = static_cast<int>(ceil_div(n, kScanTile));
  dim3 grid(nblk, n_kv, static_cast<unsigned>(ceil_div(G, GB)));
  hipLaunchKernelGGL((score_scan_kernel<T, D, GB>), grid, dim3(256), 0, st,
                     static_cast<const T*>(q), static_cast<const T*>(K), head_scale,
                     default_scale, n, G, nblk, scores, blkmax, zb, zbytes);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const void* q, const void* K, const float* hs, float ds, int64_t n, int n_q,
                    int n_kv, float* scores, float* blkmax, void* zb, size_t zbytes,
                    hipStream_t st) {
  const int G = n_q / n_kv;
  if (G == 1) return launch_t<T, D, 1>(q, K, hs, ds, n, n_q, n_kv, scores, blkmax, zb, zbytes, st);
  if (G == 2) return launch_t<T, D, 2>(q, K, hs, ds, n, n_q, n_kv, scores, blkmax, zb, zbytes, st);
  if (G <= 4) return launch_t<T, D, 4>(q, K, hs, ds, n, n_q, n_kv, scores, blkmax, zb, zbytes, st);
  return launch_t<T, D, 8>(q, K, hs, ds, n, n_q, n_kv, scores, blkmax, zb, zbytes, st);
}

}  // namespace

hipError_t launch_score_scan(const void* q, const void* K, int dtype, int d,
                             const float* head_scale, float default_scale, int64_t n, int n_q,
                             int n_kv, float* scores, float* blkmax, void* zero_base,
                             size_t zero_bytes, hipStream_t st) {
  if (dtype == 1) {
    if (d == 128)
      return launch_d<uint16_t, 128>(q, K, head_scale, default_scale, n, n_q, n_kv, scores,
                                     blkmax, zero_base, zero_bytes, st);
    return launch_d<uint16_t, 64>(q, K, head_scale, default_scale, n, n_q, n_kv, scores, blkmax,
                                  zero_base, zero_bytes, st);
  }
  if (d == 128)
    return launch_d<float, 128>(q, K, head_scale, default_scale, n, n_q, n_kv, scores, blkmax,
                                zero_base, zero_bytes, st);
  return launch_d<float, 64>(q, K, head_scale, default_scale, n, n_q, n_kv, scores, blkmax,
                             zero_base, zero_bytes, st);
}

}  // namespace ctopk
