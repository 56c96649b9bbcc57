// K4 -- head-only renormalised output (Attn_k in the Abstract of "A
// Mathematical Theory of Top-k Sparse Attention via Total Variation
// Distance", arXiv 2512.07647):
//
//   out_h = sum_{i in H_h} w_i v_i / sum_{i in H_h} w_i,   w_i = exp(s_i - m_h)
//
// where H_h = { i : key64(s_i, i) >= thr_h } comes from the select.
//
// Memory plan (HBM-bound): a block owns kVsumTile keys of one V head and up to
// 8 query heads of its group.  A prologue (one thread per key, coalesced score
// reads) evaluates membership and the weight of every (key, head) pair once,
// writes the selection mask with wave ballots and stages the weights in LDS.
// The main loop streams only V rows kept by at least one head of the group
// (the union of the group's heads), each row read once with 16-byte loads by
// LPR consecutive lanes, and accumulates w * v for every head.  Partial sums
// per block go to scratch and are combined in fp64, in a fixed order, by
// finalize_kernel (so results are bitwise reproducible).
#include "kernels.h"

namespace ctopk {
namespace {

template <typename T>
struct VSlice;

template <>
struct VSlice<uint16_t> {  // bf16: 8 values per 16 bytes
  static constexpr int kElems = 8;
  __device__ static __forceinline__ void load(const uint4& u, float* v) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[e] << 16);
      v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  }
};

template <>
struct VSlice<float> {  // fp32: 4 values per 16 bytes
  static constexpr int kElems = 4;
  __device__ static __forceinline__ void load(const uint4& u, float* v) {
    v[0] = __uint_as_float(u.x);
    v[1] = __uint_as_float(u.y);
    v[2] = __uint_as_float(u.z);
    v[3] = __uint_as_float(u.w);
  }
};

// bf16 values accumulate in fp32 (tolerance is set by the bf16 inputs); fp32
// values accumulate in fp64 so the fp32 output keeps ~1e-7 relative accuracy.
template <typename T>
struct AccOf {
  using type = float;
};
template <>
struct AccOf<float> {
  using type = double;
};

template <typename T, int D, int GB>
__global__ __launch_bounds__(256) void vsum_kernel(const float* __restrict__ scores, int64_t n,
                                                   int G, const T* __restrict__ V,
                                                   const RowSel* __restrict__ rs,
                                                   float* __restrict__ part, int nchunk,
                                                   int tpb, uint32_t* __restrict__ sel_mask,
                                                   int64_t nwords) {
  using Acc = typename AccOf<T>::type;
  constexpr int EPL = VSlice<T>::kElems;
  constexpr int LPR = D / EPL;
  constexpr int RPW = kWave / LPR;
  constexpr int WAVES = 4;
  constexpr int NRG = WAVES * RPW;  // row groups per block
  constexpr int ITER = kVsumTile / NRG;
  __shared__ float s_w[GB][kVsumTile];
  __shared__ uint32_t s_any[kVsumTile];
  __shared__ Acc s_red[WAVES][GB * D];
  __shared__ double s_wsum[GB][WAVES];

  const int chunk = blockIdx.x;
  const int vh = blockIdx.y;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = t / kWave;
  const int h0 = vh * G + blockIdx.z * GB;
  const int nh = min(GB, G - static_cast<int>(blockIdx.z) * GB);
  const int seg = lane % LPR;
  const int rg = lane / LPR;
  const T* Vb = V + static_cast<size_t>(vh) * static_cast<size_t>(n) * D;
  Acc acc[GB][EPL];
#pragma unroll
  for (int j = 0; j < GB; ++j)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[j][e] = Acc(0);
  double wsum[GB];
#pragma unroll
  for (int j = 0; j < GB; ++j) wsum[j] = 0.0;

  for (int tb = 0; tb < tpb; ++tb) {
    const int64_t tile0 = (static_cast<int64_t>(chunk) * tpb + tb) * kVsumTile;
    if (tile0 >= n) break;
    // Prologue: membership and weights, one thread per key.
    {
      const int64_t i = tile0 + t;
      uint32_t any = 0u;
#pragma unroll
      for (int j = 0; j < GB; ++j) {
        float w = 0.0f;
        bool kept = false;
        if (j < nh && i < n) {
          const float s = scores[static_cast<size_t>(h0 + j) * static_cast<size_t>(n) + i];
          const RowSel r = rs[h0 + j];
          kept = key64(s, static_cast<uint32_t>(i)) >= r.thr;
          if (kept) w = weight(s, r.m);
        }
        any |= kept ? 1u : 0u;
        s_w[j][t] = w;
        wsum[j] += static_cast<double>(w);
        if (sel_mask != nullptr && j < nh) {
          const uint64_t b = __ballot(kept);
          const int64_t w0 = (tile0 + wave * kWave) / 32;
          uint32_t* mrow = sel_mask + static_cast<size_t>(h0 + j) * static_cast<size_t>(nwords);
          if (lane == 0 && w0 < nwords) mrow[w0] = static_cast<uint32_t>(b);
          if (lane == 1 && w0 + 1 < nwords) mrow[w0 + 1] = static_cast<uint32_t>(b >> 32);
        }
      }
      s_any[t] = any;
    }
    __syncthreads();

    // Main loop: stream the union of kept V rows.
#pragma unroll 4
    for (int it = 0; it < ITER; ++it) {
      const int lr = it * NRG + wave * RPW + rg;
      if (s_any[lr] != 0u) {
        const int64_t r = tile0 + lr;
        const uint4 u = *reinterpret_cast<const uint4*>(Vb + r * D + seg * EPL);
        float v[EPL];
        VSlice<T>::load(u, v);
#pragma unroll
        for (int j = 0; j < GB; ++j) {
          const Acc w = static_cast<Acc>(s_w[j][lr]);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[j][e] += w * static_cast<Acc>(v[e]);
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < GB; ++j) {
    const double ws = wave_sum(wsum[j]);
    if (lane == 0) s_wsum[j][wave] = ws;
  }

  // Combine the RPW row groups of each wave (xor butterfly over lane / LPR),
  // then the waves through LDS, always in the same order.
#pragma unroll
  for (int o = LPR; o < kWave; o <<= 1) {
#pragma unroll
    for (int j = 0; j < GB; ++j)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[j][e] += __shfl_xor(acc[j][e], o, kWave);
  }
  if (rg == 0) {
#pragma unroll
    for (int j = 0; j < GB; ++j)
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_red[wave][j * D + seg * EPL + e] = acc[j][e];
  }
  __syncthreads();

  for (int idx = t; idx < GB * D; idx += blockDim.x) {
    const int j = idx / D;
    if (j < nh) {
      const int e = idx - j * D;
      Acc sum = Acc(0);
#pragma unroll
      for (int g = 0; g < WAVES; ++g) sum += s_red[g][idx];
      part[(static_cast<size_t>(h0 + j) * nchunk + chunk) * (D + 1) + e] =
          static_cast<float>(sum);
    }
  }
  if (t < nh) {
    double ws = 0.0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) ws += s_wsum[t][w];
    part[(static_cast<size_t>(h0 + t) * nchunk + chunk) * (D + 1) + D] = static_cast<float>(ws);
  }
}

__global__ __launch_bounds__(256) void finalize_kernel(const float* __restrict__ part, int nchunk,
                                                       int dv, float* __restrict__ out) {
  __shared__ double s_den;
  const int row = blockIdx.x;
  const int e = threadIdx.x;
  double acc = 0.0;
  if (e <= dv) {
    const float* p = part + static_cast<size_t>(row) * nchunk * (dv + 1) + e;
    for (int c = 0; c < nchunk; ++c) acc += static_cast<double>(p[static_cast<size_t>(c) * (dv + 1)]);
  }
  if (e == dv) s_den = acc;
  __syncthreads();
  if (e < dv) out[static_cast<size_t>(row) * dv + e] = static_cast<float>(acc / s_den);
}

template <typename T, int D, int GB>
hipError_t launch_t(const float* scores, int64_t n, int rows, int n_v, const void* V,
                    const RowSel* rs, float* part, int nchunk, uint32_t* sel_mask,
                    hipStream_t st) {
  const int G = rows / n_v;
  const int tpb = static_cast<int>(ceil_div(ceil_div(n, kVsumTile), nchunk));
  dim3 grid(nchunk, n_v, static_cast<unsigned>(ceil_div(G, GB)));
  hipLaunchKernelGGL((vsum_kernel<T, D, GB>), grid, dim3(256), 0, st, scores, n, G,
                     static_cast<const T*>(V), rs, part, nchunk, tpb, sel_mask, ceil_div(n, 32));
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const float* scores, int64_t n, int rows, int n_v, const void* V,
                    const RowSel* rs, float* part, int nchunk, uint32_t* sel_mask,
                    hipStream_t st) {
  const int G = rows / n_v;
  if (G == 1) return launch_t<T, D, 1>(scores, n, rows, n_v, V, rs, part, nchunk, sel_mask, st);
  if (G == 2) return launch_t<T, D, 2>(scores, n, rows, n_v, V, rs, part, nchunk, sel_mask, st);
  if (G <= 4) return launch_t<T, D, 4>(scores, n, rows, n_v, V, rs, part, nchunk, sel_mask, st);
  return launch_t<T, D, 8>(scores, n, rows, n_v, V, rs, part, nchunk, sel_mask, st);
}

}  // namespace

hipError_t launch_vsum(const float* scores, int64_t n, int rows, int n_v, const void* V,
                       int v_dtype, int dv, const RowSel* rs, float* part, int nchunk,
                       uint32_t* sel_mask, hipStream_t st) {
  if (v_dtype == 1) {
    if (dv == 128) return launch_d<uint16_t, 128>(scores, n, rows, n_v, V, rs, part, nchunk, sel_mask, st);
    return launch_d<uint16_t, 64>(scores, n, rows, n_v, V, rs, part, nchunk, sel_mask, st);
  }
  if (dv == 128) return launch_d<float, 128>(scores, n, rows, n_v, V, rs, part, nchunk, sel_mask, st);
  return launch_d<float, 64>(scores, n, rows, n_v, V, rs, part, nchunk, sel_mask, st);
}

int vsum_nchunk(int64_t n, int rows, int n_v) {
  // Enough blocks to fill the chip (~4096), few enough partial sums to keep
  // their traffic small next to the value rows.
  const int64_t tiles = ceil_div(n, kVsumTile);
  const int G = rows / n_v;
  const int64_t zb = ceil_div(G, 8);
  const int64_t base = tiles * n_v * zb;
  int64_t tpb = 1;
  while (tpb < 256 && base / (tpb * 2) >= 4096) tpb *= 2;
  return static_cast<int>(ceil_div(tiles, tpb));
}

hipError_t launch_finalize(const float* part, int rows, int nchunk, int dv, float* out,
                           hipStream_t st) {
  hipLaunchKernelGGL(finalize_kernel, dim3(rows), dim3(256), 0, st, part, nchunk, dv, out);
  return hipGetLastError();
}

}  // namespace ctopk
