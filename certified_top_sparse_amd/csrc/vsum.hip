// K4 -- head-only renormalised output (Attn_k in the Abstract of "A
// Mathematical Theory of Top-k Sparse Attention via Total Variation
// Distance", arXiv 2512.07647):
//
//   out_h = sum_{i in H_h} w_i v_i / sum_{i in H_h} w_i,   w_i = exp(s_i - m_h)
//
// where H_h = { i : key64(s_i, i) >= thr_h } comes from the select.
//
// Memory plan (HBM-bound).  A block of 8 waves owns up to 8 query heads of one
// V head and `tpb` consecutive tiles of kVsumTile keys; each wave streams its
// 32 keys of a tile on its own, with no block barrier inside the stream:
//   * the V rows and the scores of a wave's keys are loaded together (each V
//     row once, 16-byte loads by LPR consecutive lanes), so the stream never
//     waits on a score read or on any other dependent load; keys outside a
//     head's set get weight 0 (on these workloads the union of a group's head
//     sets covers nearly every key, so loading every row costs little);
//   * each (key, head) weight is computed once, by one lane, and staged in a
//     wave-private LDS slot from which the LPR lanes of the row read all G
//     weights;
//   * w * v is accumulated for every head in registers.
// Block sums go to per-(head, block) partials, and finalize_kernel adds them
// in block order in fp64 and writes out, so results are bitwise reproducible.
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

constexpr int kVsumThreads = 512;


// Heads per block: 8, except fp32 values at d = 128, whose fp64 block sums
// would not fit LDS for 8 heads.
template <typename T, int D>
constexpr int kGroupMax = (sizeof(typename AccOf<T>::type) == 8 && D == 128) ? 4 : 8;
constexpr int kVsumWaves = kVsumThreads / kWave;

// With TAIL the kernel also accumulates the tail: w * v and w over the keys
// outside the head, so the combine can form the untruncated output and the
// truncation's output error; partials then hold [head num | head w | tail num
// | tail w] per (row, block).
template <typename T, int D, int GB, bool TAIL>
__global__ __launch_bounds__(kVsumThreads) void vsum_kernel(
    const float* __restrict__ scores, int64_t n, int G, const T* __restrict__ V,
    const RowSel* __restrict__ rs, float* __restrict__ part, int nchunk, int tpb) {
  using Acc = typename AccOf<T>::type;
  constexpr int EPL = VSlice<T>::kElems;
  constexpr int LPR = D / EPL;
  constexpr int RPW = kWave / LPR;
  constexpr int PASS = kVsumTile / kVsumWaves;  // keys per wave per tile
  constexpr int ITER = PASS / RPW;              // rows per lane per tile
  constexpr int NPAIR = PASS * GB;              // (key, head) weights per wave per tile
  constexpr int PPL = (NPAIR + kWave - 1) / kWave;  // weights per lane
  static_assert(kVsumTile % (kVsumWaves * RPW) == 0, "whole rows per lane");
  static_assert(GB <= LPR && kWave % GB == 0, "head groups tile the wave");
  constexpr int NS = TAIL ? 2 : 1;  // head sums, and tail sums with TAIL
  __shared__ Acc s_red[NS][kVsumWaves][GB * D];
  __shared__ double s_wsum[NS][kVsumWaves][GB];
  __shared__ float s_w[kVsumWaves][PASS][GB];  // wave-private weight staging

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

  // Weights are computed once per (key, head): pair p = lane + 64 * u covers
  // key p / GB and head p % GB, so each lane always works for head lane % GB.
  // That head's selection parameters are read with block-uniform addresses.
  const int hw = lane % GB;
  uint64_t thr = ~0ull;
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < GB; ++j) {
    const RowSel r = rs[h0 + min(j, nh - 1)];
    if (hw == j) {
      thr = j < nh ? r.thr : ~0ull;
      m = r.m;
    }
  }
  const float* srow = scores + static_cast<size_t>(h0 + min(hw, nh - 1)) * static_cast<size_t>(n);

  Acc acc[GB][EPL];
  Acc acct[TAIL ? GB : 1][EPL];
#pragma unroll
  for (int j = 0; j < GB; ++j)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[j][e] = Acc(0);
#pragma unroll
  for (int j = 0; j < (TAIL ? GB : 1); ++j)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acct[j][e] = Acc(0);
  double wsum = 0.0;   // weight of head hw over this lane's pairs
  double wsumt = 0.0;  // and of its tail (TAIL)

  for (int tb = 0; tb < tpb; ++tb) {
    const int64_t p0 = (static_cast<int64_t>(chunk) * tpb + tb) * kVsumTile + wave * PASS;
    if (p0 >= n) break;  // uniform per wave; waves do not synchronise in this loop
    // Value rows and the pass's scores, issued together (rows past n re-read
    // row n-1 and get weight 0).
    uint4 u[ITER];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int64_t r = min(p0 + it * RPW + rg, n - 1);
      u[it] = load_stream16(Vb + r * D + seg * EPL);
    }
    float s[PPL];
#pragma unroll
    for (int q = 0; q < PPL; ++q) {
      const int key = (lane + kWave * q) / GB;
      s[q] = srow[min(p0 + min(key, PASS - 1), n - 1)];
    }
#pragma unroll
    for (int q = 0; q < PPL; ++q) {
      const int pair = lane + kWave * q;
      if (pair < NPAIR) {
        const int key = pair / GB;
        const int64_t r = p0 + key;
        const bool kept = r < n && key64(s[q], static_cast<uint32_t>(r)) >= thr;
        if constexpr (TAIL) {
          // staged as +w for head keys and -w for tail keys
          const float w = r < n ? weight(s[q], m) : 0.0f;
          wsum += kept ? static_cast<double>(w) : 0.0;
          wsumt += kept ? 0.0 : static_cast<double>(w);
          s_w[wave][key][hw] = kept ? w : -w;
        } else {
          const float w = kept ? weight(s[q], m) : 0.0f;
          wsum += static_cast<double>(w);
          s_w[wave][key][hw] = w;
        }
      }
    }
    // s_w is private to this wave, and one wave's LDS operations complete in
    // order, so a wavefront-scope fence (which only stops the compiler from
    // moving the reads above the writes) is all the ordering needed.
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int key = it * RPW + rg;
      float wj[GB];
#pragma unroll
      for (int j = 0; j < GB; ++j) wj[j] = s_w[wave][key][j];
      float v[EPL];
      VSlice<T>::load(u[it], v);
      if constexpr (TAIL) {
#pragma unroll
        for (int j = 0; j < GB; ++j) {
          const Acc wh = static_cast<Acc>(fmaxf(wj[j], 0.0f));
          const Acc wt = static_cast<Acc>(fmaxf(-wj[j], 0.0f));
#pragma unroll
          for (int e = 0; e < EPL; ++e) {
            acc[j][e] += wh * static_cast<Acc>(v[e]);
            acct[j][e] += wt * static_cast<Acc>(v[e]);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < GB; ++j)
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[j][e] += static_cast<Acc>(wj[j]) * static_cast<Acc>(v[e]);
      }
    }
  }

  // Block sums: row groups of a wave (xor butterfly over lane / LPR), then the
  // waves in order through LDS.
#pragma unroll
  for (int o = LPR; o < kWave; o <<= 1) {
#pragma unroll
    for (int j = 0; j < GB; ++j)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[j][e] += __shfl_xor(acc[j][e], o, kWave);
    if constexpr (TAIL) {
#pragma unroll
      for (int j = 0; j < GB; ++j)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acct[j][e] += __shfl_xor(acct[j][e], o, kWave);
    }
  }
#pragma unroll
  for (int o = GB; o < kWave; o <<= 1) {
    wsum += __shfl_xor(wsum, o, kWave);
    if constexpr (TAIL) wsumt += __shfl_xor(wsumt, o, kWave);
  }
  if (rg == 0) {
#pragma unroll
    for (int j = 0; j < GB; ++j)
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        s_red[0][wave][j * D + seg * EPL + e] = acc[j][e];
        if constexpr (TAIL) s_red[NS - 1][wave][j * D + seg * EPL + e] = acct[j][e];
      }
  }
  if (lane < GB) {
    s_wsum[0][wave][lane] = wsum;
    if constexpr (TAIL) s_wsum[NS - 1][wave][lane] = wsumt;
  }
  __syncthreads();
  const size_t pstride = static_cast<size_t>(NS * (D + 1));
  for (int idx = t; idx < NS * GB * (D + 1); idx += kVsumThreads) {
    const int part_k = idx / (GB * (D + 1));  // 0 head, 1 tail
    const int rem = idx - part_k * GB * (D + 1);
    const int j = rem / (D + 1);
    const int e = rem - j * (D + 1);
    if (j < nh) {
      double sum = 0.0;
      if (e < D) {
#pragma unroll
        for (int g = 0; g < kVsumWaves; ++g) sum += static_cast<double>(s_red[part_k][g][j * D + e]);
      } else {
#pragma unroll
        for (int g = 0; g < kVsumWaves; ++g) sum += s_wsum[part_k][g][j];
      }
      part[(static_cast<size_t>(h0 + j) * nchunk + chunk) * pstride + part_k * (D + 1) + e] =
          static_cast<float>(sum);
    }
  }

}

// out[h, e] = sum_c part[h, c, e] / sum_c part[h, c, dv], fp64 sums in a fixed
// order: thread (k, e) adds chunks k, k + NK, ... and the NK partial sums are
// then added in k order.  Runs as its own kernel so that the kernel boundary
// makes every block's partials visible (an in-kernel device-scope fence costs
// a full L2 writeback and invalidate per block on this multi-XCD part).
// With tail sums (ns == 2) it also writes the untruncated output
// (num_head + num_tail) / (w_head + w_tail) and the output error
// ||Attn - Attn_k||_2 = tau * ||mu_tail - mu_head||_2, tau = w_tail / (w_head +
// w_tail) (the head-tail factorisation in the Abstract of "A Mathematical
// Theory of Top-k Sparse Attention via Total Variation Distance", arXiv
// 2512.07647).
__global__ __launch_bounds__(1024) void finalize_kernel(const float* __restrict__ part,
                                                        int nchunk, int dv, int ns,
                                                        float* __restrict__ out,
                                                        float* __restrict__ dense,
                                                        double* __restrict__ err) {
  __shared__ double s_col[1024];
  __shared__ double s_e2[16];
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int cols = ns * (dv + 1);
  const int NK = 1024 / cols;
  const int k = t / cols;
  const int e = t - k * cols;
  double a = 0.0;
  if (k < NK) {
    const float* p = part + static_cast<size_t>(row) * nchunk * cols + e;
    for (int c0 = k; c0 < nchunk; c0 += 8 * NK) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = min(c0 + u * NK, nchunk - 1);
        v[u] = p[static_cast<size_t>(c) * cols];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (c0 + u * NK < nchunk) a += static_cast<double>(v[u]);
    }
  }
  s_col[t] = a;
  __syncthreads();
  double e2 = 0.0;
  double wt_tau = 0.0;
  if (t < dv) {
    double num = 0.0, den = 0.0, numt = 0.0, dent = 0.0;
    for (int j = 0; j < NK; ++j) {
      num += s_col[j * cols + t];
      den += s_col[j * cols + dv];
      if (ns == 2) {
        numt += s_col[j * cols + dv + 1 + t];
        dent += s_col[j * cols + 2 * dv + 1];
      }
    }
    const double mh = num / den;
    out[static_cast<size_t>(row) * dv + t] = static_cast<float>(mh);
    if (ns == 2) {
      if (dense != nullptr)
        dense[static_cast<size_t>(row) * dv + t] = static_cast<float>((num + numt) / (den + dent));
      const double diff = dent > 0.0 ? numt / dent - mh : 0.0;
      e2 = diff * diff;
      wt_tau = dent / (den + dent);
    }
  }
  if (ns == 2 && err != nullptr) {  // uniform: the whole block reduces ||mu_t - mu_h||^2
    e2 = wave_sum(e2);
    if ((t & 63) == 0) s_e2[t >> 6] = e2;
    __syncthreads();
    if (t == 0) {
      double s2 = 0.0;
      for (int w = 0; w < 16; ++w) s2 += s_e2[w];
      err[row] = wt_tau * sqrt(s2);
    }
  }
}

template <typename T, int D, int GB>
hipError_t launch_t(const float* scores, int64_t n, int rows, int n_v, const void* V,
                    const RowSel* rs, float* part, int nchunk, float* out, float* dense,
                    double* err, hipStream_t st) {
  const int G = rows / n_v;
  const int tpb = static_cast<int>(ceil_div(ceil_div(n, kVsumTile), nchunk));
  dim3 grid(nchunk, n_v, static_cast<unsigned>(ceil_div(G, GB)));
  const bool tail = dense != nullptr || err != nullptr;
  const hipError_t e =
      tail ? launch(vsum_kernel<T, D, GB, true>, grid, dim3(kVsumThreads), 0, st, scores, n, G,
                    static_cast<const T*>(V), rs, part, nchunk, tpb)
           : launch(vsum_kernel<T, D, GB, false>, grid, dim3(kVsumThreads), 0, st, scores, n, G,
                    static_cast<const T*>(V), rs, part, nchunk, tpb);
  if (e != hipSuccess) return e;
  return launch(finalize_kernel, dim3(rows), dim3(1024), 0, st, part, nchunk, D, tail ? 2 : 1,
                out, dense, err);
}

template <typename T, int D>
hipError_t launch_d(const float* scores, int64_t n, int rows, int n_v, const void* V,
                    const RowSel* rs, float* part, int nchunk, float* out, float* dense,
                    double* err, hipStream_t st) {
  const int G = rows / n_v;
  if (G == 1)
    return launch_t<T, D, 1>(scores, n, rows, n_v, V, rs, part, nchunk, out, dense, err, st);
  if (G == 2)
    return launch_t<T, D, 2>(scores, n, rows, n_v, V, rs, part, nchunk, out, dense, err, st);
  if constexpr (kGroupMax<T, D> == 4) {
    return launch_t<T, D, 4>(scores, n, rows, n_v, V, rs, part, nchunk, out, dense, err, st);
  } else {
    if (G <= 4)
      return launch_t<T, D, 4>(scores, n, rows, n_v, V, rs, part, nchunk, out, dense, err, st);
    return launch_t<T, D, 8>(scores, n, rows, n_v, V, rs, part, nchunk, out, dense, err, st);
  }
}

}  // namespace

hipError_t launch_vsum(const float* scores, int64_t n, int rows, int n_v, const void* V,
                       int v_dtype, int dv, const RowSel* rs, float* part, int nchunk, float* out,
                       float* dense, double* err, hipStream_t st) {
  if (v_dtype == 1) {
    if (dv == 128)
      return launch_d<uint16_t, 128>(scores, n, rows, n_v, V, rs, part, nchunk, out, dense, err,
                                     st);
    return launch_d<uint16_t, 64>(scores, n, rows, n_v, V, rs, part, nchunk, out, dense, err, st);
  }
  if (dv == 128)
    return launch_d<float, 128>(scores, n, rows, n_v, V, rs, part, nchunk, out, dense, err, st);
  return launch_d<float, 64>(scores, n, rows, n_v, V, rs, part, nchunk, out, dense, err, st);
}

int vsum_groups(int rows, int n_v, int v_dtype, int dv) {
  const int G = rows / n_v;
  const int gmax = (v_dtype == 0 && dv == 128) ? 4 : 8;
  const int gb = G == 1 ? 1 : (G == 2 ? 2 : (G <= 4 ? 4 : gmax));
  return n_v * static_cast<int>(ceil_div(G, gb));
}

int vsum_nchunk(int64_t n, int rows, int n_v, int v_dtype, int dv) {
  // Blocks per group: about one block per compute unit in total (measured
  // fastest on MI355X: each block streams several tiles and amortises its
  // reduction epilogue), and never more blocks than tiles.
  const int64_t tiles = ceil_div(n, kVsumTile);
  const int64_t groups = vsum_groups(rows, n_v, v_dtype, dv);
  int64_t want = ceil_div(kNumCUs, groups);
  if (want > tiles) want = tiles;
  if (want < 1) want = 1;
  const int64_t tpb = ceil_div(tiles, want);
  return static_cast<int>(ceil_div(tiles, tpb));
}

}  // namespace ctopk
