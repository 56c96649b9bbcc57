// K4 -- head-only renormalised output (Attn_k in the Abstract of "A
// Mathematical Theory of Top-k Sparse Attention via Total Variation
// Distance", arXiv 2512.07647):
//
//   out_h = sum_{i in H_h} w_i v_i / sum_{i in H_h} w_i,   w_i = exp(s_i - m_h)
//
// where H_h = { i : key64(s_i, i) >= thr_h } comes from the select.
//
// Two ways to the same sums (HBM-bound either way):
//   * after the select: vsum_kernel streams V once with each key's head
//     weights (the stream body is in vsum_body.h) and the finalize below
//     combines the chunks;
//   * beside the select (select.hip): a stream over a provisional head runs in
//     the select's own launch on the compute units the select leaves idle,
//     corrects its sums by the keys between the provisional and the exact cut,
//     and the last chunk of each head group combines the partials.
// Chunk sums go to per-(head, chunk) partials, and finalize_kernel adds them
// in chunk order in fp64 and writes out, so results are bitwise reproducible.

#include "vsum_body.h"

namespace ctopk {
namespace {

constexpr int kVsumThreads = 512;
constexpr int kVsumWaves = kVsumThreads / kWave;

// With TAIL the kernel also accumulates the tail: w * v and w over the keys
// outside the head, so the combine can form the untruncated output and the
// truncation's output error; partials then hold [head num | head w | tail num
// | tail w] per (row, chunk).
template <typename T, int D, int GB, bool TAIL>
__global__ __launch_bounds__(kVsumThreads) void vsum_kernel(
    const float* __restrict__ scores, int64_t n, int G, const T* __restrict__ V,
    const RowSel* __restrict__ rs, float* __restrict__ part, int nchunk, int tpb) {
  constexpr int MODE = TAIL ? kStreamHeadTail : kStreamHead;
  __shared__ StreamSmem<T, D, GB, MODE, kVsumWaves> sm;
  value_stream_block<T, D, GB, MODE, kVsumWaves>(sm, scores, n, G, V, rs, part,
                                                 nchunk, tpb, static_cast<int>(blockIdx.x),
                                                 static_cast<int>(blockIdx.y),
                                                 static_cast<int>(blockIdx.z));
}

// out[h, e] = sum_c part[h, c, e] / sum_c part[h, c, dv], fp64 sums in a fixed
// order: thread (k, e) adds chunks k, k + NK, ... and the NK partial sums are
// then added in k order.  Runs as its own kernel so that the kernel boundary
// makes every block's partials visible (an in-kernel device-scope fence costs
// a full L2 writeback and invalidate per block on this multi-XCD part).
// With tail sums (ns == 2) it also writes the untruncated output
// (num_head + num_tail) / (w_head + w_tail), the output error
// ||Attn - Attn_k||_2 = tau * ||mu_tail - mu_head||_2, tau = w_tail / (w_head +
// w_tail) (the head-tail factorisation in the Abstract of "A Mathematical
// Theory of Top-k Sparse Attention via Total Variation Distance", arXiv
// 2512.07647), and Var_P(V) = sum_i P_i ||v_i||^2 - ||Attn||^2, the spread of
// the value rows under P that bounds that error by sqrt(tau Var_P(V) /
// (1 - tau)) (the same Abstract's refinement by Var_P(V); the bound follows
// from the law of total variance over the head and the tail).
__global__ __launch_bounds__(1024) void finalize_kernel(const float* __restrict__ part,
                                                        int nchunk, int dv, int ns,
                                                        float* __restrict__ out,
                                                        float* __restrict__ dense,
                                                        double* __restrict__ err,
                                                        double* __restrict__ var) {
  __shared__ double s_col[1024];
  __shared__ double s_e2[16];
  __shared__ double s_d2[16];
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int cols = ns * (dv + 1) + (ns == 2 ? 1 : 0);
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
  double e2 = 0.0, d2 = 0.0;
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
      const double md = (num + numt) / (den + dent);
      if (dense != nullptr) dense[static_cast<size_t>(row) * dv + t] = static_cast<float>(md);
      const double diff = dent > 0.0 ? numt / dent - mh : 0.0;
      e2 = diff * diff;
      d2 = md * md;
      wt_tau = dent / (den + dent);
    }
  }
  if (ns == 2 && (err != nullptr || var != nullptr)) {
    // uniform: the whole block reduces ||mu_t - mu_h||^2 and ||Attn||^2
    e2 = wave_sum_f64(e2);
    d2 = wave_sum_f64(d2);
    if ((t & 63) == 0) {
      s_e2[t >> 6] = e2;
      s_d2[t >> 6] = d2;
    }
    __syncthreads();
    if (t == 0) {
      double s2 = 0.0, m2 = 0.0, q2 = 0.0, wall = 0.0;
      for (int w = 0; w < 16; ++w) {
        s2 += s_e2[w];
        m2 += s_d2[w];
      }
      for (int j = 0; j < NK; ++j) {
        q2 += s_col[j * cols + 2 * (dv + 1)];
        wall += s_col[j * cols + dv] + s_col[j * cols + 2 * dv + 1];
      }
      if (err != nullptr) err[row] = wt_tau * sqrt(s2);
      if (var != nullptr) var[row] = fmax(q2 / wall - m2, 0.0);
    }
  }
}

template <typename T, int D, int GB>
hipError_t launch_t(const float* scores, int64_t n, int rows, int n_v, const void* V,
                    const RowSel* rs, float* part, int nchunk, float* out, float* dense,
                    double* err, double* var, hipStream_t st) {
  const int G = rows / n_v;
  const int tpb = static_cast<int>(ceil_div(ceil_div(n, kVsumTile), nchunk));
  dim3 grid(nchunk, n_v, static_cast<unsigned>(ceil_div(G, GB)));
  const bool tail = dense != nullptr || err != nullptr || var != nullptr;
  const hipError_t e =
      tail ? launch(vsum_kernel<T, D, GB, true>, grid, dim3(kVsumThreads), 0, st, scores, n, G,
                    static_cast<const T*>(V), rs, part, nchunk, tpb)
           : launch(vsum_kernel<T, D, GB, false>, grid, dim3(kVsumThreads), 0, st, scores, n, G,
                    static_cast<const T*>(V), rs, part, nchunk, tpb);
  if (e != hipSuccess) return e;
  return launch(finalize_kernel, dim3(rows), dim3(1024), 0, st, part, nchunk, D, tail ? 2 : 1,
                out, dense, err, var);
}


// Many query rows per V (a group of at least kGemmRows rows, as on given
// logits with one shared V): the head sums of a chunk of keys are the product
// W V of the masked weight matrix (w_ri = exp(s_ri - m_r) on the head, else
// 0) with V, so a block of 64 rows runs it on MFMA (v_mfma_f32_16x16x4f32:
// fp32 operands and sums) instead of re-reading V once per 8 rows.  Layouts:
// A[i][k] in lane i + 16 k, B[k][j] in lane j + 16 k, D[i][j] in lane
// j + 16 (i / 4), element i % 4.  In step s of a 64-key super-step, k slot
// kk holds key 16 kk + s, so each lane reads 16 consecutive logits of its
// row; the super-step's V rows are staged in LDS at row 4 s + kk with the
// D / 16 values a lane multiplies in one step side by side ([col % 16][col /
// 16]), so a step's B operands are one or two 16-byte reads per lane, the
// wave reading 1 KB contiguous.
constexpr int kGemmRows = 64;
constexpr int kGemmKeys = 64;

typedef float gemm_f32x4_t __attribute__((ext_vector_type(4)));

template <typename T, int D>
__global__ __launch_bounds__(256) void vsum_gemm_kernel(
    const float* __restrict__ scores, int64_t n, int G, const T* __restrict__ V,
    const RowSel* __restrict__ rs, float* __restrict__ part, int nchunk, int64_t chunk_keys) {
  constexpr int CT = D / 16;  // 16-column tiles
  constexpr int EPL = VSlice<T>::kElems;
  constexpr int VLOADS = kGemmKeys * D / EPL / 256;  // 16-byte V loads per thread and super-step
  static_assert(VLOADS * 256 * EPL == kGemmKeys * D, "whole V tile per super-step");
  __shared__ float s_v[kGemmKeys][16][CT];

  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = t / kWave;
  const int chunk = blockIdx.x;
  const int kvh = blockIdx.z;
  const int li = lane & 15;   // A row / B column within the tile
  const int kk = lane >> 4;   // k slot
  const int rloc = static_cast<int>(blockIdx.y) * kGemmRows + 16 * wave + li;  // row in group
  const bool row_live = rloc < G;
  const int row = kvh * G + min(rloc, G - 1);
  const RowSel sel = rs[row];
  const float* srow = scores + static_cast<size_t>(row) * static_cast<size_t>(n);
  const T* Vb = V + static_cast<size_t>(kvh) * static_cast<size_t>(n) * D;
  const int64_t k_begin = static_cast<int64_t>(chunk) * chunk_keys;
  const int64_t k_end = min(n, k_begin + chunk_keys);
  const bool vec_rows = (n & 3) == 0;

  gemm_f32x4_t acc[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) acc[c] = gemm_f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float wsum = 0.0f;

  for (int64_t k0 = k_begin; k0 < k_end; k0 += kGemmKeys) {
    // V rows k0 .. k0 + 63 (past n: row n - 1, weighted 0) into LDS.
    uint4 vv[VLOADS];
#pragma unroll
    for (int u = 0; u < VLOADS; ++u) {
      const int f = (u * 256 + t) * EPL;  // flat element index in the tile
      const int64_t key = min(k0 + f / D, n - 1);
      vv[u] = *reinterpret_cast<const uint4*>(Vb + static_cast<size_t>(key) * D + f % D);
    }
    // This lane's 16 logits: keys k0 + 16 kk .. + 15 of its row (16-byte loads
    // when rows are 16-byte aligned, that is n % 4 == 0).
    float sv[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int64_t key = k0 + 16 * kk + 4 * q4;
      if (vec_rows && key + 3 < n) {
        const float4 x = *reinterpret_cast<const float4*>(srow + key);
        sv[4 * q4] = x.x;
        sv[4 * q4 + 1] = x.y;
        sv[4 * q4 + 2] = x.z;
        sv[4 * q4 + 3] = x.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[4 * q4 + e] = srow[min(key + e, n - 1)];
      }
    }
    float wv[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t key = k0 + 16 * kk + e;
      const bool kept = row_live && key < k_end &&
                        key64(sv[e], static_cast<uint32_t>(key)) >= sel.thr;
      wv[e] = kept ? weight(sv[e], sel.m) : 0.0f;
      wsum += wv[e];
    }
    __syncthreads();  // the previous super-step's reads of s_v are done
#pragma unroll
    for (int u = 0; u < VLOADS; ++u) {
      const int f = (u * 256 + t) * EPL;
      const int key = f / D;  // 16 kk' + s' -> LDS row 4 s' + kk'
      float x[EPL];
      VSlice<T>::load(vv[u], x);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int col = f % D + e;
        s_v[4 * (key & 15) + (key >> 4)][col & 15][col >> 4] = x[e];
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      float b[CT];
#pragma unroll
      for (int c4 = 0; c4 < CT; c4 += 4) {
        const float4 v4 = *reinterpret_cast<const float4*>(&s_v[4 * s + kk][li][c4]);
        b[c4] = v4.x;
        b[c4 + 1] = v4.y;
        b[c4 + 2] = v4.z;
        b[c4 + 3] = v4.w;
      }
#pragma unroll
      for (int c = 0; c < CT; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(wv[s], b[c], acc[c], 0, 0, 0);
    }
  }

  // Partials: lane (j, q) holds rows 4 q + e of the wave's 16, column 16 c + j.
  const int q = lane >> 4;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = static_cast<int>(blockIdx.y) * kGemmRows + 16 * wave + 4 * q + e;
    if (r < G) {
      float* p = part + (static_cast<size_t>(kvh * G + r) * nchunk + chunk) * (D + 1);
#pragma unroll
      for (int c = 0; c < CT; ++c) p[16 * c + li] = acc[c][e];
    }
  }
  wsum = xrow32_sum(xrow16_sum(wsum));
  if (kk == 0 && row_live)
    part[(static_cast<size_t>(row) * nchunk + chunk) * (D + 1) + D] = wsum;
}

template <typename T, int D>
hipError_t launch_gemm(const float* scores, int64_t n, int rows, int n_v, const void* V,
                       const RowSel* rs, float* part, int nchunk, float* out, hipStream_t st) {
  const int G = rows / n_v;
  // chunks past the keys (ck rounds up) write zero partials
  const int64_t ck = ceil_div(ceil_div(n, nchunk), kGemmKeys) * kGemmKeys;
  dim3 grid(nchunk, static_cast<unsigned>(ceil_div(G, kGemmRows)), n_v);
  const hipError_t e = launch(vsum_gemm_kernel<T, D>, grid, dim3(256), 0, st, scores, n, G,
                              static_cast<const T*>(V), rs, part, nchunk, ck);
  if (e != hipSuccess) return e;
  return launch(finalize_kernel, dim3(rows), dim3(1024), 0, st, static_cast<const float*>(part),
                nchunk, D, 1, out, static_cast<float*>(nullptr), static_cast<double*>(nullptr),
                static_cast<double*>(nullptr));
}

template <typename T, int D>
hipError_t launch_d(const float* scores, int64_t n, int rows, int n_v, const void* V,
                    const RowSel* rs, float* part, int nchunk, float* out, float* dense,
                    double* err, double* var, hipStream_t st) {
  const int G = rows / n_v;
  if (G >= kGemmRows && dense == nullptr && err == nullptr && var == nullptr)
    return launch_gemm<T, D>(scores, n, rows, n_v, V, rs, part, nchunk, out, st);
  if (G == 1)
    return launch_t<T, D, 1>(scores, n, rows, n_v, V, rs, part, nchunk, out, dense, err, var, st);
  if (G == 2)
    return launch_t<T, D, 2>(scores, n, rows, n_v, V, rs, part, nchunk, out, dense, err, var, st);
  if constexpr (kGroupMax<T, D> == 4) {
    return launch_t<T, D, 4>(scores, n, rows, n_v, V, rs, part, nchunk, out, dense, err, var, st);
  } else {
    if (G <= 4)
      return launch_t<T, D, 4>(scores, n, rows, n_v, V, rs, part, nchunk, out, dense, err, var, st);
    return launch_t<T, D, 8>(scores, n, rows, n_v, V, rs, part, nchunk, out, dense, err, var, st);
  }
}

}  // namespace

hipError_t launch_vsum(const float* scores, int64_t n, int rows, int n_v, const void* V,
                       int v_dtype, int dv, const RowSel* rs, float* part, int nchunk, float* out,
                       float* dense, double* err, double* var, hipStream_t st) {
  if (v_dtype == 1) {
    if (dv == 128)
      return launch_d<uint16_t, 128>(scores, n, rows, n_v, V, rs, part, nchunk, out, dense, err,
                                     var, st);
    return launch_d<uint16_t, 64>(scores, n, rows, n_v, V, rs, part, nchunk, out, dense, err, var, st);
  }
  if (dv == 128)
    return launch_d<float, 128>(scores, n, rows, n_v, V, rs, part, nchunk, out, dense, err, var, st);
  return launch_d<float, 64>(scores, n, rows, n_v, V, rs, part, nchunk, out, dense, err, var, st);
}

int vsum_groups(int rows, int n_v, int v_dtype, int dv) {
  const int G = rows / n_v;
  const int gmax = (v_dtype == 0 && dv == 128) ? 4 : 8;
  const int gb = G == 1 ? 1 : (G == 2 ? 2 : (G <= 4 ? 4 : gmax));
  return n_v * static_cast<int>(ceil_div(G, gb));
}

int stream_nchunk(int64_t n, int groups, int blocks) {
  const int64_t tiles = ceil_div(n, kVsumTile);
  int64_t want = ceil_div(blocks, groups);
  if (want > tiles) want = tiles;
  if (want < 1) want = 1;
  const int64_t tpb = ceil_div(tiles, want);
  return static_cast<int>(ceil_div(tiles, tpb));
}

int vsum_nchunk(int64_t n, int rows, int n_v, int v_dtype, int dv) {
  const int G = rows / n_v;
  if (G >= kGemmRows) {
    // The MFMA stream: about four blocks per compute unit over the row tiles,
    // chunks of at least 512 keys (fp32 sums within a chunk stay short).
    const int64_t tiles = static_cast<int64_t>(n_v) * ceil_div(G, kGemmRows);
    int64_t want = ceil_div(4 * kNumCUs, tiles);
    const int64_t most = ceil_div(n, 512);
    if (want > most) want = most;
    return static_cast<int>(want < 1 ? 1 : want);
  }
  // Blocks per group: about one block per compute unit in total (measured
  // fastest on MI355X: each block streams several tiles and amortises its
  // reduction epilogue), and never more blocks than tiles.
  return stream_nchunk(n, vsum_groups(rows, n_v, v_dtype, dv), kNumCUs);
}

}  // namespace ctopk
