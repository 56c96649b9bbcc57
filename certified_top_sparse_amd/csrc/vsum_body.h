// The value stream's per-workgroup body, shared by the stand-alone value
// stream kernel and by the kernel that runs the select beside a stream over
// provisional heads.
//
// A workgroup of NW waves owns up to GB query heads of one V head and `tpb`
// consecutive tiles of kVsumTile keys; each wave streams its kVsumTile / NW
// keys of a tile on its own, with no workgroup barrier inside the stream:
//   * the V rows and the scores of a wave's keys are loaded together (each V
//     row once, 16-byte loads by LPR consecutive lanes), so the stream never
//     waits on a score read or on any other dependent load; keys outside a
//     head's set get weight 0;
//   * each (key, head) weight is computed once, by one lane, and staged in a
//     wave-private LDS slot from which the LPR lanes of the row read all GB
//     weights;
//   * w * v is accumulated for every head in registers.
// Workgroup sums go to per-(head, workgroup) partials [numerator | weight].
#pragma once

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

// Heads per workgroup: 8, except fp32 values at d = 128, whose fp64 sums
// would not fit LDS for 8 heads.
template <typename T, int D>
constexpr int kGroupMax = (sizeof(typename AccOf<T>::type) == 8 && D == 128) ? 4 : 8;

// What a stream sums: the head only (weights of keys outside the head are
// 0); head and tail separately; or the keys at or above per-head thresholds
// the caller puts in StreamSmem::thr (a provisional head, with the row maxima
// in StreamSmem::m), whose scores are also copied to the caller's LDS array
// `stash` ([GB][kFixKeys], by the key's place in the chunk; chunks of at most
// kFixKeys keys) and whose lane sums go to the hook alone: the hook finishes
// them, and no partials are written.
enum StreamMode { kStreamHead = 0, kStreamHeadTail = 1, kStreamGiven = 3 };

template <typename T, int D, int GB, int MODE, int NW>
struct StreamShape {
  using Acc = typename AccOf<T>::type;
  static constexpr int EPL = VSlice<T>::kElems;
  static constexpr int LPR = D / EPL;                  // lanes per V row
  static constexpr int RPW = kWave / LPR;              // rows per wave load
  static constexpr int PASS = kVsumTile / NW;          // keys per wave per tile
  static constexpr int ITER = PASS / RPW;              // rows per lane per tile
  static constexpr int NPAIR = PASS * GB;              // (key, head) weights per wave per tile
  static constexpr int PPL = (NPAIR + kWave - 1) / kWave;
  static constexpr int NS = MODE == kStreamHeadTail ? 2 : 1;
  static_assert(kVsumTile % (NW * RPW) == 0, "whole rows per lane");
  static_assert(GB <= LPR && kWave % GB == 0, "head groups tile the wave");
};

template <typename T, int D, int GB, int MODE, int NW>
struct StreamSmem {
  using S = StreamShape<T, D, GB, MODE, NW>;
  typename S::Acc red[S::NS][NW][GB * D];
  double wsum[S::NS][NW][GB];
  double q2[MODE == kStreamHeadTail ? NW : 1][GB];  // head and tail: sum of w ||v||^2
  float w[NW][S::PASS][GB];  // wave-private weight staging
  uint64_t thr[GB];          // given mode: key64 thresholds per head
  float m[GB];               // given mode: row maxima per head
};

// What a lane holds when the stream loop ends: acc[j][e] sums w v for head
// j over V elements seg * EPL + e of its rows, wsum the weight of head
// hw = lane % GB over its (key, head) pairs.
template <typename T, int D, int GB>
struct StreamLane {
  typename AccOf<T>::type (&acc)[GB][VSlice<T>::kElems];
  double& wsum;
  float m;  // the maximum of head hw's row
};

struct NoHook {
  template <typename L>
  __device__ __forceinline__ void operator()(L&) const {}
};

// One workgroup of the stream: chunk `chunk` of V head `vh`, query heads
// vh * G + hz * GB + [0, GB).  Head and tail modes take each head's maximum
// and cut from rs; the given mode takes them from StreamSmem.  `hook` sees every lane's sums (StreamLane)
// after the stream and before the workgroup reduction and may change them.
// Partials: part[(head, chunk)] holds NS blocks of [D numerators | weight
// sum], and in head and tail mode one more float: sum over all keys of
// w ||v||^2 (from which the combine forms Var_P(V)).
template <typename T, int D, int GB, int MODE, int NW, typename Hook = NoHook>
__device__ __forceinline__ void value_stream_block(
    StreamSmem<T, D, GB, MODE, NW>& sm, const float* __restrict__ scores, int64_t n, int G,
    const T* __restrict__ V, const RowSel* __restrict__ rs, float* __restrict__ part, int nchunk,
    int tpb, int chunk, int vh, int hz,
    Hook hook = Hook(), float* stash = nullptr) {
  using S = StreamShape<T, D, GB, MODE, NW>;
  using Acc = typename S::Acc;
  constexpr int EPL = S::EPL, LPR = S::LPR, RPW = S::RPW, PASS = S::PASS, ITER = S::ITER;
  constexpr int NPAIR = S::NPAIR, PPL = S::PPL, NS = S::NS;
  constexpr int NT = NW * kWave;
  constexpr bool TAIL = MODE == kStreamHeadTail;

  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = t / kWave;
  const int h0 = vh * G + hz * GB;
  const int nh = min(GB, G - hz * GB);
  const int seg = lane % LPR;
  const int rg = lane / LPR;
  const T* Vb = V + static_cast<size_t>(vh) * static_cast<size_t>(n) * D;

  // Weights are computed once per (key, head): pair p = lane + 64 * u covers
  // key p / GB and head p % GB, so each lane always works for head lane % GB.
  const int hw = lane % GB;
  uint64_t thr = ~0ull;
  float m = 0.0f;
  if constexpr (MODE == kStreamGiven) {
    thr = hw < nh ? sm.thr[hw] : ~0ull;
    m = sm.m[hw];
  } else {
    // That head's selection parameters are read with workgroup-uniform addresses.
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      const RowSel r = rs[h0 + min(j, nh - 1)];
      if (hw == j) {
        thr = j < nh ? r.thr : ~0ull;
        m = r.m;
      }
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
  Acc q2[TAIL ? GB : 1];  // TAIL: sum of w * (this lane's part of ||v||^2), per head
#pragma unroll
  for (int j = 0; j < (TAIL ? GB : 1); ++j) q2[j] = Acc(0);

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
          sm.w[wave][key][hw] = kept ? w : -w;
        } else {
          const float w = kept ? weight(s[q], m) : 0.0f;
          wsum += static_cast<double>(w);
          sm.w[wave][key][hw] = w;
          if constexpr (MODE == kStreamGiven) {  // the chunk's scores, kept for the caller
            if (r < n) stash[hw * kFixKeys + tb * kVsumTile + wave * PASS + key] = s[q];
          }
        }
      }
    }
    // sm.w[wave] is private to this wave, and one wave's LDS operations
    // complete in order, so a wavefront-scope fence (which only stops the
    // compiler from moving the reads above the writes) is all the ordering
    // needed.
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int key = it * RPW + rg;
      float wj[GB];
#pragma unroll
      for (int j = 0; j < GB; ++j) wj[j] = sm.w[wave][key][j];
      float v[EPL];
      VSlice<T>::load(u[it], v);
      if constexpr (TAIL) {
        Acc vv = Acc(0);  // this lane's slice of ||v||^2
#pragma unroll
        for (int e = 0; e < EPL; ++e) vv += static_cast<Acc>(v[e]) * static_cast<Acc>(v[e]);
#pragma unroll
        for (int j = 0; j < GB; ++j) {
          const Acc wh = static_cast<Acc>(fmaxf(wj[j], 0.0f));
          const Acc wt = static_cast<Acc>(fmaxf(-wj[j], 0.0f));
#pragma unroll
          for (int e = 0; e < EPL; ++e) {
            acc[j][e] += wh * static_cast<Acc>(v[e]);
            acct[j][e] += wt * static_cast<Acc>(v[e]);
          }
          q2[j] += (wh + wt) * vv;
        }
      } else {
#pragma unroll
        for (int j = 0; j < GB; ++j)
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[j][e] += static_cast<Acc>(wj[j]) * static_cast<Acc>(v[e]);
      }
    }
  }

  {
    StreamLane<T, D, GB> ln{acc, wsum, m};
    hook(ln);
  }
  if constexpr (MODE == kStreamGiven) return;  // the hook finished the sums

  // Workgroup sums: row groups of a wave (lanes that share lane % LPR, by
  // cross-lane adds), then the waves in order through LDS.
#pragma unroll
  for (int j = 0; j < GB; ++j)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      acc[j][e] = stride_sum<LPR>(acc[j][e]);
      if constexpr (TAIL) acct[j][e] = stride_sum<LPR>(acct[j][e]);
    }
#pragma unroll
  for (int o = GB; o < 16; o <<= 1) {
    wsum += __shfl_xor(wsum, o, kWave);
    if constexpr (TAIL) wsumt += __shfl_xor(wsumt, o, kWave);
  }
  wsum = xrow32_sum(xrow16_sum(wsum));
  if constexpr (TAIL) wsumt = xrow32_sum(xrow16_sum(wsumt));
  if constexpr (TAIL) {
    // every lane of the wave holds a part of each head's sum: a fixed tree
    // over all 64 lanes
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      double x = static_cast<double>(q2[j]);
      x = wave_sum_f64(x);
      if (lane == 0) sm.q2[wave][j] = x;
    }
  }
  if (rg == 0) {
#pragma unroll
    for (int j = 0; j < GB; ++j)
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        sm.red[0][wave][j * D + seg * EPL + e] = acc[j][e];
        if constexpr (TAIL) sm.red[NS - 1][wave][j * D + seg * EPL + e] = acct[j][e];
      }
  }
  if (lane < GB) {
    sm.wsum[0][wave][lane] = wsum;
    if constexpr (TAIL) sm.wsum[NS - 1][wave][lane] = wsumt;
  }
  __syncthreads();
  const size_t pstride = static_cast<size_t>(NS * (D + 1) + (TAIL ? 1 : 0));
  if constexpr (TAIL) {
    if (t < nh) {
      double sum = 0.0;
#pragma unroll
      for (int g = 0; g < NW; ++g) sum += sm.q2[g][t];
      part[(static_cast<size_t>(h0 + t) * nchunk + chunk) * pstride + NS * (D + 1)] =
          static_cast<float>(sum);
    }
  }
  for (int idx = t; idx < NS * GB * (D + 1); idx += NT) {
    const int part_k = idx / (GB * (D + 1));  // 0 head (or dense), 1 tail
    const int rem = idx - part_k * GB * (D + 1);
    const int j = rem / (D + 1);
    const int e = rem - j * (D + 1);
    if (j < nh) {
      double sum = 0.0;
      if (e < D) {
#pragma unroll
        for (int g = 0; g < NW; ++g) sum += static_cast<double>(sm.red[part_k][g][j * D + e]);
      } else {
#pragma unroll
        for (int g = 0; g < NW; ++g) sum += sm.wsum[part_k][g][j];
      }
      part[(static_cast<size_t>(h0 + j) * nchunk + chunk) * pstride + part_k * (D + 1) + e] =
          static_cast<float>(sum);
    }
  }
}

}  // namespace
}  // namespace ctopk
