// Encoder-shaped path: every query row of a head against all n <= 512 keys of
// that head, bf16 inputs (dense QK^T on MFMA).
//
// What is computed follows the Abstract of "A Mathematical Theory of Top-k
// Sparse Attention via Total Variation Distance" (arXiv 2512.07647): per query
// row s_i = scale * q.k_i, the head is the k largest-score keys (equal scores:
// lower index first), k_eps is the smallest k whose discarded softmax mass is
// at most eps, tau is that mass, and the output is the softmax average of V
// over the head, renormalised over the head.
//
// One workgroup = 4 wavefronts = 32 query rows of one KV head: two row
// groups of 16 rows, each row's keys split into two halves of NT / 2 tiles,
// one wave per (row group, half).  About 79 KiB of LDS and up to 256 VGPRs
// (the scores stay in registers), so two workgroups share a CU.  Lane (r, g) = (lane % 16, lane / 16) of a
// wave holds row r and the keys kh * 8 NT + 16 t + 4 g + e (t < NT / 2, e < 4),
// which is the fp32 result layout of a 16x16x32 bf16 MFMA computing
// S^T = K Q^T.  A row's scores therefore live in four lanes of each of two
// waves, 2 NT registers per lane, and never leave registers.
//
//  1. S^T = K Q^T on MFMA; K is staged through LDS in chunks that the eight
//     waves share.
//  2. Per row: max and min, weights w = exp(s - max), Z; then the certified
//     cut by a mass-weighted bin descent: fp64 LDS histograms of weight mass
//     over 64 bins per row (equal-width value bins first, bins over the
//     order-preserving integer encoding of the score below that), each level
//     keeping the one bin that holds the cut.  It ends exactly, either by
//     pairwise key comparison once a row has <= 48 candidates, or by index
//     rank when all remaining candidates share one score.
//  3. out^T = V^T P^T on MFMA, V staged transposed through LDS.  P holds the
//     head weights split into bf16 high and low parts, so the products carry
//     about 16 bits of weight precision; accumulation is fp32.
#include "device_common.h"
#include "kernels.h"

namespace ctopk {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kEncGroups = 2;             // row groups of 16 rows
constexpr int kEncWaves = 2 * kEncGroups; // x 2 key halves
constexpr int kEncThreads = kEncWaves * kWave;
constexpr int kEncRows = 16 * kEncGroups; // query rows per workgroup
constexpr int kEncMaxKeys = 512;
constexpr int kEncMinGroup = 64;
constexpr int kEncBins = 64;              // bins per row and level
constexpr int kHistStride = kEncBins + 1; // doubles per histogram row (bank padding)
constexpr int kLaneCand = 10;             // candidate slots per lane
constexpr int kLaneSlots = kLaneCand + 1; // plus one slot that takes every other write
constexpr int kFinishMax = 48;            // exact finish at or below this many candidates
// Every level below the first drops at least one candidate, so n levels suffice.
constexpr int kMaxLevels = 2 * kEncMaxKeys;

// A row's finish list: up to kFinishMax (key64, weight) entries, one 16-byte
// word each, rows kFinStride words apart (the pad keeps the 16 rows' entry j
// in different banks).
constexpr int kFinStride = kFinishMax + 1;
struct GroupSel {  // select scratch of one row group (two waves), aliased with the stages
  double hist[16 * kHistStride];
  uint64_t key[2 * kWave * kLaneSlots];
  uint4 fin[16 * kFinStride];
};
struct GroupXchg {  // per-row values the two waves of a row group exchange
  float f[2][16][4];   // max, min, candidate min, candidate max
  int i[2][16][4];     // candidate count, overflow flag, head count
  uint64_t k[2][16];   // best key
  double d[2][16];     // its lower mass
  int lcnt[2][kWave];  // candidates per lane
  uint32_t bm[16][16]; // candidate bitmap per row (tied scores)
};
// The K and V stages (at most 2 x 256 x 72 bf16) share the buffer with the
// select scratch of the row groups.
constexpr int kEncStage = 2 * 256 * 72 * 2;
constexpr int kEncSelect = kEncGroups * static_cast<int>(sizeof(GroupSel));
constexpr int kEncSmem = kEncSelect > kEncStage ? kEncSelect : kEncStage;

template <int D>
struct Geo {
  static constexpr int kChunk = D == 64 ? 256 : 64;  // keys per staged chunk and half
  static constexpr int kKStride = D + 8;              // bf16 per staged K row
};
static_assert(2 * Geo<64>::kChunk * Geo<64>::kKStride * 2 <= kEncSmem, "K stage");
static_assert(2 * 64 * (Geo<64>::kChunk + 8) * 2 <= kEncSmem, "V stage");
static_assert(2 * Geo<128>::kChunk * Geo<128>::kKStride * 2 <= kEncSmem, "K stage");
static_assert(2 * 128 * (Geo<128>::kChunk + 8) * 2 <= kEncSmem, "V stage");
static_assert(kEncGroups * 16 * 128 * 4 <= kEncSmem, "half combine");

// Reductions over the four lanes (r, 0..3) of a row within one wave (lanes
// r + 16 g), with the cross-row swaps; every lane of the wave must be active.
template <typename Op>
__device__ __forceinline__ uint32_t row_reduce(uint32_t v, Op op) {
  uint2 p = lane_pair<16>(v);
  v = op(p.x, p.y);
  p = lane_pair<32>(v);
  return op(p.x, p.y);
}
__device__ __forceinline__ float row_max(float v) {
  return __uint_as_float(row_reduce(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
__device__ __forceinline__ float row_min(float v) {
  return __uint_as_float(row_reduce(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fminf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
__device__ __forceinline__ int row_sum(int v) {
  return static_cast<int>(
      row_reduce(static_cast<uint32_t>(v), [](uint32_t a, uint32_t b) { return a + b; }));
}
__device__ __forceinline__ uint32_t row_or(uint32_t v) {
  return row_reduce(v, [](uint32_t a, uint32_t b) { return a | b; });
}

// Bin of a score at one level.  Both forms are non-decreasing in s, so every
// bin holds a contiguous range of the key order.  fmaxf also maps the -inf of
// absent keys (weight 0) to bin 0.
__device__ __forceinline__ int value_bin(float s, float lo, float inv) {
  const float x = fmaxf((s - lo) * inv, 0.0f);
  return x < static_cast<float>(kEncBins) ? static_cast<int>(x) : kEncBins - 1;
}
__device__ __forceinline__ int ukey_bin(float s, uint32_t ulo, float inv) {
  const float x = static_cast<float>(ukey(s) - ulo) * inv;
  return x < static_cast<float>(kEncBins) ? static_cast<int>(x) : kEncBins - 1;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// weight as bf16 high part (low half-word) and bf16 residual (high half-word)
__device__ __forceinline__ uint32_t pack_weight(float w) {
  const __bf16 wh = static_cast<__bf16>(w);
  const __bf16 wl = static_cast<__bf16>(w - static_cast<float>(wh));
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, wh)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, wl)) << 16);
}

// Two floats rounded to bf16 (nearest even) in one word, the first in the low
// half-word: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2v_t));
}

// The weight e^{s - m} for the output pass when level 0's packed weights do
// not fit in registers: one hardware base-2 exponential of the fp32
// (s - m) * log2(e).  Its relative error (about |s - m| * 2^-23 plus the
// instruction's own) stays below the 2^-17 to which the packed bf16 high and
// low parts carry any weight into the MFMA, for every weight above e^-16 of
// the row maximum; the head's mass Z - R, by which the sums are divided,
// still comes from the select's exact weights.
__device__ __forceinline__ float output_weight(float s, float m) {
  constexpr float kLog2e = 1.44269502162933349609375f;
  return __builtin_amdgcn_exp2f((s - m) * kLog2e);
}

template <int D, int NT>
__global__ __launch_bounds__(kEncThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void encoder_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const float* __restrict__ head_scale, float default_scale,
    int n, int G, double eps, float* __restrict__ out, int32_t* __restrict__ k_eps,
    double* __restrict__ tau, uint32_t* __restrict__ sel_mask, float* __restrict__ scores_out,
    double* __restrict__ lse) {
  using Gm = Geo<D>;
  constexpr int NTH = NT / 2;                             // tiles per key half
  constexpr int H = 16 * NTH;                             // keys per half
  constexpr int CK = H < Gm::kChunk ? H : Gm::kChunk;     // keys per staged chunk
  constexpr int TPC = CK / 16;                            // tiles per chunk
  constexpr int NCH = H / CK;                             // chunks per half
  constexpr int KS = Gm::kKStride;
  constexpr int VS = CK + 4;                              // bf16 per staged V^T row
  static_assert(H % CK == 0 && TPC % 2 == 0, "chunking");
  __shared__ __align__(16) unsigned char smem[kEncSmem];
  __shared__ GroupXchg xs[kEncGroups];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rg = wave >> 1, kh = wave & 1;  // row group, key half
  const int r = lane & 15, g = lane >> 4;
  // Workgroups are dealt to the 8 XCDs round robin by id; when the count
  // allows, give every row tile of one head the same id mod 8, so that head's
  // K and V are fetched into one XCD's L2 instead of eight.
  const int tiles = (G + kEncRows - 1) / kEncRows;
  const int nwg = static_cast<int>(gridDim.x);
  const int lin = (nwg % 8 == 0 && (nwg / 8) % tiles == 0)
                      ? static_cast<int>(blockIdx.x % 8) * (nwg / 8) + static_cast<int>(blockIdx.x / 8)
                      : static_cast<int>(blockIdx.x);
  const int h = lin / tiles;
  const int qr = (lin % tiles) * kEncRows + rg * 16 + r;
  const bool row_ok = qr < G;
  const int64_t row = static_cast<int64_t>(h) * G + (row_ok ? qr : G - 1);
  const float scale = head_scale ? head_scale[row] : default_scale;
  const uint16_t* Kh = K + static_cast<size_t>(h) * n * D;
  const uint16_t* Vh = V + static_cast<size_t>(h) * n * D;
  GroupXchg& xg = xs[rg];
  const int kbase = kh * H;  // this wave's keys: kbase + 16 t + 4 g + e, t < NTH
  // Key kbase + 16 t + 4 g + e exists iff 16 t + e < nl; tests against nl compare a
  // constant with one register instead of materialising per-key indices.
  int nl = n - kbase - 4 * g;

  // ---- 1. scores: S^T tile t = K[16t .. 16t+15] Q^T on MFMA
  bf16x8_t qf[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
    qf[c] = as_bf16x8(*reinterpret_cast<const uint4*>(q + row * D + 32 * c + 8 * g));

  float s[NTH][4];
  float mx = -INFINITY, mn = INFINITY;  // lane-local, over existing keys
  int nlq = nl;
  asm volatile("" : "+v"(nlq));  // existence masks stay local to this phase
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem);  // [2 halves][CK][KS]
#pragma unroll
  for (int cc = 0; cc < NCH; ++cc) {
    if (cc > 0) __syncthreads();
    constexpr int kUnitsH = CK * D / 8;  // 16-byte units per half chunk
#pragma unroll
    for (int u0 = 0; u0 < 2 * kUnitsH; u0 += kEncThreads) {
      const int u = u0 + tid;
      if (2 * kUnitsH % kEncThreads == 0 || u < 2 * kUnitsH) {
        const int hh = u / kUnitsH, rem = u % kUnitsH;
        const int rr = rem / (D / 8), c8 = rem % (D / 8);
        const int src = min(hh * H + cc * CK + rr, n - 1);
        *reinterpret_cast<uint4*>(Ks + (hh * CK + rr) * KS + c8 * 8) =
            *reinterpret_cast<const uint4*>(Kh + static_cast<size_t>(src) * D + c8 * 8);
      }
    }
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < TPC; ++tt) {
      const int t = cc * TPC + tt;
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        const bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4*>(
            Ks + (kh * CK + tt * 16 + r) * KS + 32 * c + 8 * g));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[c], acc, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool live = 16 * t + e < nlq;
        s[t][e] = live ? acc[e] * scale : -INFINITY;
        mx = fmaxf(mx, s[t][e]);
        mn = live ? fminf(mn, s[t][e]) : mn;
      }
    }
  }

  // ---- 2. the certified cut, per row (both waves of a row group agree on it)
  mx = row_max(mx);
  mn = row_min(mn);
  if (g == 0) {
    xg.f[kh][r][0] = mx;
    xg.f[kh][r][1] = mn;
  }
  __syncthreads();  // the K stage is free: it becomes the select scratch
  GroupSel& gs = reinterpret_cast<GroupSel*>(smem)[rg];
  double* hrow = gs.hist + r * kHistStride;
  mx = fmaxf(xg.f[0][r][0], xg.f[1][r][0]);
  mn = fminf(xg.f[0][r][1], xg.f[1][r][1]);
  if (kh == 0) {
#pragma unroll
    for (int j = 0; j < 16; ++j) hrow[16 * g + j] = 0.0;
  }
  __syncthreads();
  // Level 0: the mass histogram over equal-width value bins on [mn, mx], and
  // every weight kept, packed, for the output pass.
  const float vrng = mx - mn;
  float vinv = static_cast<float>(kEncBins) / vrng;
  vinv = (vrng > 0.0f && isfinite(vinv)) ? vinv : 0.0f;
  // Scores more than 200 below the maximum have weight 0 in fp32 (exp
  // underflows below -104), so clamping there changes no weight; it maps the
  // -inf of absent keys to weight 0 without a branch.
  const float wfloor = mx - 200.0f;
  // Packed weights are kept for the output pass when registers allow.
  constexpr bool kKeepW = NTH <= 8;
  uint32_t pw[kKeepW ? NTH : 1][4];
#pragma unroll
  for (int t = 0; t < NTH; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = s[t][e];
      const float w = weight(fmaxf(v, wfloor), mx);
      atomicAdd(hrow + value_bin(v, mn, vinv), static_cast<double>(w));
      if constexpr (kKeepW) pw[t][e] = pack_weight(w);
    }
  __syncthreads();
  // Z = the histogram's total, summed in one fixed order by every lane of a row.
  double zp = 0.0;
#pragma unroll
  for (int j = 0; j < 16; ++j) zp += hrow[16 * g + j];
  const double Z = xrow32_sum(xrow16_sum(zp));  // (g0 + g1) + (g2 + g3)
  const double thr = eps * Z;

  bool active = true;
  double P = 0.0;            // mass of the keys below the current interval
  float ilo = mn, ihi = mx;  // closed score interval known to hold the cut key
  uint64_t cut = 0;
  double R = 0.0;
  uint64_t* klist = gs.key + (kh * kWave + lane) * kLaneSlots;

  for (int level = 0; level < kMaxLevels; ++level) {
    // Opaque to the optimiser: keeps per-key values derived from s from being
    // hoisted out of the level loop.
#pragma unroll
    for (int t = 0; t < NTH; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(s[t][e]));
    const uint32_t ulo = ukey(ilo);
    float uinv = 0.0f;
    if (level > 0) {  // histogram of the interval over bins of the integer encoding
      uinv = static_cast<float>(kEncBins) / (static_cast<float>(ukey(ihi) - ulo) + 1.0f);
      if (kh == 0) {
#pragma unroll
        for (int j = 0; j < 16; ++j) hrow[16 * g + j] = 0.0;
      }
      __syncthreads();
#pragma unroll
      for (int t = 0; t < NTH; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = s[t][e];
          if (active && v >= ilo && v <= ihi)
            atomicAdd(hrow + ukey_bin(v, ulo, uinv), static_cast<double>(weight(v, mx)));
        }
      __syncthreads();
    }

    // The bin holding the cut: the largest b whose mass below is <= thr.
    // (the lane's 16 bins are read twice from LDS rather than held in registers)
    double S = 0.0;
#pragma unroll
    for (int j = 0; j < 16; ++j) S += hrow[16 * g + j];
    // the row's partial sums of the four lanes g = 0..3, in every lane
    const double Sx = xor_lane<16>(S);               // lane g ^ 1
    const double Sa = (g & 1) ? Sx : S;              // lane g & 2
    const double Sb = (g & 1) ? S : Sx;              // lane (g & 2) + 1
    const double Sa2 = xor_lane<32>(Sa), Sb2 = xor_lane<32>(Sb);
    const double S0 = g < 2 ? Sa : Sa2, S1 = g < 2 ? Sb : Sb2, S2 = g < 2 ? Sa2 : Sa;
    double Pc = P;
    if (g > 0) Pc += S0;
    if (g > 1) Pc += S1;
    if (g > 2) Pc += S2;
    int best = -1;
    double bestP = 0.0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (Pc <= thr) {
        best = 16 * g + j;
        bestP = Pc;
      }
      Pc += hrow[16 * g + j];
    }
    {
      const int ob = xor_lane<16>(best);
      const double oP = xor_lane<16>(bestP);
      if (ob > best) {
        best = ob;
        bestP = oP;
      }
    }
    {
      const int ob = xor_lane<32>(best);
      const double oP = xor_lane<32>(bestP);
      if (ob > best) {
        best = ob;
        bestP = oP;
      }
    }

    // Candidates: the keys of that bin.  Branch-free: every key is written,
    // those outside the bin (and any past kLaneCand) into the lane's spare
    // slot; entries hold (index, score bits).
    int kofs = kbase + 4 * g;
    asm volatile("" : "+v"(kofs));  // recomputed per use, not held per key
    int cnt = 0;
    float cmn = INFINITY, cmx = -INFINITY;
#pragma unroll
    for (int t = 0; t < NTH; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = s[t][e];
        const bool in = active && v >= ilo && v <= ihi &&
                        (level == 0 ? value_bin(v, mn, vinv) : ukey_bin(v, ulo, uinv)) == best;
        klist[in ? min(cnt, kLaneCand) : kLaneCand] =
            (static_cast<uint64_t>(kofs + 16 * t + e) << 32) | __float_as_uint(v);
        cnt += in ? 1 : 0;
        cmn = fminf(cmn, in ? v : INFINITY);
        cmx = fmaxf(cmx, in ? v : -INFINITY);
      }
    xg.lcnt[kh][lane] = cnt;
    {
      const int c = row_sum(cnt);
      const int o = row_sum(cnt > kLaneCand ? 1 : 0);
      const float a = row_min(cmn), b = row_max(cmx);
      if (g == 0) {
        xg.i[kh][r][0] = c;
        xg.i[kh][r][1] = o;
        xg.f[kh][r][2] = a;
        xg.f[kh][r][3] = b;
      }
    }
    __syncthreads();
    const int ctot = xg.i[0][r][0] + xg.i[1][r][0];
    const int over = xg.i[0][r][1] + xg.i[1][r][1];
    cmn = fminf(xg.f[0][r][2], xg.f[1][r][2]);
    cmx = fmaxf(xg.f[0][r][3], xg.f[1][r][3]);
    const bool fin_list = active && over == 0 && ctot <= kFinishMax;
    const bool fin_eq = active && !fin_list && cmn == cmx;

    // Exact finish on <= kFinishMax candidates: the cut is the largest candidate key
    // whose strictly smaller keys carry mass <= thr.  The row's candidates go
    // into one list (each lane's after those of the row's lanes before it),
    // and lane (kh, g) of the row tests candidates 4 kh + g, + 8, ...
    // against the whole list.
    if (fin_list) {
      int off = 0;
#pragma unroll
      for (int li = 0; li < 8; ++li)
        off += li < 4 * kh + g ? xg.lcnt[li >> 2][r + 16 * (li & 3)] : 0;
      uint4* dst = gs.fin + r * kFinStride + off;
      for (int y = 0; y < cnt; ++y) {
        const uint64_t en = klist[y];
        const float v = __uint_as_float(static_cast<uint32_t>(en));
        const uint64_t kk = key64(v, static_cast<uint32_t>(en >> 32));
        dst[y] = make_uint4(static_cast<uint32_t>(kk), static_cast<uint32_t>(kk >> 32),
                            __float_as_uint(weight(v, mx)), 0u);
      }
    }
    // Equal scores: the candidates differ only in index; rank by index.
    if (fin_eq && kh == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) xg.bm[r][4 * g + j] = 0u;
    }
    __syncthreads();
    if (fin_list) {
      const uint4* lst = gs.fin + r * kFinStride;
      uint64_t bk = 0;
      double bR = 0.0;
      for (int c = 4 * kh + g; c < ctot; c += 8) {
        const uint4 ec = lst[c];
        const uint64_t kc = (static_cast<uint64_t>(ec.y) << 32) | ec.x;
        double ml = 0.0;
        for (int j = 0; j < ctot; ++j) {
          const uint4 ej = lst[j];
          const uint64_t kj = (static_cast<uint64_t>(ej.y) << 32) | ej.x;
          if (kj < kc) ml += static_cast<double>(__uint_as_float(ej.z));
        }
        const double Pm = bestP + ml;
        if (Pm <= thr && kc > bk) {
          bk = kc;
          bR = Pm;
        }
      }
#pragma unroll
      for (int off = 16; off <= 32; off <<= 1) {
        const uint64_t ok = __shfl_xor(bk, off, kWave);
        const double oR = __shfl_xor(bR, off, kWave);
        if (ok > bk) {
          bk = ok;
          bR = oR;
        }
      }
      if (g == 0) {
        xg.k[kh][r] = bk;
        xg.d[kh][r] = bR;
      }
    }
    if (fin_eq) {
      int kb = kbase + 4 * g;
      asm volatile("" : "+v"(kb));  // per-key bits are recomputed, not kept across levels
#pragma unroll
      for (int t = 0; t < NTH; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = kb + 16 * t + e;
          if (s[t][e] == cmn) atomicOr(&xg.bm[r][key >> 5], 1u << (key & 31));
        }
    }
    __syncthreads();
    if (fin_list) {
      const uint64_t k0 = xg.k[0][r], k1 = xg.k[1][r];
      cut = k1 > k0 ? k1 : k0;
      R = k1 > k0 ? xg.d[1][r] : xg.d[0][r];
    }
    if (fin_eq) {
      // The tail takes the tied candidates from the highest index down; j of
      // them fit under thr beside the mass below, so the cut is the one of
      // rank j counted from the highest index.
      const double wc = static_cast<double>(weight(cmn, mx));
      int j = ctot - 1;
      if (wc > 0.0) {
        const double qj = floor((thr - bestP) / wc);
        j = qj < static_cast<double>(ctot - 1) ? static_cast<int>(qj) : ctot - 1;
        if (j < 0) j = 0;
        while (j + 1 < ctot && bestP + (j + 1) * wc <= thr) ++j;
        while (j > 0 && bestP + j * wc > thr) --j;
      }
      int idx = 0;
      if (g == 0) {
        int rem = j;
        for (int wd = 15; wd >= 0; --wd) {
          uint32_t word = xg.bm[r][wd];
          const int c = __popc(word);
          if (rem < c) {
            for (int b = 0; b < 32; ++b) {
              const int hb = 31 - __clz(word);
              if (rem == 0) {
                idx = 32 * wd + hb;
                break;
              }
              word &= ~(1u << hb);
              --rem;
            }
            break;
          }
          rem -= c;
        }
      }
      idx = __shfl(idx, r, kWave);
      cut = key64(cmn, static_cast<uint32_t>(idx));
      R = bestP + j * wc;
    }
    if (active && !fin_list && !fin_eq) {  // descend into the bin
      P = bestP;
      ilo = cmn;
      ihi = cmx;
    }
    active = active && !fin_list && !fin_eq;
    // block-uniform exit; also orders this level's reads before the next
    // level's histogram reset
    if (__syncthreads_or(active ? 1 : 0) == 0) break;
  }
  const bool failed = active;  // not reached: each level drops a candidate

  // ---- 3. head-only output: out^T = V^T P^T over this wave's key half
  __syncthreads();  // select scratch becomes the V^T stage
  const float cs = key64_score(cut);
  // head iff s > cs or (s == cs and 16 t + e <= cil)
  const int cil = static_cast<int>(key64_index(cut)) - kbase - 4 * g;
  const uint32_t gbit = 1u << (4 * g);
  const int nw = (n + 31) >> 5;
  f32x4_t acc[D / 16];
#pragma unroll
  for (int f = 0; f < D / 16; ++f) acc[f] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  int kc = 0;
  uint16_t* Vt = reinterpret_cast<uint16_t*>(smem);  // [2 halves][D][VS]
#pragma unroll
  for (int cc = 0; cc < NCH; ++cc) {
    if (cc > 0) __syncthreads();
    // Stage V rows of chunk cc of both halves as V^T: two keys per 32-bit word.
    constexpr int kOct = D / 8;
    constexpr int kItemsH = (CK / 2) * kOct;
#pragma unroll
    for (int i0 = 0; i0 < 2 * kItemsH; i0 += kEncThreads) {
      const int it = i0 + tid;
      if (2 * kItemsH % kEncThreads == 0 || it < 2 * kItemsH) {
        const int hh = it / kItemsH, rem = it % kItemsH;
        const int fo = rem % kOct, kp = rem / kOct;
        const int k0 = min(hh * H + cc * CK + 2 * kp, n - 1);
        const int k1 = min(hh * H + cc * CK + 2 * kp + 1, n - 1);
        const uint4 a = *reinterpret_cast<const uint4*>(Vh + static_cast<size_t>(k0) * D + 8 * fo);
        const uint4 b = *reinterpret_cast<const uint4*>(Vh + static_cast<size_t>(k1) * D + 8 * fo);
        const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
        uint32_t* dst = reinterpret_cast<uint32_t*>(Vt + (hh * D + 8 * fo) * VS + 2 * kp);
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          dst[(2 * f) * (VS / 2)] = (av[f] & 0xFFFFu) | (bv[f] << 16);
          dst[(2 * f + 1) * (VS / 2)] = (av[f] >> 16) | (bv[f] & 0xFFFF0000u);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int st = 0; st < TPC / 2; ++st) {
      const int t0 = cc * TPC + 2 * st;
      uint32_t ph[4], pl[4];
      uint32_t bits = 0;
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          uint32_t p2[2];
          float w2[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const float v = s[t0 + half][e + k];
            const bool head = v > cs || (v == cs && 16 * (t0 + half) + e + k <= cil);
            kc += head ? 1 : 0;
            bits |= head ? (gbit << (16 * half + e + k)) : 0u;
            if constexpr (kKeepW)
              p2[k] = head ? pw[t0 + half][e + k] : 0u;
            else
              w2[k] = head ? output_weight(v, mx) : 0.0f;
          }
          if constexpr (kKeepW) {
            ph[2 * half + e / 2] = (p2[0] & 0xFFFFu) | (p2[1] << 16);
            pl[2 * half + e / 2] = (p2[0] >> 16) | (p2[1] & 0xFFFF0000u);
          } else {
            // both keys' high parts in one conversion, then both residuals
            const uint32_t hi = bf16_pair(w2[0], w2[1]);
            ph[2 * half + e / 2] = hi;
            pl[2 * half + e / 2] = bf16_pair(w2[0] - __uint_as_float(hi << 16),
                                             w2[1] - __uint_as_float(hi & 0xFFFF0000u));
          }
        }
      const bf16x8_t bh = as_bf16x8(make_uint4(ph[0], ph[1], ph[2], ph[3]));
      const bf16x8_t bl = as_bf16x8(make_uint4(pl[0], pl[1], pl[2], pl[3]));
#pragma unroll
      for (int f = 0; f < D / 16; ++f) {
        const uint16_t* vr = Vt + (kh * D + 16 * f + r) * VS + 32 * st + 4 * g;
        const uint2 lo2 = *reinterpret_cast<const uint2*>(vr);
        const uint2 hi2 = *reinterpret_cast<const uint2*>(vr + 16);
        const bf16x8_t av = as_bf16x8(make_uint4(lo2.x, lo2.y, hi2.x, hi2.y));
        acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bh, acc[f], 0, 0, 0);
        acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bl, acc[f], 0, 0, 0);
      }
      if (sel_mask) {
        bits = row_or(bits);
        const int wd = kbase / 32 + cc * (TPC / 2) + st;
        if (row_ok && g == 0 && wd < nw) sel_mask[row * nw + wd] = bits;
      }
    }
  }
  kc = row_sum(kc);
  if (g == 0) xg.i[kh][r][2] = kc;
  // Add the two halves: the upper half's wave hands its sums over through LDS.
  __syncthreads();
  float* comb = reinterpret_cast<float*>(smem) + rg * 16 * D;  // [16 rows][D]
  if (kh == 1) {
#pragma unroll
    for (int f = 0; f < D / 16; ++f)
      *reinterpret_cast<float4*>(comb + r * D + 16 * f + 4 * g) =
          make_float4(acc[f][0], acc[f][1], acc[f][2], acc[f][3]);
  }
  __syncthreads();
  if (scores_out && row_ok) {
    float* srow = scores_out + row * n + kbase + 4 * g;
    asm volatile("" : "+v"(nl));
#pragma unroll
    for (int t = 0; t < NTH; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (16 * t + e < nl) srow[16 * t + e] = s[t][e];
      }
  }
  if (kh == 1 || !row_ok) return;
  const double den = Z - R;  // head mass
  const float invd = static_cast<float>(1.0 / den);
#pragma unroll
  for (int f = 0; f < D / 16; ++f) {
    const float4 o = *reinterpret_cast<const float4*>(comb + r * D + 16 * f + 4 * g);
    *reinterpret_cast<float4*>(out + row * D + 16 * f + 4 * g) =
        make_float4((acc[f][0] + o.x) * invd, (acc[f][1] + o.y) * invd, (acc[f][2] + o.z) * invd,
                    (acc[f][3] + o.w) * invd);
  }
  if (g == 0) {
    k_eps[row] = failed ? -1 : xg.i[0][r][2] + xg.i[1][r][2];
    tau[row] = R / Z;
    if (lse) lse[row] = static_cast<double>(mx) + log(Z);
  }
}

template <int D, int NT>
hipError_t launch_t(const void* q, const void* K, const void* V, const float* head_scale,
                    float default_scale, int n, int G, int n_kv, double eps, float* out,
                    int32_t* k_eps, double* tau, uint32_t* sel_mask, float* scores, double* lse,
                    hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(ceil_div(G, kEncRows) * n_kv));
  return launch(encoder_kernel<D, NT>, grid, dim3(kEncThreads), 0, st,
                static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(K),
                static_cast<const uint16_t*>(V), head_scale, default_scale, n, G, eps, out, k_eps,
                tau, sel_mask, scores, lse);
}

template <int D>
hipError_t launch_d(const void* q, const void* K, const void* V, const float* head_scale,
                    float default_scale, int n, int G, int n_kv, double eps, float* out,
                    int32_t* k_eps, double* tau, uint32_t* sel_mask, float* scores, double* lse,
                    hipStream_t st) {
  if (n <= 128)
    return launch_t<D, 8>(q, K, V, head_scale, default_scale, n, G, n_kv, eps, out, k_eps, tau,
                          sel_mask, scores, lse, st);
  if (n <= 256)
    return launch_t<D, 16>(q, K, V, head_scale, default_scale, n, G, n_kv, eps, out, k_eps,
                           tau, sel_mask, scores, lse, st);
  return launch_t<D, 32>(q, K, V, head_scale, default_scale, n, G, n_kv, eps, out, k_eps, tau,
                         sel_mask, scores, lse, st);
}

}  // namespace

bool encoder_supported(int dtype, int d, int64_t n, int n_q, int n_kv) {
  return dtype == 1 && (d == 64 || d == 128) && n >= 1 && n <= kEncMaxKeys && n_kv >= 1 &&
         n_q % n_kv == 0 && n_q / n_kv >= kEncMinGroup;
}

hipError_t launch_encoder(const void* q, const void* K, const void* V, int d,
                          const float* head_scale, float default_scale, int64_t n, int n_q,
                          int n_kv, double eps, float* out, int32_t* k_eps, double* tau,
                          uint32_t* sel_mask, float* scores, double* lse, hipStream_t st) {
  if (!encoder_supported(1, d, n, n_q, n_kv)) return hipErrorInvalidValue;
  const int G = n_q / n_kv;
  if (d == 64)
    return launch_d<64>(q, K, V, head_scale, default_scale, static_cast<int>(n), G, n_kv, eps,
                        out, k_eps, tau, sel_mask, scores, lse, st);
  return launch_d<128>(q, K, V, head_scale, default_scale, static_cast<int>(n), G, n_kv, eps, out,
                       k_eps, tau, sel_mask, scores, lse, st);
}

}  // namespace ctopk
