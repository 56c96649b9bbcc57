// Host-side launchers of the libctopk kernels (internal interface; the public
// C ABI is include/ctopk.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "device_common.h"

namespace ctopk {

// Keys per block of the score scan; per-block maxima are emitted per tile.
constexpr int kScanTile = 256;
// Scores per block of the first (global) histogram pass.
constexpr int kHistChunk = 4096;
// Keys per block of the value stream.
constexpr int kVsumTile = 256;
// Largest candidate set the resolve kernel keeps in LDS.
constexpr int kCandCap = 8192;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// K1: scores[h, i] = scale_h * <q_h, K[h / G, i]> and blkmax[h, tile].
// Also zeroes `zero_bytes` at `zero_base` (the histogram scratch).
hipError_t launch_score_scan(const void* q, const void* K, int dtype, int d,
                             const float* head_scale, float default_scale, int64_t n,
                             int n_q, int n_kv, float* scores, float* blkmax,
                             void* zero_base, size_t zero_bytes, hipStream_t st);

// Row maxima of given logits, per chunk of keys: blkmax[row, chunk].
int rowmax_nblk(int64_t n);
hipError_t launch_rowmax(const float* logits, int64_t n, int rows, float* blkmax,
                         void* zero_base, size_t zero_bytes, hipStream_t st);

// Pass 1 of the select: row max m from blkmax, weights w = exp(s - m), and the
// top-digit (count, mass) histogram of every row, merged with global atomics.
hipError_t launch_hist0(const float* scores, int64_t n, int rows, const float* blkmax,
                        int nblk, RowSel* rs, uint32_t* hcnt, double* hmass, hipStream_t st);

// Remaining select levels, one workgroup per row: k_eps, tau, lse, thr.
hipError_t launch_resolve(const float* scores, int64_t n, int rows, const uint32_t* hcnt,
                          const double* hmass, double eps, RowSel* rs, int32_t* k_eps,
                          double* tau, double* lse, hipStream_t st);

// Number of key chunks the value stream splits each row into.
int vsum_nchunk(int64_t n, int rows, int n_v);
// K4: per-chunk partial sums of w * v over kept keys, and the selection mask.
hipError_t launch_vsum(const float* scores, int64_t n, int rows, int n_v, const void* V,
                       int v_dtype, int dv, const RowSel* rs, float* part, int nchunk,
                       uint32_t* sel_mask, hipStream_t st);

// Combine the per-chunk partials (fp64, fixed order) into out = num / den.
hipError_t launch_finalize(const float* part, int rows, int nchunk, int dv, float* out,
                           hipStream_t st);

// Encoder-shaped path (all queries of a head, n <= 1024, bf16, MFMA QK^T).
hipError_t launch_encoder(const void* q, const void* K, const void* V, int d,
                          const float* head_scale, float default_scale, int64_t n, int n_q,
                          int n_kv, double eps, float* out, int32_t* k_eps, double* tau,
                          uint32_t* sel_mask, float* scores, double* lse, hipStream_t st);
bool encoder_supported(int dtype, int d, int64_t n, int n_q, int n_kv);

}  // namespace ctopk
