// Host-side launchers of the libctopk kernels (internal interface; the public
// C ABI is include/ctopk.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "device_common.h"

namespace ctopk {

// Compute units of an MI355X.
constexpr int kNumCUs = 256;
// Keys per tile (one workgroup) of the score scan; its (min, max) is emitted
// per tile.  64 keys per 4-wave group measured fastest on MI355X (more, shorter
// workgroups keep more loads in flight across the chip).
constexpr int kScanTile = 64;
// Keys per tile of the value stream (8 waves x 32 keys).
constexpr int kVsumTile = 256;
// Largest candidate set the resolve kernel keeps in LDS.
constexpr int kCandCap = 8192;
// Most keys per chunk of the value stream of the overlapped decode plan (the
// keys its correction needs are listed in LDS).
constexpr int kFixKeys = 2048;
// Most score-scan tiles per row for the blockwise bound (staged in LDS).
constexpr int kBoundMaxTiles = 4096;

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Instrumentation: pops the next (start, stop) event pair armed for the
// current call on this host thread (ctopk_record_kernel_events); false if none.
bool take_kernel_events(hipEvent_t* start, hipEvent_t* stop);
// For a kernel of the path that a call does not need: records its armed pair
// (if any) back to back on st, so pairs stay aligned with the path's kernels.
void skip_kernel_events(hipStream_t st);

// Every kernel of the library is launched through here.  With an armed event
// pair the events are attached to the dispatch itself, so they time exactly
// the kernel's execution (no marker packets in between).
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shmem,
                  hipStream_t st, Args... args) {
  hipEvent_t a = nullptr, b = nullptr;
  if (take_kernel_events(&a, &b))
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, a, b, 0, static_cast<KArgs>(args)...);
  else
    hipLaunchKernelGGL(kernel, grid, block, shmem, st, static_cast<KArgs>(args)...);
  return hipGetLastError();
}

// K1: scores[h, i] = scale_h * <q_h, K[h / G, i]> and blkstat[h, tile] =
// (min, max) over the tile; with blkz non-NULL also blkz[h, tile] = the sum
// over the tile of exp(s - its max).  Also zeroes `zero_bytes` at `zero_base`
// and `zero_bytes2` at `zero_base2` (multiples of 16 bytes; NULL: nothing).
hipError_t launch_score_scan(const void* q, const void* K, int dtype, int d,
                             const float* head_scale, float default_scale, int64_t n,
                             int n_q, int n_kv, float* scores, float2* blkstat, float* blkz,
                             void* zero_base, size_t zero_bytes, void* zero_base2,
                             size_t zero_bytes2, hipStream_t st);

// Level 0 of the select for long decode rows, many blocks per row: row
// (min, max) from blkstat, weights w = exp(s - max), and an fp64 mass
// histogram over kBins equal-width value bins on [min, max] per chunk of keys,
// written to pmass [rows, hist_nchunk, kBins].
int hist_nchunk(int64_t n, int rows);
// Rows up to this many keys are held in registers by the select's block, which
// then builds level 0 itself (no hist0 pass and no partial histograms).
int resolve_register_row();
hipError_t launch_hist0(const float* scores, int64_t n, int rows, const float2* blkstat,
                        int nblk, int nchunk, double* pmass, hipStream_t st);

// Select, one workgroup per row: level-0 mass histogram from the hist0
// partials (or, with npart == 0, from a pass over the row, which the block
// holds in registers when n <= resolve_register_row(); a (min, max) pass
// first when blkstat is NULL), then the radix levels.  Writes k_eps, tau, lse (optional),
// sel_mask (optional) and RowSel.  Also zeroes `zero_bytes` at `zero_base`.
hipError_t launch_resolve(const float* scores, int64_t n, int rows, const float2* blkstat,
                          int nblk, const double* pmass, int npart,
                          double eps, RowSel* rs, int32_t* k_eps, double* tau, double* lse,
                          uint32_t* sel_mask, void* zero_base, size_t zero_bytes,
                          hipStream_t st);

// Blocks per group (nchunk) and groups of the value stream.
int vsum_groups(int rows, int n_v, int v_dtype, int dv);
int vsum_nchunk(int64_t n, int rows, int n_v, int v_dtype, int dv);
// K4: w * v over kept keys into part [rows, nchunk, dv + 1] (numerator and
// weight sum per block), then a finalize kernel writes out = num / den.  With
// dense, err or var non-NULL the tail and sum w ||v||^2 are accumulated too
// (part [rows, nchunk, 2 (dv + 1) + 1]) and the finalize also writes the
// untruncated output, the output error ||Attn - Attn_k||_2 and Var_P(V) per
// row (each only where its pointer is non-NULL).
hipError_t launch_vsum(const float* scores, int64_t n, int rows, int n_v, const void* V,
                       int v_dtype, int dv, const RowSel* rs, float* part, int nchunk, float* out,
                       float* dense, double* err, double* var, hipStream_t st);

// Chunks per group for about `blocks` workgroups in total (whole tiles of
// kVsumTile keys per chunk, never more chunks than tiles).
int stream_nchunk(int64_t n, int groups, int blocks);

// Decode rows the select holds in registers can run beside the value stream
// in one launch: select_spec_nchunk gives that stream's chunks per group (0
// when the shape does not qualify: rows of 16K..32K keys, at least half of
// the compute units left beside the rows' workgroups, and chunks of at most
// kFixKeys keys).  launch_select_spec runs the select (as launch_resolve with
// register rows; each row's head mass and cut are published in pub[row]) and
// a stream over a provisional head per chunk, corrected by the exact cut,
// whose chunk sums are added, divided by the head mass, into out with
// device-scope float atomics.  pub [rows] and out must be zero at launch.
int select_spec_nchunk(int64_t n, int rows, int n_v, int v_dtype, int dv);
hipError_t launch_select_spec(const float* scores, int64_t n, int rows, const float2* blkstat,
                              int nblk, double eps, RowSel* rs, int32_t* k_eps, double* tau,
                              double* lse, uint32_t* sel_mask, int n_v, const void* V,
                              int v_dtype, int dv, int nchunk, CutPub* pub, float* out,
                              hipStream_t st);

// Blockwise deterministic bound, one workgroup per row: from the scan's tile
// (min, max) and tile masses blkz, the largest threshold whose bound on the
// mass below it fits eps * Z; keeps every key at or above it.  Writes RowSel
// (thr at that score), k_eps (keys kept), tau (the certified bound), lse and
// sel_mask (optional).  nblk <= kBoundMaxTiles.
// 4-bit key copy: K [rows, d] (rows = n_kv * n) -> K4 [rows, d / 2] packed
// codes, kscale [rows] and kres [rows] (an upper bound on the residual norm).
hipError_t launch_quantize_k4(const void* K, int dtype, int d, int64_t rows, uint8_t* K4,
                              float* kscale, float* kres, hipStream_t st);
// Head blocks per KV head of the 4-bit scan (straddle masks are kept per block).
int k4_head_blocks(int group);
// Exact candidates {i : s_hi >= thr[h]} from the 4-bit copy: mask [n_q, ceil(n/32)],
// count [n_q], optional rescored [n_kv] (keys whose full-width row was read) and
// bounds [n_q, n] (lo, hi).  straddle: n_kv * k4_head_blocks(G) * ceil(n/64) uint64.
hipError_t launch_candidates_k4(const void* q, const void* K, int dtype, int d, const uint8_t* K4,
                                const float* kscale, const float* kres, const float* head_scale,
                                float default_scale, const float* thr, int64_t n, int n_q,
                                int n_kv, uint32_t* mask, int32_t* count, int32_t* rescored,
                                float2* bounds, void* straddle, hipStream_t st);

hipError_t launch_bound(const float* scores, int64_t n, int rows, const float2* blkstat,
                        const float* blkz, int nblk, double eps, RowSel* rs, int32_t* k_eps,
                        double* tau, double* lse, uint32_t* sel_mask, hipStream_t st);

// Fused decode for short rows (n <= kShortRowMaxN): one workgroup per query
// row computes its scores (bitwise the score scan's), selects the certified
// head and writes out, k_eps, tau, and lse, sel_mask and scores when given.
constexpr int kShortRowMaxN = 1024;
hipError_t launch_short_row(const void* q, const void* K, const void* V, int dtype, int d,
                            const float* head_scale, float default_scale, int64_t n, int n_q,
                            int n_kv, double eps, float* out, int32_t* k_eps, double* tau,
                            double* lse, uint32_t* sel_mask, float* scores, hipStream_t st);

// Encoder-shaped path (all queries of a head, n <= 512, bf16, MFMA QK^T).
hipError_t launch_encoder(const void* q, const void* K, const void* V, int d,
                          const float* head_scale, float default_scale, int64_t n, int n_q,
                          int n_kv, double eps, float* out, int32_t* k_eps, double* tau,
                          uint32_t* sel_mask, float* scores, double* lse, hipStream_t st);
bool encoder_supported(int dtype, int d, int64_t n, int n_q, int n_kv);

}  // namespace ctopk
