// libctopk C ABI: argument validation, workspace layout and launch sequencing.
//
// Decode path (ctopk_certify / ctopk_certify_ex):
//   score_scan (scores, per-tile min/max) -> [hist0 (level-0 partial
//   histograms), rows longer than the select holds in registers] -> resolve
//   (lse, k_eps, tau, cut key, mask) -> vsum (w * v over the head, out)
// Logits path (ctopk_certify_logits):
//   resolve (including level 0) -> vsum
// Encoder-shaped path (all queries of a head, small n): one fused kernel.
// 4-bit candidates (ctopk_candidates_k4): 4-bit scan (intervals, settled
//   bits, straddle masks) -> rescoring of straddling keys, with the counts.
// Every launch goes to the caller's stream; nothing is copied to the host.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/ctopk.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

// Kernel events armed by ctopk_record_kernel_events for the next call, and
// the pairs the current call is consuming.
constexpr int kMaxKernelEvents = 16;
thread_local hipEvent_t g_armed_ev[kMaxKernelEvents];
thread_local int g_armed_n = 0;
thread_local hipEvent_t g_call_ev[kMaxKernelEvents];
thread_local int g_call_n = 0;
thread_local int g_call_pos = 0;

// Moves the armed events to the call in progress (so they apply to this call
// only, even when it fails validation) and drops what it left unused.
struct CallEvents {
  CallEvents() {
    for (int i = 0; i < g_armed_n; ++i) g_call_ev[i] = g_armed_ev[i];
    g_call_n = g_armed_n;
    g_call_pos = 0;
    g_armed_n = 0;
  }
  ~CallEvents() { g_call_n = g_call_pos = 0; }
};

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return CTOPK_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr size_t kAlign = 256;
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

constexpr int64_t kMaxN = 2147483647LL;
constexpr int64_t kMaxElems = 1LL << 36;  // rows * n

// Scratch layout shared by both paths.  Every region is fully written before
// it is read within a call, except `sync` (the overlapped plan's published
// head masses and cuts), which the score scan of the same call zeroes; so
// nothing needs clearing between calls.
struct Layout {
  size_t rowsel = 0, blkstat = 0, blkz = 0, part = 0, pmass = 0, sync = 0;
  size_t scores = 0, total = 0;
  size_t sync_bytes = 0;
  int nblk = 0, nchunk = 0, hchunk = 0;
  int dchunk = 0;  // value-stream chunks of the overlapped decode plan (0: not taken)
};

Layout layout(int64_t n, int dv, int rows, int n_v, int v_dtype, bool decode) {
  Layout L;
  L.nblk = decode ? static_cast<int>(ctopk::ceil_div(n, ctopk::kScanTile)) : 0;
  L.nchunk = ctopk::vsum_nchunk(n, rows, n_v, v_dtype, dv);
  L.hchunk = (decode && n > ctopk::resolve_register_row()) ? ctopk::hist_nchunk(n, rows) : 0;
  L.dchunk = decode ? ctopk::select_spec_nchunk(n, rows, n_v, v_dtype, dv) : 0;
  // partial slots per row: head + tail per value-stream chunk, or one per
  // chunk of the overlapped plan's stream; and one float per chunk for the
  // sum of w ||v||^2
  const size_t pchunks = static_cast<size_t>(L.nchunk > L.dchunk ? L.nchunk : L.dchunk);
  const size_t pslots = 2 * pchunks;
  size_t off = 0;
  L.rowsel = off;
  off += up(static_cast<size_t>(rows) * sizeof(ctopk::RowSel));
  L.blkstat = off;
  off += up(static_cast<size_t>(rows) * L.nblk * sizeof(float2));
  L.blkz = off;  // per-tile softmax masses (blockwise-bound calls)
  off += up(static_cast<size_t>(rows) * L.nblk * sizeof(float));
  L.part = off;
  off += up(static_cast<size_t>(rows) * (pslots * (dv + 1) + pchunks) * sizeof(float));
  L.pmass = off;
  off += up(static_cast<size_t>(rows) * L.hchunk * ctopk::kBins * sizeof(double));
  L.sync = off;  // CutPub [rows]
  L.sync_bytes = L.dchunk > 0 ? up(static_cast<size_t>(rows) * sizeof(ctopk::CutPub)) : 0;
  off += L.sync_bytes;
  L.scores = off;
  off += up(decode ? static_cast<size_t>(rows) * static_cast<size_t>(n) * sizeof(float) : 0);
  L.total = off;
  return L;
}

// Per-device cached workspace for calls that pass none.
struct Cache {
  std::mutex mu;
  std::vector<void*> ptr;
  std::vector<size_t> bytes;
};
Cache g_cache;

int cached_workspace(size_t need, hipStream_t st, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(CTOPK_ERR_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_cache.mu);
  if (static_cast<int>(g_cache.ptr.size()) <= dev) {
    g_cache.ptr.resize(dev + 1, nullptr);
    g_cache.bytes.resize(dev + 1, 0);
  }
  if (g_cache.bytes[dev] < need) {
    if (g_cache.ptr[dev] != nullptr) {
      // Earlier work on any stream may still use the old buffer.
      if (hipDeviceSynchronize() != hipSuccess)
        return fail(CTOPK_ERR_HIP, "hipDeviceSynchronize failed before growing the workspace");
      (void)hipFree(g_cache.ptr[dev]);
      g_cache.ptr[dev] = nullptr;
      g_cache.bytes[dev] = 0;
    }
    size_t sz = need + need / 4;
    void* p = nullptr;
    if (hipMalloc(&p, sz) != hipSuccess) {
      return fail(CTOPK_ERR_HIP, "hipMalloc of %zu workspace bytes failed", sz);
    }
    g_cache.ptr[dev] = p;
    g_cache.bytes[dev] = sz;
  }
  (void)st;
  *out = g_cache.ptr[dev];
  return CTOPK_OK;
}

// Scratch of ctopk_certify_noalloc: one fixed device array per GPU (every
// device that loads the library holds its own copy).  In host code `scratch`
// names a host-side stand-in, never the device memory: the device address is
// looked up once per device with hipGetSymbolAddress and only that address is
// handed to kernels.
static __device__ __align__(256) unsigned char scratch[CTOPK_NOALLOC_SCRATCH_BYTES];

struct ScratchAddrs {
  std::mutex mu;
  std::vector<void*> ptr;  // per device; nullptr until looked up
};
ScratchAddrs g_scratch;

int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(CTOPK_ERR_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_scratch.mu);
  if (static_cast<int>(g_scratch.ptr.size()) <= dev) g_scratch.ptr.resize(dev + 1, nullptr);
  if (g_scratch.ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(CTOPK_ERR_HIP, "hipGetSymbolAddress of the scratch array failed: %s",
                  hipGetErrorString(e));
    g_scratch.ptr[dev] = p;
  }
  *out = g_scratch.ptr[dev];
  return CTOPK_OK;
}

int check_eps(double eps) {
  if (!(eps > 0.0 && eps < 1.0) || !isfinite(eps))
    return fail(CTOPK_ERR_EPS, "eps must be a finite number in (0, 1), got %g", eps);
  return CTOPK_OK;
}

int validate_args(const ctopk_args* a) {
  if (a == nullptr) return fail(CTOPK_ERR_NULL, "args is NULL");
  if (!a->q || !a->K || !a->V) return fail(CTOPK_ERR_NULL, "q, K and V must be non-NULL");
  if (!a->out || !a->k_eps || !a->tau)
    return fail(CTOPK_ERR_NULL, "out, k_eps and tau must be non-NULL");
  if (a->dtype != CTOPK_F32 && a->dtype != CTOPK_BF16)
    return fail(CTOPK_ERR_UNSUPPORTED, "dtype %d is not CTOPK_F32 or CTOPK_BF16", a->dtype);
  if (a->n < 1 || a->n > kMaxN) return fail(CTOPK_ERR_SHAPE, "n must be in [1, 2^31-1], got %lld",
                                            static_cast<long long>(a->n));
  if (a->d != 64 && a->d != 128) return fail(CTOPK_ERR_SHAPE, "d must be 64 or 128, got %d", a->d);
  if (a->n_q_heads < 1 || a->n_kv_heads < 1)
    return fail(CTOPK_ERR_SHAPE, "head counts must be >= 1 (n_q_heads=%d, n_kv_heads=%d)",
                a->n_q_heads, a->n_kv_heads);
  if (a->n_q_heads % a->n_kv_heads != 0)
    return fail(CTOPK_ERR_SHAPE, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)",
                a->n_q_heads, a->n_kv_heads);
  if (a->n_kv_heads > 65535)
    return fail(CTOPK_ERR_UNSUPPORTED, "n_kv_heads above 65535 is not supported");
  if ((a->flags & ~CTOPK_FLAG_BOUND) != 0u)
    return fail(CTOPK_ERR_UNSUPPORTED, "unknown flags 0x%x", a->flags & ~CTOPK_FLAG_BOUND);
  if ((a->flags & CTOPK_FLAG_BOUND) && ctopk::ceil_div(a->n, ctopk::kScanTile) > ctopk::kBoundMaxTiles)
    return fail(CTOPK_ERR_UNSUPPORTED, "the blockwise bound supports n <= %d",
                ctopk::kBoundMaxTiles * ctopk::kScanTile);
  if (static_cast<int64_t>(a->n_q_heads) * a->n > kMaxElems)
    return fail(CTOPK_ERR_UNSUPPORTED, "n_q_heads * n above 2^36 is not supported");
  int rc = check_eps(a->eps);
  if (rc != CTOPK_OK) return rc;
  if (!aligned16(a->q) || !aligned16(a->K) || !aligned16(a->V))
    return fail(CTOPK_ERR_ALIGN, "q, K and V must be 16-byte aligned");
  if (!aligned(a->out, 4) || !aligned(a->k_eps, 4) || !aligned(a->tau, 8) ||
      (a->scores && !aligned(a->scores, 4)) || (a->sel_mask && !aligned(a->sel_mask, 4)) ||
      (a->lse && !aligned(a->lse, 8)) || (a->head_scale && !aligned(a->head_scale, 4)) ||
      (a->out_err && !aligned(a->out_err, 8)) || (a->out_dense && !aligned(a->out_dense, 4)) ||
      (a->out_var && !aligned(a->out_var, 8)))
    return fail(CTOPK_ERR_ALIGN, "outputs must be aligned to their element size");
  if (a->workspace != nullptr) {
    if (!aligned(a->workspace, kAlign)) return fail(CTOPK_ERR_ALIGN, "workspace must be 256-byte aligned");
    const size_t need =
        ctopk_workspace_bytes(a->n, a->d, a->n_q_heads, a->n_kv_heads, a->dtype);
    if (a->workspace_bytes < need)
      return fail(CTOPK_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", a->workspace_bytes,
                  need);
  }
  return CTOPK_OK;
}

// The plan of a validated call (ctopk_plan_id).
int plan_of(const ctopk_args* a) {
  if (a->flags & CTOPK_FLAG_BOUND) return CTOPK_PLAN_DECODE_BOUND;
  const bool certificate =
      a->out_err != nullptr || a->out_dense != nullptr || a->out_var != nullptr;
  if (certificate) return CTOPK_PLAN_DECODE;
  if (ctopk::encoder_supported(a->dtype, a->d, a->n, a->n_q_heads, a->n_kv_heads))
    return CTOPK_PLAN_ENCODER;
  if (a->n <= ctopk::kShortRowMaxN) return CTOPK_PLAN_DECODE_FUSED;
  if (ctopk::select_spec_nchunk(a->n, a->n_q_heads, a->n_kv_heads, a->dtype, a->d) > 0)
    return CTOPK_PLAN_DECODE_OVERLAP;
  return CTOPK_PLAN_DECODE;
}

int hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(CTOPK_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return CTOPK_OK;
}

size_t k4_workspace(int64_t n, int n_q, int n_kv) {
  const int nzb = ctopk::k4_head_blocks(n_q / n_kv);
  return up(static_cast<size_t>(n_kv) * nzb * static_cast<size_t>(ctopk::ceil_div(n, ctopk::kScanTile)) *
            sizeof(unsigned long long));
}

int check_k4_shape(const void* K, int32_t dtype, int64_t n, int32_t d, int32_t n_kv) {
  if (dtype != CTOPK_F32 && dtype != CTOPK_BF16)
    return fail(CTOPK_ERR_UNSUPPORTED, "dtype %d is not CTOPK_F32 or CTOPK_BF16", dtype);
  if (n < 1 || n > kMaxN) return fail(CTOPK_ERR_SHAPE, "n must be in [1, 2^31-1], got %lld",
                                      static_cast<long long>(n));
  if (d != 64 && d != 128) return fail(CTOPK_ERR_SHAPE, "d must be 64 or 128, got %d", d);
  if (n_kv < 1) return fail(CTOPK_ERR_SHAPE, "n_kv_heads must be >= 1, got %d", n_kv);
  if (n_kv > 65535) return fail(CTOPK_ERR_UNSUPPORTED, "n_kv_heads above 65535 is not supported");
  if (static_cast<int64_t>(n_kv) * n > kMaxElems)
    return fail(CTOPK_ERR_UNSUPPORTED, "n_kv_heads * n above 2^36 is not supported");
  if (!aligned16(K)) return fail(CTOPK_ERR_ALIGN, "K must be 16-byte aligned");
  return CTOPK_OK;
}

int validate_k4(const ctopk_k4_args* a) {
  if (a == nullptr) return fail(CTOPK_ERR_NULL, "args is NULL");
  if (!a->q || !a->K || !a->K4 || !a->kscale || !a->kres || !a->threshold)
    return fail(CTOPK_ERR_NULL, "q, K, K4, kscale, kres and threshold must be non-NULL");
  if (!a->sel_mask || !a->count) return fail(CTOPK_ERR_NULL, "sel_mask and count must be non-NULL");
  int rc = check_k4_shape(a->K, a->dtype, a->n, a->d, a->n_kv_heads);
  if (rc != CTOPK_OK) return rc;
  if (a->n_q_heads < 1 || a->n_q_heads % a->n_kv_heads != 0)
    return fail(CTOPK_ERR_SHAPE, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)",
                a->n_q_heads, a->n_kv_heads);
  if (static_cast<int64_t>(a->n_q_heads) * a->n > kMaxElems)
    return fail(CTOPK_ERR_UNSUPPORTED, "n_q_heads * n above 2^36 is not supported");
  if (!aligned16(a->q) || !aligned(a->K4, 4) || !aligned(a->kscale, 4) || !aligned(a->kres, 4) ||
      !aligned(a->threshold, 4) || !aligned(a->sel_mask, 4) || !aligned(a->count, 4) ||
      (a->head_scale && !aligned(a->head_scale, 4)) || (a->rescored && !aligned(a->rescored, 4)) ||
      (a->bounds && !aligned(a->bounds, 8)))
    return fail(CTOPK_ERR_ALIGN, "q must be 16-byte aligned, K4 and the other arrays element aligned");
  if (a->workspace != nullptr) {
    if (!aligned(a->workspace, kAlign)) return fail(CTOPK_ERR_ALIGN, "workspace must be 256-byte aligned");
    const size_t need = k4_workspace(a->n, a->n_q_heads, a->n_kv_heads);
    if (a->workspace_bytes < need)
      return fail(CTOPK_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", a->workspace_bytes, need);
  }
  return CTOPK_OK;
}

}  // namespace

namespace ctopk {
bool take_kernel_events(hipEvent_t* start, hipEvent_t* stop) {
  if (g_call_pos + 2 > g_call_n) return false;
  *start = g_call_ev[g_call_pos];
  *stop = g_call_ev[g_call_pos + 1];
  g_call_pos += 2;
  return true;
}
void skip_kernel_events(hipStream_t st) {
  hipEvent_t a, b;
  if (take_kernel_events(&a, &b)) {
    (void)hipEventRecord(a, st);
    (void)hipEventRecord(b, st);
  }
}
}  // namespace ctopk

extern "C" {

size_t ctopk_workspace_bytes(int64_t n, int32_t d, int32_t n_q_heads, int32_t n_kv_heads,
                             int32_t dtype) {
  if (n < 1 || n > kMaxN || (d != 64 && d != 128) || n_q_heads < 1 || n_kv_heads < 1 ||
      n_q_heads % n_kv_heads != 0 || (dtype != CTOPK_F32 && dtype != CTOPK_BF16))
    return 0;
  // Sized for the general path, which every call can take (the encoder-shaped
  // path needs none, but calls asking for the output certificate use the
  // general path on any shape).
  return layout(n, d, n_q_heads, n_kv_heads, dtype, true).total;
}

size_t ctopk_logits_workspace_bytes(int64_t n, int32_t dv, int32_t rows, int32_t n_v) {
  if (n < 1 || n > kMaxN || (dv != 64 && dv != 128) || rows < 1 || n_v < 1 || rows % n_v != 0)
    return 0;
  return layout(n, dv, rows, n_v, CTOPK_F32, false).total;
}

int ctopk_validate(const ctopk_args* a) {
  const int rc = validate_args(a);
  if (rc == CTOPK_OK) return ok();
  return rc;
}

int ctopk_plan(const ctopk_args* a) {
  const int rc = validate_args(a);
  if (rc != CTOPK_OK) return rc;
  ok();
  return plan_of(a);
}

int ctopk_certify_ex(const ctopk_args* a, ctopk_stream_t stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  CallEvents events;  // consumes armed events even if validation fails
  int rc = validate_args(a);
  if (rc != CTOPK_OK) return rc;
  const float default_scale = static_cast<float>(1.0 / sqrt(static_cast<double>(a->d)));
  const int plan = plan_of(a);

  if (plan == CTOPK_PLAN_ENCODER) {
    rc = hip_check(ctopk::launch_encoder(a->q, a->K, a->V, a->d, a->head_scale, default_scale,
                                         a->n, a->n_q_heads, a->n_kv_heads, a->eps, a->out,
                                         a->k_eps, a->tau, a->sel_mask, a->scores, a->lse, st),
                   "encoder launch");
    return rc == CTOPK_OK ? ok() : rc;
  }
  if (plan == CTOPK_PLAN_DECODE_FUSED) {
    rc = hip_check(ctopk::launch_short_row(a->q, a->K, a->V, a->dtype, a->d, a->head_scale,
                                           default_scale, a->n, a->n_q_heads, a->n_kv_heads,
                                           a->eps, a->out, a->k_eps, a->tau, a->lse,
                                           a->sel_mask, a->scores, st),
                   "short-row launch");
    return rc == CTOPK_OK ? ok() : rc;
  }

  const Layout L = layout(a->n, a->d, a->n_q_heads, a->n_kv_heads, a->dtype, true);
  char* ws = static_cast<char*>(a->workspace);
  if (ws == nullptr) {
    void* p = nullptr;
    rc = cached_workspace(L.total, st, &p);
    if (rc != CTOPK_OK) return rc;
    ws = static_cast<char*>(p);
  }
  float* scores = a->scores ? a->scores : reinterpret_cast<float*>(ws + L.scores);
  float2* blkstat = reinterpret_cast<float2*>(ws + L.blkstat);
  float* blkz = plan == CTOPK_PLAN_DECODE_BOUND ? reinterpret_cast<float*>(ws + L.blkz) : nullptr;
  float* part = reinterpret_cast<float*>(ws + L.part);
  double* pmass = reinterpret_cast<double*>(ws + L.pmass);
  ctopk::RowSel* rs = reinterpret_cast<ctopk::RowSel*>(ws + L.rowsel);
  const int rows = a->n_q_heads;

  const bool overlap = plan == CTOPK_PLAN_DECODE_OVERLAP;
  rc = hip_check(ctopk::launch_score_scan(a->q, a->K, a->dtype, a->d, a->head_scale,
                                          default_scale, a->n, rows, a->n_kv_heads, scores,
                                          blkstat, blkz, overlap ? ws + L.sync : nullptr,
                                          overlap ? L.sync_bytes : 0, overlap ? a->out : nullptr,
                                          overlap ? static_cast<size_t>(rows) * a->d * sizeof(float) : 0,
                                          st),
                 "score_scan launch");
  if (rc != CTOPK_OK) return rc;
  if (L.hchunk > 0 && plan != CTOPK_PLAN_DECODE_BOUND) {  // long rows: level 0 from many blocks per row
    rc = hip_check(ctopk::launch_hist0(scores, a->n, rows, blkstat, L.nblk, L.hchunk, pmass,
                                       st),
                   "hist0 launch");
    if (rc != CTOPK_OK) return rc;
  } else {
    ctopk::skip_kernel_events(st);
  }
  if (overlap) {
    // The select beside the value stream over provisional heads, corrected
    // and added into out inside the same launch (out zeroed by the scan).
    rc = hip_check(ctopk::launch_select_spec(scores, a->n, rows, blkstat, L.nblk, a->eps, rs,
                                             a->k_eps, a->tau, a->lse, a->sel_mask,
                                             a->n_kv_heads, a->V, a->dtype, a->d, L.dchunk,
                                             reinterpret_cast<ctopk::CutPub*>(ws + L.sync),
                                             a->out, st),
                   "select launch");
    if (rc != CTOPK_OK) return rc;
    return ok();
  }
  if (plan == CTOPK_PLAN_DECODE_BOUND) {
    rc = hip_check(ctopk::launch_bound(scores, a->n, rows, blkstat, blkz, L.nblk, a->eps, rs,
                                       a->k_eps, a->tau, a->lse, a->sel_mask, st),
                   "bound launch");
  } else {
    rc = hip_check(ctopk::launch_resolve(scores, a->n, rows, blkstat, L.nblk, pmass,
                                         L.hchunk, a->eps, rs, a->k_eps, a->tau, a->lse,
                                         a->sel_mask, nullptr, 0, st),
                   "resolve launch");
  }
  if (rc != CTOPK_OK) return rc;
  rc = hip_check(ctopk::launch_vsum(scores, a->n, rows, a->n_kv_heads, a->V, a->dtype, a->d, rs,
                                    part, L.nchunk, a->out, a->out_dense, a->out_err,
                                    a->out_var, st),
                 "vsum launch");
  if (rc != CTOPK_OK) return rc;
  return ok();
}

int ctopk_certify(const void* q, const void* K, const void* V, int64_t n, int32_t d,
                  int32_t n_q_heads, int32_t n_kv_heads, double eps, ctopk_stream_t stream,
                  float* out, int32_t* k_eps, double* tau) {
  ctopk_args a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.K = K;
  a.V = V;
  a.dtype = CTOPK_BF16;
  a.n = n;
  a.d = d;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.eps = eps;
  a.out = out;
  a.k_eps = k_eps;
  a.tau = tau;
  return ctopk_certify_ex(&a, stream);
}

int ctopk_certify_noalloc(const void* q, const void* K, const void* V, int64_t n, int32_t d,
                          int32_t n_q_heads, int32_t n_kv_heads, double eps,
                          ctopk_stream_t stream, float* out, int32_t* k_eps, double* tau) {
  ctopk_args a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.K = K;
  a.V = V;
  a.dtype = CTOPK_BF16;
  a.n = n;
  a.d = d;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.eps = eps;
  a.out = out;
  a.k_eps = k_eps;
  a.tau = tau;
  {
    CallEvents events;  // an armed event list applies to this call even if it fails here
    int rc = validate_args(&a);
    if (rc != CTOPK_OK) return rc;
    const size_t need = ctopk_workspace_bytes(n, d, n_q_heads, n_kv_heads, CTOPK_BF16);
    if (need > static_cast<size_t>(CTOPK_NOALLOC_SCRATCH_BYTES))
      return fail(CTOPK_ERR_WORKSPACE,
                  "these sizes need %zu bytes of scratch, more than the fixed %zu-byte array of "
                  "ctopk_certify_noalloc",
                  need, static_cast<size_t>(CTOPK_NOALLOC_SCRATCH_BYTES));
    void* p = nullptr;
    rc = scratch_address(&p);
    if (rc != CTOPK_OK) return rc;
    a.workspace = p;
    a.workspace_bytes = CTOPK_NOALLOC_SCRATCH_BYTES;
    // hand the armed events on to the call below
    for (int i = 0; i < g_call_n; ++i) g_armed_ev[i] = g_call_ev[i];
    g_armed_n = g_call_n;
  }
  return ctopk_certify_ex(&a, stream);
}

int ctopk_certify_logits(const float* logits, const void* V, int32_t v_dtype, int64_t n,
                         int32_t dv, int32_t rows, int32_t n_v, double eps, void* workspace,
                         size_t workspace_bytes, ctopk_stream_t stream, float* out,
                         int32_t* k_eps, double* tau, uint32_t* sel_mask, double* lse) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  CallEvents events;  // consumes armed events even if validation fails
  if (!logits || !V || !out || !k_eps || !tau)
    return fail(CTOPK_ERR_NULL, "logits, V, out, k_eps and tau must be non-NULL");
  if (v_dtype != CTOPK_F32 && v_dtype != CTOPK_BF16)
    return fail(CTOPK_ERR_UNSUPPORTED, "v_dtype %d is not CTOPK_F32 or CTOPK_BF16", v_dtype);
  if (n < 1 || n > kMaxN)
    return fail(CTOPK_ERR_SHAPE, "n must be in [1, 2^31-1], got %lld", static_cast<long long>(n));
  if (dv != 64 && dv != 128) return fail(CTOPK_ERR_SHAPE, "dv must be 64 or 128, got %d", dv);
  if (rows < 1 || n_v < 1 || rows % n_v != 0)
    return fail(CTOPK_ERR_SHAPE, "rows (%d) must be a positive multiple of n_v (%d)", rows, n_v);
  if (n_v > 65535) return fail(CTOPK_ERR_UNSUPPORTED, "n_v above 65535 is not supported");
  if (static_cast<int64_t>(rows) * n > kMaxElems)
    return fail(CTOPK_ERR_UNSUPPORTED, "rows * n above 2^36 is not supported");
  int rc = check_eps(eps);
  if (rc != CTOPK_OK) return rc;
  if (!aligned(logits, 4) || !aligned16(V) || !aligned(out, 4) || !aligned(k_eps, 4) ||
      !aligned(tau, 8) || (sel_mask && !aligned(sel_mask, 4)) || (lse && !aligned(lse, 8)))
    return fail(CTOPK_ERR_ALIGN, "V must be 16-byte aligned and outputs element aligned");
  const Layout L = layout(n, dv, rows, n_v, v_dtype, false);
  char* ws = static_cast<char*>(workspace);
  if (ws != nullptr) {
    if (!aligned(ws, kAlign)) return fail(CTOPK_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (workspace_bytes < L.total)
      return fail(CTOPK_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                  L.total);
  } else {
    void* p = nullptr;
    rc = cached_workspace(L.total, st, &p);
    if (rc != CTOPK_OK) return rc;
    ws = static_cast<char*>(p);
  }
  float* part = reinterpret_cast<float*>(ws + L.part);
  ctopk::RowSel* rs = reinterpret_cast<ctopk::RowSel*>(ws + L.rowsel);

  rc = hip_check(ctopk::launch_resolve(logits, n, rows, nullptr, 0, nullptr, 0, eps, rs,
                                       k_eps, tau, lse, sel_mask, nullptr, 0, st),
                 "resolve launch");
  if (rc != CTOPK_OK) return rc;
  rc = hip_check(ctopk::launch_vsum(logits, n, rows, n_v, V, v_dtype, dv, rs, part, L.nchunk,
                                    out, nullptr, nullptr, nullptr, st),
                 "vsum launch");
  if (rc != CTOPK_OK) return rc;
  return ok();
}

int ctopk_quantize_k4(const void* K, int32_t dtype, int64_t n, int32_t d, int32_t n_kv_heads,
                      uint8_t* K4, float* kscale, float* kres, ctopk_stream_t stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  CallEvents events;
  if (!K || !K4 || !kscale || !kres) return fail(CTOPK_ERR_NULL, "K, K4, kscale and kres must be non-NULL");
  int rc = check_k4_shape(K, dtype, n, d, n_kv_heads);
  if (rc != CTOPK_OK) return rc;
  if (!aligned(K4, 4) || !aligned(kscale, 4) || !aligned(kres, 4))
    return fail(CTOPK_ERR_ALIGN, "K4, kscale and kres must be 4-byte aligned");
  if (static_cast<int64_t>(n_kv_heads) * n > (int64_t{1} << 34))  // the copy's grid is rows / 16 blocks
    return fail(CTOPK_ERR_UNSUPPORTED, "n_kv_heads * n above 2^34 is not supported by the copy");
  rc = hip_check(ctopk::launch_quantize_k4(K, dtype, d, static_cast<int64_t>(n_kv_heads) * n, K4,
                                           kscale, kres, st),
                 "quantize launch");
  return rc == CTOPK_OK ? ok() : rc;
}

int ctopk_validate_k4(const ctopk_k4_args* a) {
  const int rc = validate_k4(a);
  return rc == CTOPK_OK ? ok() : rc;
}

size_t ctopk_k4_workspace_bytes(int64_t n, int32_t n_q_heads, int32_t n_kv_heads) {
  if (n < 1 || n > kMaxN || n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads != 0) return 0;
  return k4_workspace(n, n_q_heads, n_kv_heads);
}

int ctopk_candidates_k4(const ctopk_k4_args* a, ctopk_stream_t stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  CallEvents events;
  int rc = validate_k4(a);
  if (rc != CTOPK_OK) return rc;
  void* ws = a->workspace;
  if (ws == nullptr) {
    rc = cached_workspace(k4_workspace(a->n, a->n_q_heads, a->n_kv_heads), st, &ws);
    if (rc != CTOPK_OK) return rc;
  }
  const float default_scale = static_cast<float>(1.0 / sqrt(static_cast<double>(a->d)));
  rc = hip_check(ctopk::launch_candidates_k4(a->q, a->K, a->dtype, a->d, a->K4, a->kscale, a->kres,
                                             a->head_scale, default_scale, a->threshold, a->n,
                                             a->n_q_heads, a->n_kv_heads, a->sel_mask, a->count,
                                             a->rescored, reinterpret_cast<float2*>(a->bounds), ws,
                                             st),
                 "candidates launch");
  return rc == CTOPK_OK ? ok() : rc;
}

int ctopk_record_kernel_events(void* const* events, int32_t count) {
  if (count < 0 || count > kMaxKernelEvents || (count & 1))
    return fail(CTOPK_ERR_SHAPE, "count must be even and in 0..%d, got %d", kMaxKernelEvents,
                count);
  if (count > 0 && events == nullptr) return fail(CTOPK_ERR_NULL, "events is NULL");
  for (int i = 0; i < count; ++i) {
    if (events[i] == nullptr) return fail(CTOPK_ERR_NULL, "events[%d] is NULL", i);
    g_armed_ev[i] = static_cast<hipEvent_t>(events[i]);
  }
  g_armed_n = count;
  return ok();
}

const char* ctopk_last_error_string(void) { return g_err; }

const char* ctopk_version(void) { return "libctopk 0.1 gfx950"; }

}  // extern "C"
