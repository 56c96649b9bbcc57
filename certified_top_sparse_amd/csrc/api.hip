// libctopk C ABI: argument validation, workspace layout and launch sequencing.
//
// Decode path (ctopk_certify / ctopk_certify_ex):
//   K1 score_scan -> hist0 (row max, level-0 histogram) -> resolve (k_eps, tau)
//   -> vsum (w * v over the head, selection mask) -> finalize (out)
// Logits path (ctopk_certify_logits):
//   rowmax -> hist0 -> resolve -> vsum -> finalize
// Encoder-shaped path (all queries of a head, small n): one fused kernel.
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

// Scratch layout shared by both paths.
struct Layout {
  size_t scores = 0, blkmax = 0, hcnt = 0, hmass = 0, rowsel = 0, part = 0, total = 0;
  size_t scores_b = 0, blkmax_b = 0, hist_b = 0;
  int nblk = 0, nchunk = 0;
};

Layout layout(int64_t n, int dv, int rows, int n_v, bool decode) {
  Layout L;
  L.nblk = decode ? static_cast<int>(ctopk::ceil_div(n, ctopk::kScanTile)) : ctopk::rowmax_nblk(n);
  L.nchunk = ctopk::vsum_nchunk(n, rows, n_v);
  size_t off = 0;
  // hcnt and hmass are contiguous so that one zeroing range clears both.
  L.hcnt = off;
  off += up(static_cast<size_t>(rows) * ctopk::kBins * sizeof(uint32_t));
  L.hmass = off;
  off += up(static_cast<size_t>(rows) * ctopk::kBins * sizeof(double));
  L.hist_b = off;
  L.rowsel = off;
  off += up(static_cast<size_t>(rows) * sizeof(ctopk::RowSel));
  L.blkmax = off;
  L.blkmax_b = static_cast<size_t>(rows) * L.nblk * sizeof(float);
  off += up(L.blkmax_b);
  L.part = off;
  off += up(static_cast<size_t>(rows) * L.nchunk * (dv + 1) * sizeof(float));
  L.scores = off;
  L.scores_b = decode ? static_cast<size_t>(rows) * static_cast<size_t>(n) * sizeof(float) : 0;
  off += up(L.scores_b);
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
  if (static_cast<int64_t>(a->n_q_heads) * a->n > kMaxElems)
    return fail(CTOPK_ERR_UNSUPPORTED, "n_q_heads * n above 2^36 is not supported");
  int rc = check_eps(a->eps);
  if (rc != CTOPK_OK) return rc;
  if (!aligned16(a->q) || !aligned16(a->K) || !aligned16(a->V))
    return fail(CTOPK_ERR_ALIGN, "q, K and V must be 16-byte aligned");
  if (!aligned(a->out, 4) || !aligned(a->k_eps, 4) || !aligned(a->tau, 8) ||
      (a->scores && !aligned(a->scores, 4)) || (a->sel_mask && !aligned(a->sel_mask, 4)) ||
      (a->lse && !aligned(a->lse, 8)) || (a->head_scale && !aligned(a->head_scale, 4)))
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

int hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(CTOPK_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return CTOPK_OK;
}

}  // namespace

extern "C" {

size_t ctopk_workspace_bytes(int64_t n, int32_t d, int32_t n_q_heads, int32_t n_kv_heads,
                             int32_t dtype) {
  if (n < 1 || n > kMaxN || (d != 64 && d != 128) || n_q_heads < 1 || n_kv_heads < 1 ||
      n_q_heads % n_kv_heads != 0 || (dtype != CTOPK_F32 && dtype != CTOPK_BF16))
    return 0;
  if (ctopk::encoder_supported(dtype, d, n, n_q_heads, n_kv_heads)) return kAlign;
  return layout(n, d, n_q_heads, n_kv_heads, true).total;
}

size_t ctopk_logits_workspace_bytes(int64_t n, int32_t dv, int32_t rows, int32_t n_v) {
  if (n < 1 || n > kMaxN || (dv != 64 && dv != 128) || rows < 1 || n_v < 1 || rows % n_v != 0)
    return 0;
  return layout(n, dv, rows, n_v, false).total;
}

int ctopk_validate(const ctopk_args* a) {
  const int rc = validate_args(a);
  if (rc == CTOPK_OK) return ok();
  return rc;
}

int ctopk_certify_ex(const ctopk_args* a, ctopk_stream_t stream) {
  int rc = validate_args(a);
  if (rc != CTOPK_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const float default_scale = static_cast<float>(1.0 / sqrt(static_cast<double>(a->d)));

  if (ctopk::encoder_supported(a->dtype, a->d, a->n, a->n_q_heads, a->n_kv_heads)) {
    rc = hip_check(ctopk::launch_encoder(a->q, a->K, a->V, a->d, a->head_scale, default_scale,
                                         a->n, a->n_q_heads, a->n_kv_heads, a->eps, a->out,
                                         a->k_eps, a->tau, a->sel_mask, a->scores, a->lse, st),
                   "encoder launch");
    return rc == CTOPK_OK ? ok() : rc;
  }

  const Layout L = layout(a->n, a->d, a->n_q_heads, a->n_kv_heads, true);
  char* ws = static_cast<char*>(a->workspace);
  if (ws == nullptr) {
    void* p = nullptr;
    rc = cached_workspace(L.total, st, &p);
    if (rc != CTOPK_OK) return rc;
    ws = static_cast<char*>(p);
  }
  float* scores = a->scores ? a->scores : reinterpret_cast<float*>(ws + L.scores);
  float* blkmax = reinterpret_cast<float*>(ws + L.blkmax);
  uint32_t* hcnt = reinterpret_cast<uint32_t*>(ws + L.hcnt);
  double* hmass = reinterpret_cast<double*>(ws + L.hmass);
  ctopk::RowSel* rs = reinterpret_cast<ctopk::RowSel*>(ws + L.rowsel);
  float* part = reinterpret_cast<float*>(ws + L.part);
  const int rows = a->n_q_heads;

  rc = hip_check(ctopk::launch_score_scan(a->q, a->K, a->dtype, a->d, a->head_scale,
                                          default_scale, a->n, rows, a->n_kv_heads, scores,
                                          blkmax, ws + L.hcnt, L.hist_b - L.hcnt, st),
                 "score_scan launch");
  if (rc != CTOPK_OK) return rc;
  rc = hip_check(ctopk::launch_hist0(scores, a->n, rows, blkmax, L.nblk, rs, hcnt, hmass, st),
                 "hist0 launch");
  if (rc != CTOPK_OK) return rc;
  rc = hip_check(ctopk::launch_resolve(scores, a->n, rows, hcnt, hmass, a->eps, rs, a->k_eps,
                                       a->tau, a->lse, st),
                 "resolve launch");
  if (rc != CTOPK_OK) return rc;
  rc = hip_check(ctopk::launch_vsum(scores, a->n, rows, a->n_kv_heads, a->V, a->dtype, a->d, rs,
                                    part, L.nchunk, a->sel_mask, st),
                 "vsum launch");
  if (rc != CTOPK_OK) return rc;
  rc = hip_check(ctopk::launch_finalize(part, rows, L.nchunk, a->d, a->out, st),
                 "finalize launch");
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

int ctopk_certify_logits(const float* logits, const void* V, int32_t v_dtype, int64_t n,
                         int32_t dv, int32_t rows, int32_t n_v, double eps, void* workspace,
                         size_t workspace_bytes, ctopk_stream_t stream, float* out,
                         int32_t* k_eps, double* tau, uint32_t* sel_mask, double* lse) {
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
  const Layout L = layout(n, dv, rows, n_v, false);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
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
  float* blkmax = reinterpret_cast<float*>(ws + L.blkmax);
  uint32_t* hcnt = reinterpret_cast<uint32_t*>(ws + L.hcnt);
  double* hmass = reinterpret_cast<double*>(ws + L.hmass);
  ctopk::RowSel* rs = reinterpret_cast<ctopk::RowSel*>(ws + L.rowsel);
  float* part = reinterpret_cast<float*>(ws + L.part);

  rc = hip_check(ctopk::launch_rowmax(logits, n, rows, blkmax, ws + L.hcnt, L.hist_b - L.hcnt, st),
                 "rowmax launch");
  if (rc != CTOPK_OK) return rc;
  rc = hip_check(ctopk::launch_hist0(logits, n, rows, blkmax, L.nblk, rs, hcnt, hmass, st),
                 "hist0 launch");
  if (rc != CTOPK_OK) return rc;
  rc = hip_check(ctopk::launch_resolve(logits, n, rows, hcnt, hmass, eps, rs, k_eps, tau, lse, st),
                 "resolve launch");
  if (rc != CTOPK_OK) return rc;
  rc = hip_check(ctopk::launch_vsum(logits, n, rows, n_v, V, v_dtype, dv, rs, part, L.nchunk,
                                    sel_mask, st),
                 "vsum launch");
  if (rc != CTOPK_OK) return rc;
  rc = hip_check(ctopk::launch_finalize(part, rows, L.nchunk, dv, out, st), "finalize launch");
  if (rc != CTOPK_OK) return rc;
  return ok();
}

const char* ctopk_last_error_string(void) { return g_err; }

const char* ctopk_version(void) { return "libctopk 0.1 gfx950"; }

}  // extern "C"
