"""ctypes binding of libctopk (include/ctopk.h).

Argument marshalling only: every step of certified Top-k truncation runs in
the library's HIP kernels.  torch supplies device memory (output tensors) and
the current HIP stream.  The functions carry the C names.

If libctopk.so is missing the import still succeeds, but every call raises
RuntimeError: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libctopk.so")

CTOPK_OK = 0
CTOPK_ERR_NULL = -1
CTOPK_ERR_SHAPE = -2
CTOPK_ERR_EPS = -3
CTOPK_ERR_ALIGN = -4
CTOPK_ERR_UNSUPPORTED = -5
CTOPK_ERR_WORKSPACE = -6
CTOPK_ERR_HIP = -7
CTOPK_F32 = 0
CTOPK_BF16 = 1
CTOPK_PLAN_ENCODER = 1
CTOPK_PLAN_DECODE = 2
CTOPK_PLAN_DECODE_OVERLAP = 3
CTOPK_PLAN_DECODE_BOUND = 4
CTOPK_PLAN_DECODE_FUSED = 5
CTOPK_FLAG_BOUND = 1

STATUS_NAMES = {
    0: "CTOPK_OK", -1: "CTOPK_ERR_NULL", -2: "CTOPK_ERR_SHAPE", -3: "CTOPK_ERR_EPS",
    -4: "CTOPK_ERR_ALIGN", -5: "CTOPK_ERR_UNSUPPORTED", -6: "CTOPK_ERR_WORKSPACE",
    -7: "CTOPK_ERR_HIP",
}

# Every symbol include/ctopk.h declares.
EXPORTED = (
    "ctopk_certify", "ctopk_certify_ex", "ctopk_workspace_bytes", "ctopk_certify_logits",
    "ctopk_logits_workspace_bytes", "ctopk_validate", "ctopk_last_error_string",
    "ctopk_version", "ctopk_record_kernel_events", "ctopk_plan", "ctopk_quantize_k4",
    "ctopk_candidates_k4", "ctopk_validate_k4", "ctopk_k4_workspace_bytes",
    "ctopk_certify_noalloc",
)


class CtopkArgs(ctypes.Structure):
    """Mirror of struct ctopk_args."""
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("K", ctypes.c_void_p),
        ("V", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("n", ctypes.c_int64),
        ("d", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("eps", ctypes.c_double),
        ("head_scale", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("out", ctypes.c_void_p),
        ("k_eps", ctypes.c_void_p),
        ("tau", ctypes.c_void_p),
        ("sel_mask", ctypes.c_void_p),
        ("scores", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("out_err", ctypes.c_void_p),
        ("out_dense", ctypes.c_void_p),
        ("flags", ctypes.c_uint32),
        ("out_var", ctypes.c_void_p),
    ]


class CtopkK4Args(ctypes.Structure):
    """Mirror of ctopk_k4_args."""
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("K", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("n", ctypes.c_int64),
        ("d", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_scale", ctypes.c_void_p),
        ("K4", ctypes.c_void_p),
        ("kscale", ctypes.c_void_p),
        ("kres", ctypes.c_void_p),
        ("threshold", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("sel_mask", ctypes.c_void_p),
        ("count", ctypes.c_void_p),
        ("rescored", ctypes.c_void_p),
        ("bounds", ctypes.c_void_p),
    ]


class CtopkError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


_lib = None


def load(path: str = LIB_PATH):
    """Load libctopk.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"libctopk.so not found at {path}; build it with "
            "`python -m certified_top_sparse_amd.build` (no CPU fallback exists)")
    # Import torch first: its bundled HIP runtime (soname libamdhip64.so.7) is
    # then the one libctopk binds to, so streams and memory are shared.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    vp, i32, i64, f64, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                             ctypes.c_double, ctypes.c_size_t)
    lib.ctopk_certify.argtypes = [vp, vp, vp, i64, i32, i32, i32, f64, vp, vp, vp, vp]
    lib.ctopk_certify.restype = ctypes.c_int
    lib.ctopk_certify_noalloc.argtypes = [vp, vp, vp, i64, i32, i32, i32, f64, vp, vp, vp, vp]
    lib.ctopk_certify_noalloc.restype = ctypes.c_int
    lib.ctopk_certify_ex.argtypes = [ctypes.POINTER(CtopkArgs), vp]
    lib.ctopk_certify_ex.restype = ctypes.c_int
    lib.ctopk_workspace_bytes.argtypes = [i64, i32, i32, i32, i32]
    lib.ctopk_workspace_bytes.restype = sz
    lib.ctopk_certify_logits.argtypes = [vp, vp, i32, i64, i32, i32, i32, f64, vp, sz, vp,
                                         vp, vp, vp, vp, vp]
    lib.ctopk_certify_logits.restype = ctypes.c_int
    lib.ctopk_logits_workspace_bytes.argtypes = [i64, i32, i32, i32]
    lib.ctopk_logits_workspace_bytes.restype = sz
    lib.ctopk_validate.argtypes = [ctypes.POINTER(CtopkArgs)]
    lib.ctopk_validate.restype = ctypes.c_int
    lib.ctopk_plan.argtypes = [ctypes.POINTER(CtopkArgs)]
    lib.ctopk_plan.restype = ctypes.c_int
    lib.ctopk_last_error_string.argtypes = []
    lib.ctopk_last_error_string.restype = ctypes.c_char_p
    lib.ctopk_version.argtypes = []
    lib.ctopk_version.restype = ctypes.c_char_p
    lib.ctopk_record_kernel_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), i32]
    lib.ctopk_record_kernel_events.restype = ctypes.c_int
    lib.ctopk_quantize_k4.argtypes = [vp, i32, i64, i32, i32, vp, vp, vp, vp]
    lib.ctopk_quantize_k4.restype = ctypes.c_int
    lib.ctopk_candidates_k4.argtypes = [ctypes.POINTER(CtopkK4Args), vp]
    lib.ctopk_candidates_k4.restype = ctypes.c_int
    lib.ctopk_validate_k4.argtypes = [ctypes.POINTER(CtopkK4Args)]
    lib.ctopk_validate_k4.restype = ctypes.c_int
    lib.ctopk_k4_workspace_bytes.argtypes = [i64, i32, i32]
    lib.ctopk_k4_workspace_bytes.restype = sz
    _lib = lib
    return lib


def _check(code):
    if code != CTOPK_OK:
        raise CtopkError(code, ctopk_last_error_string())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return CTOPK_BF16
    if t.dtype == torch.float32:
        return CTOPK_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _require_cuda_contig(name, t):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ---------------------------------------------------------------------------
# the C entry points
# ---------------------------------------------------------------------------
def ctopk_version() -> str:
    return load().ctopk_version().decode()


def ctopk_last_error_string() -> str:
    return load().ctopk_last_error_string().decode()


def ctopk_workspace_bytes(n, d, n_q_heads, n_kv_heads, dtype=CTOPK_BF16) -> int:
    return int(load().ctopk_workspace_bytes(n, d, n_q_heads, n_kv_heads, dtype))


def ctopk_logits_workspace_bytes(n, dv, rows, n_v) -> int:
    return int(load().ctopk_logits_workspace_bytes(n, dv, rows, n_v))


def ctopk_record_kernel_events(events) -> None:
    """Arm the calling thread's next certify call to attach the raw hipEvent_t
    handles (ints), taken in (start, stop) pairs, to its kernels in launch order."""
    arr = (ctypes.c_void_p * max(1, len(events)))(*[ctypes.c_void_p(e) for e in events])
    _check(load().ctopk_record_kernel_events(arr, len(events)))


def ctopk_validate(args: CtopkArgs) -> int:
    """Host-only argument check; returns the status code (no exception)."""
    return int(load().ctopk_validate(ctypes.byref(args)))


def ctopk_plan(args: CtopkArgs) -> int:
    """Host-only: the plan (CTOPK_PLAN_*) ctopk_certify_ex takes for these
    arguments, or the negative status of their validation."""
    return int(load().ctopk_plan(ctypes.byref(args)))


def ctopk_certify(q, K, V, eps, out=None, k_eps=None, tau=None, stream=None):
    """The decode call: bf16 q [Hq, d], K/V [Hkv, n, d]; scale 1/sqrt(d).

    Returns (out [Hq, d] fp32, k_eps [Hq] int32, tau [Hq] fp64)."""
    import torch
    lib = load()
    for name, t in (("q", q), ("K", K), ("V", V)):
        _require_cuda_contig(name, t)
    n_q, d = q.shape
    n_kv, n, _ = K.shape
    dev = q.device
    out = torch.empty((n_q, d), dtype=torch.float32, device=dev) if out is None else out
    k_eps = torch.empty(n_q, dtype=torch.int32, device=dev) if k_eps is None else k_eps
    tau = torch.empty(n_q, dtype=torch.float64, device=dev) if tau is None else tau
    _check(lib.ctopk_certify(_ptr(q), _ptr(K), _ptr(V), n, d, n_q, n_kv, float(eps),
                             _stream(stream), _ptr(out), _ptr(k_eps), _ptr(tau)))
    return out, k_eps, tau


def ctopk_certify_noalloc(q, K, V, eps, out, k_eps, tau, stream=None):
    """ctopk_certify with the library's fixed scratch array instead of an
    allocated workspace (no device allocation by the library); the caller
    passes the outputs.  Returns (out, k_eps, tau)."""
    lib = load()
    for name, t in (("q", q), ("K", K), ("V", V), ("out", out), ("k_eps", k_eps),
                    ("tau", tau)):
        _require_cuda_contig(name, t)
    n_q, d = q.shape
    n_kv, n, _ = K.shape
    _check(lib.ctopk_certify_noalloc(_ptr(q), _ptr(K), _ptr(V), n, d, n_q, n_kv, float(eps),
                                     _stream(stream), _ptr(out), _ptr(k_eps), _ptr(tau)))
    return out, k_eps, tau


CTOPK_NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024


def make_args(q, K, V, eps, *, head_scale=None, workspace=None, out=None, k_eps=None,
              tau=None, sel_mask=None, scores=None, lse=None, out_err=None,
              out_dense=None, out_var=None, flags=0) -> CtopkArgs:
    n_q, d = q.shape
    n_kv, n, _ = K.shape
    a = CtopkArgs()
    a.q, a.K, a.V = q.data_ptr(), K.data_ptr(), V.data_ptr()
    a.dtype = _dtype_code(q)
    a.n, a.d, a.n_q_heads, a.n_kv_heads = n, d, n_q, n_kv
    a.eps = float(eps)
    a.head_scale = None if head_scale is None else head_scale.data_ptr()
    a.workspace = None if workspace is None else workspace.data_ptr()
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    for f, t in (("out", out), ("k_eps", k_eps), ("tau", tau), ("sel_mask", sel_mask),
                 ("scores", scores), ("lse", lse), ("out_err", out_err),
                 ("out_dense", out_dense), ("out_var", out_var)):
        setattr(a, f, None if t is None else t.data_ptr())
    a.flags = int(flags)
    return a


def ctopk_certify_ex(q, K, V, eps, *, head_scale=None, workspace=None, want_mask=False,
                     want_scores=False, want_lse=False, want_err=False, want_dense=False,
                     want_var=False, bound=False, stream=None):
    """Full form: q [Hq, d], K/V [Hkv, n, d] in bf16 or fp32, optional per-head
    scale [Hq] fp32 and caller workspace (uint8 tensor).

    Returns a dict with out, k_eps, tau and, on request, sel_mask
    [Hq, ceil(n/32)] int32 bit words, scores [Hq, n] fp32, lse [Hq] fp64,
    out_err [Hq] fp64 (||Attn - Attn_k||_2), out_dense [Hq, d] fp32 (Attn) and
    out_var [Hq] fp64 (Var_P(V), which bounds the output error by
    sqrt(tau Var_P(V) / (1 - tau))).
    bound=True certifies with the blockwise bound (CTOPK_FLAG_BOUND): k_eps is
    then the number of keys kept and tau the certified bound on their TV."""
    import torch
    lib = load()
    for name, t in (("q", q), ("K", K), ("V", V)):
        _require_cuda_contig(name, t)
    if not (q.dtype == K.dtype == V.dtype):
        raise TypeError("q, K and V must share one dtype")
    n_q, d = q.shape
    n_kv, n, _ = K.shape
    dev = q.device
    res = {
        "out": torch.empty((n_q, d), dtype=torch.float32, device=dev),
        "k_eps": torch.empty(n_q, dtype=torch.int32, device=dev),
        "tau": torch.empty(n_q, dtype=torch.float64, device=dev),
    }
    if want_mask:
        res["sel_mask"] = torch.empty((n_q, (n + 31) // 32), dtype=torch.int32, device=dev)
    if want_scores:
        res["scores"] = torch.empty((n_q, n), dtype=torch.float32, device=dev)
    if want_lse:
        res["lse"] = torch.empty(n_q, dtype=torch.float64, device=dev)
    if want_err:
        res["out_err"] = torch.empty(n_q, dtype=torch.float64, device=dev)
    if want_dense:
        res["out_dense"] = torch.empty((n_q, d), dtype=torch.float32, device=dev)
    if want_var:
        res["out_var"] = torch.empty(n_q, dtype=torch.float64, device=dev)
    if head_scale is not None:
        _require_cuda_contig("head_scale", head_scale)
        if head_scale.dtype != torch.float32 or head_scale.numel() != n_q:
            raise ValueError("head_scale must be float32 with one entry per query head")
    a = make_args(q, K, V, eps, head_scale=head_scale, workspace=workspace, out=res["out"],
                  k_eps=res["k_eps"], tau=res["tau"], sel_mask=res.get("sel_mask"),
                  scores=res.get("scores"), lse=res.get("lse"), out_err=res.get("out_err"),
                  out_dense=res.get("out_dense"), out_var=res.get("out_var"),
                  flags=CTOPK_FLAG_BOUND if bound else 0)
    _check(lib.ctopk_certify_ex(ctypes.byref(a), _stream(stream)))
    return res


def ctopk_certify_logits(logits, V, eps, *, n_v=None, workspace=None, want_mask=False,
                         want_lse=False, stream=None):
    """Select-only path on given fp32 logits [rows, n]; V [n_v, n, dv] (bf16 or
    fp32), row r reads V[r // (rows // n_v)]."""
    import torch
    lib = load()
    _require_cuda_contig("logits", logits)
    _require_cuda_contig("V", V)
    if logits.dtype != torch.float32:
        raise TypeError("logits must be float32")
    rows, n = logits.shape
    if V.dim() == 2:
        V = V.unsqueeze(0)
    nv, nn, dv = V.shape
    if n_v is None:
        n_v = nv
    dev = logits.device
    out = torch.empty((rows, dv), dtype=torch.float32, device=dev)
    k_eps = torch.empty(rows, dtype=torch.int32, device=dev)
    tau = torch.empty(rows, dtype=torch.float64, device=dev)
    mask = torch.empty((rows, (n + 31) // 32), dtype=torch.int32, device=dev) if want_mask else None
    lse = torch.empty(rows, dtype=torch.float64, device=dev) if want_lse else None
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.ctopk_certify_logits(_ptr(logits), _ptr(V), _dtype_code(V), n, dv, rows, n_v,
                                    float(eps), _ptr(workspace), wsb, _stream(stream),
                                    _ptr(out), _ptr(k_eps), _ptr(tau), _ptr(mask), _ptr(lse)))
    res = {"out": out, "k_eps": k_eps, "tau": tau}
    if want_mask:
        res["sel_mask"] = mask
    if want_lse:
        res["lse"] = lse
    return res


def default_scale(d: int) -> float:
    """The float32 value of 1/sqrt(d) the library uses when no scale is given."""
    import numpy as np
    return float(np.float32(1.0 / math.sqrt(d)))


# ---------------------------------------------------------------------------
# 4-bit key copy and exact candidates
# ---------------------------------------------------------------------------
def ctopk_quantize_k4(K, *, stream=None):
    """4-bit copy of K [Hkv, n, d] (bf16 or fp32): returns (K4 uint8
    [Hkv, n, d/2], kscale fp32 [Hkv, n], kres fp32 [Hkv, n])."""
    import torch
    lib = load()
    _require_cuda_contig("K", K)
    n_kv, n, d = K.shape
    dev = K.device
    K4 = torch.empty((n_kv, n, d // 2), dtype=torch.uint8, device=dev)
    ks = torch.empty((n_kv, n), dtype=torch.float32, device=dev)
    kr = torch.empty((n_kv, n), dtype=torch.float32, device=dev)
    _check(lib.ctopk_quantize_k4(_ptr(K), _dtype_code(K), n, d, n_kv, _ptr(K4), _ptr(ks), _ptr(kr),
                                 _stream(stream)))
    return K4, ks, kr


def make_k4_args(q, K, K4, kscale, kres, threshold, *, head_scale=None, workspace=None,
                 sel_mask=None, count=None, rescored=None, bounds=None) -> CtopkK4Args:
    """Fill a CtopkK4Args from tensors (no checks beyond what the C side does)."""
    n_q, d = q.shape
    n_kv, n, _ = K.shape
    a = CtopkK4Args()
    a.q, a.K = _ptr(q), _ptr(K)
    a.dtype = _dtype_code(K)
    a.n, a.d, a.n_q_heads, a.n_kv_heads = n, d, n_q, n_kv
    a.head_scale = _ptr(head_scale)
    a.K4, a.kscale, a.kres, a.threshold = _ptr(K4), _ptr(kscale), _ptr(kres), _ptr(threshold)
    if workspace is not None:
        a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel()
    a.sel_mask, a.count, a.rescored, a.bounds = _ptr(sel_mask), _ptr(count), _ptr(rescored), _ptr(bounds)
    return a


def ctopk_validate_k4(args: CtopkK4Args) -> int:
    return int(load().ctopk_validate_k4(ctypes.byref(args)))


def ctopk_k4_workspace_bytes(n, n_q_heads, n_kv_heads) -> int:
    return int(load().ctopk_k4_workspace_bytes(n, n_q_heads, n_kv_heads))


def ctopk_candidates_k4(q, K, K4, kscale, kres, threshold, *, head_scale=None, workspace=None,
                        want_bounds=False, stream=None):
    """Exact candidates {i : s_hi >= threshold[h]} from the 4-bit copy.
    Returns a dict: sel_mask [Hq, ceil(n/32)] int32 words, count [Hq] int32,
    rescored [Hkv] int32 and, on request, bounds [Hq, n, 2] fp32 (lo, hi)."""
    import torch
    lib = load()
    for name, t in (("q", q), ("K", K), ("K4", K4), ("kscale", kscale), ("kres", kres),
                    ("threshold", threshold)):
        _require_cuda_contig(name, t)
    if q.dtype != K.dtype:
        raise TypeError("q and K must share one dtype")
    n_q, d = q.shape
    n_kv, n, _ = K.shape
    dev = q.device
    res = {
        "sel_mask": torch.empty((n_q, (n + 31) // 32), dtype=torch.int32, device=dev),
        "count": torch.empty(n_q, dtype=torch.int32, device=dev),
        "rescored": torch.empty(n_kv, dtype=torch.int32, device=dev),
    }
    if want_bounds:
        res["bounds"] = torch.empty((n_q, n, 2), dtype=torch.float32, device=dev)
    if head_scale is not None:
        _require_cuda_contig("head_scale", head_scale)
    a = make_k4_args(q, K, K4, kscale, kres, threshold, head_scale=head_scale, workspace=workspace,
                     sel_mask=res["sel_mask"], count=res["count"], rescored=res["rescored"],
                     bounds=res.get("bounds"))
    _check(lib.ctopk_candidates_k4(ctypes.byref(a), _stream(stream)))
    return res
