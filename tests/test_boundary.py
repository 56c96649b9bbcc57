"""The C ABI boundary on the host: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching a GPU.  CPU only:
ctopk_validate and the workspace-size functions make no HIP call, and the
certify entry points check their arguments before any HIP call."""
import ctypes
import math
import os
import re

import pytest

import certified_top_sparse_amd as ct
from certified_top_sparse_amd import ctopk as cb

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "ctopk.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(cb.LIB_PATH):
        pytest.skip("libctopk.so not built")
    return cb.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"CTOPK_API\s+[\w\s\*]+?\b(ctopk_\w+)\s*\(", text)))


def test_header_declarations_match_binding():
    assert sorted(cb.EXPORTED) == declared_functions()


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    # nothing internal leaks out of the shared object
    out = os.popen(f"nm -D --defined-only {cb.LIB_PATH}").read()
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert exported == set(declared_functions())


def test_version_string(lib):
    assert ct.ctopk_version().startswith("libctopk")


A16 = 1 << 20  # a fake 16-byte-aligned device address (validate never dereferences it)


def good_args(**kw):
    a = cb.CtopkArgs()
    a.q, a.K, a.V = A16, A16 * 2, A16 * 3
    a.dtype = cb.CTOPK_BF16
    a.n, a.d, a.n_q_heads, a.n_kv_heads = 32768, 128, 32, 8
    a.eps = 0.01
    a.out, a.k_eps, a.tau = A16 * 4, A16 * 5, A16 * 6
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_valid_arguments_pass(lib):
    assert ct.ctopk_validate(good_args()) == cb.CTOPK_OK
    assert ct.ctopk_last_error_string() == ""


@pytest.mark.parametrize("field", ["q", "K", "V", "out", "k_eps", "tau"])
def test_null_pointers(lib, field):
    assert ct.ctopk_validate(good_args(**{field: None})) == cb.CTOPK_ERR_NULL
    assert "NULL" in ct.ctopk_last_error_string()


@pytest.mark.parametrize("kw,code", [
    ({"n": 0}, cb.CTOPK_ERR_SHAPE),
    ({"n": -5}, cb.CTOPK_ERR_SHAPE),
    ({"n": 2 ** 31}, cb.CTOPK_ERR_SHAPE),
    ({"d": 96}, cb.CTOPK_ERR_SHAPE),
    ({"d": 256}, cb.CTOPK_ERR_SHAPE),
    ({"n_q_heads": 0}, cb.CTOPK_ERR_SHAPE),
    ({"n_kv_heads": 0}, cb.CTOPK_ERR_SHAPE),
    ({"n_q_heads": 30, "n_kv_heads": 8}, cb.CTOPK_ERR_SHAPE),
    ({"n_q_heads": 70000, "n_kv_heads": 70000}, cb.CTOPK_ERR_UNSUPPORTED),
    ({"n": 2 ** 31 - 1, "n_q_heads": 64, "n_kv_heads": 8}, cb.CTOPK_ERR_UNSUPPORTED),
    ({"dtype": 7}, cb.CTOPK_ERR_UNSUPPORTED),
])
def test_shape_errors(lib, kw, code):
    assert ct.ctopk_validate(good_args(**kw)) == code
    assert ct.ctopk_last_error_string() != ""


@pytest.mark.parametrize("eps", [0.0, 1.0, -0.5, 1.5, math.nan, math.inf, -math.inf])
def test_eps_errors(lib, eps):
    assert ct.ctopk_validate(good_args(eps=eps)) == cb.CTOPK_ERR_EPS


@pytest.mark.parametrize("field,value", [("q", A16 + 8), ("K", A16 + 2), ("V", A16 + 4),
                                         ("out", A16 + 2), ("tau", A16 + 4),
                                         ("k_eps", A16 + 1), ("out_err", A16 + 4),
                                         ("out_dense", A16 + 2), ("out_var", A16 + 4)])
def test_alignment_errors(lib, field, value):
    assert ct.ctopk_validate(good_args(**{field: value})) == cb.CTOPK_ERR_ALIGN


def test_workspace_checks(lib):
    need = ct.ctopk_workspace_bytes(32768, 128, 32, 8, cb.CTOPK_BF16)
    assert need > 32 * 32768 * 4  # at least the score buffer
    assert ct.ctopk_validate(good_args(workspace=A16 * 8, workspace_bytes=need)) == cb.CTOPK_OK
    assert ct.ctopk_validate(good_args(workspace=A16 * 8, workspace_bytes=need - 1)) == \
        cb.CTOPK_ERR_WORKSPACE
    assert ct.ctopk_validate(good_args(workspace=A16 * 8 + 16, workspace_bytes=need)) == \
        cb.CTOPK_ERR_ALIGN


def test_struct_layout_matches_header():
    # the binding's mirror of ctopk_args must keep the header's field order
    text = open(HEADER).read()
    body = text[text.index("typedef struct ctopk_args {"):text.index("} ctopk_args;")]
    body = body[body.index("{") + 1:]
    names = re.findall(r"\b(\w+);", re.sub(r"/\*.*?\*/", "", body, flags=re.S))
    assert names == [f for f, _ in cb.CtopkArgs._fields_]


def test_workspace_sizes(lib):
    assert ct.ctopk_workspace_bytes(0, 128, 32, 8) == 0
    assert ct.ctopk_workspace_bytes(100, 96, 32, 8) == 0
    assert ct.ctopk_workspace_bytes(100, 128, 30, 8) == 0
    a = ct.ctopk_workspace_bytes(1000, 128, 32, 8)
    b = ct.ctopk_workspace_bytes(100000, 128, 32, 8)
    assert 0 < a < b
    assert ct.ctopk_workspace_bytes(4096, 64, 1, 1, cb.CTOPK_F32) > 0
    assert ct.ctopk_logits_workspace_bytes(4096, 64, 1024, 1) > 0
    assert ct.ctopk_logits_workspace_bytes(4096, 100, 1024, 1) == 0
    assert ct.ctopk_logits_workspace_bytes(4096, 64, 1000, 3) == 0


def test_certify_rejects_before_any_gpu_call(lib):
    vp = ctypes.c_void_p
    rc = lib.ctopk_certify(vp(A16), vp(A16), vp(A16), 0, 128, 32, 8, 0.01, None, vp(A16),
                           vp(A16), vp(A16))
    assert rc == cb.CTOPK_ERR_SHAPE
    rc = lib.ctopk_certify(None, vp(A16), vp(A16), 100, 128, 32, 8, 0.01, None, vp(A16),
                           vp(A16), vp(A16))
    assert rc == cb.CTOPK_ERR_NULL
    rc = lib.ctopk_certify(vp(A16), vp(A16), vp(A16), 100, 128, 32, 8, 2.0, None, vp(A16),
                           vp(A16), vp(A16))
    assert rc == cb.CTOPK_ERR_EPS


@pytest.mark.parametrize("kw,code", [
    ({"logits": None}, cb.CTOPK_ERR_NULL),
    ({"n": 0}, cb.CTOPK_ERR_SHAPE),
    ({"dv": 32}, cb.CTOPK_ERR_SHAPE),
    ({"rows": 10, "n_v": 3}, cb.CTOPK_ERR_SHAPE),
    ({"eps": 0.0}, cb.CTOPK_ERR_EPS),
    ({"v_dtype": 5}, cb.CTOPK_ERR_UNSUPPORTED),
    ({"V": A16 + 4}, cb.CTOPK_ERR_ALIGN),
    ({"workspace": A16, "workspace_bytes": 16}, cb.CTOPK_ERR_WORKSPACE),
])
def test_logits_argument_errors(lib, kw, code):
    args = {"logits": A16, "V": A16, "v_dtype": cb.CTOPK_F32, "n": 4096, "dv": 64, "rows": 8,
            "n_v": 1, "eps": 0.01, "workspace": None, "workspace_bytes": 0}
    args.update(kw)
    vp = ctypes.c_void_p
    p = (lambda x: None if x is None else vp(x))
    rc = lib.ctopk_certify_logits(p(args["logits"]), p(args["V"]), args["v_dtype"], args["n"],
                                  args["dv"], args["rows"], args["n_v"], args["eps"],
                                  p(args["workspace"]), args["workspace_bytes"], None, vp(A16),
                                  vp(A16), vp(A16), None, None)
    assert rc == code


def test_kernel_event_arming_limits(lib):
    arr = (ctypes.c_void_p * 18)(*([A16] * 18))
    assert lib.ctopk_record_kernel_events(arr, 18) == cb.CTOPK_ERR_SHAPE
    assert lib.ctopk_record_kernel_events(arr, 3) == cb.CTOPK_ERR_SHAPE  # pairs only
    assert lib.ctopk_record_kernel_events(None, 4) == cb.CTOPK_ERR_NULL
    holes = (ctypes.c_void_p * 2)(A16, None)
    assert lib.ctopk_record_kernel_events(holes, 2) == cb.CTOPK_ERR_NULL
    assert lib.ctopk_record_kernel_events(None, 0) == cb.CTOPK_OK


def test_missing_library_fails_loudly(tmp_path):
    saved = cb._lib
    cb._lib = None
    try:
        with pytest.raises(RuntimeError, match="no CPU fallback"):
            cb.load(str(tmp_path / "nope.so"))
    finally:
        cb._lib = saved


@pytest.mark.parametrize("kw,plan", [
    ({}, cb.CTOPK_PLAN_DECODE_OVERLAP),                           # n = 32768, 32 query rows
    ({"n": 16385}, cb.CTOPK_PLAN_DECODE_OVERLAP),                 # smallest overlapped row
    ({"n": 16384}, cb.CTOPK_PLAN_DECODE),                         # below the register-row band
    ({"n": 32769}, cb.CTOPK_PLAN_DECODE),                         # above it
    ({"dtype": cb.CTOPK_F32}, cb.CTOPK_PLAN_DECODE_OVERLAP),
    ({"d": 64, "n_q_heads": 8, "n_kv_heads": 8}, cb.CTOPK_PLAN_DECODE_OVERLAP),
    ({"n_q_heads": 64, "n_kv_heads": 8}, cb.CTOPK_PLAN_DECODE_OVERLAP),
    # 128 CUs left, but 16 head groups share them: chunks of 4096 keys, more
    # than the tail pass lists
    ({"n_q_heads": 128, "n_kv_heads": 16}, cb.CTOPK_PLAN_DECODE),
    ({"n_q_heads": 136, "n_kv_heads": 136}, cb.CTOPK_PLAN_DECODE),  # fewer than half left
    ({"n_q_heads": 192, "n_kv_heads": 24}, cb.CTOPK_PLAN_DECODE),
    ({"out_err": A16 * 7}, cb.CTOPK_PLAN_DECODE),                 # certificate: serial stream
    ({"out_dense": A16 * 7}, cb.CTOPK_PLAN_DECODE),
    ({"out_var": A16 * 7}, cb.CTOPK_PLAN_DECODE),
    ({"n": 512, "d": 64, "n_q_heads": 512, "n_kv_heads": 8}, cb.CTOPK_PLAN_ENCODER),
    ({"n": 512, "d": 64, "n_q_heads": 512, "n_kv_heads": 8, "out_err": A16 * 7},
     cb.CTOPK_PLAN_DECODE),
    # rows of at most 1024 keys the encoder path does not take: one fused kernel
    ({"n": 1024, "d": 64, "n_q_heads": 1, "n_kv_heads": 1, "dtype": cb.CTOPK_F32},
     cb.CTOPK_PLAN_DECODE_FUSED),
    ({"n": 1024}, cb.CTOPK_PLAN_DECODE_FUSED),
    ({"n": 1}, cb.CTOPK_PLAN_DECODE_FUSED),
    ({"n": 1025}, cb.CTOPK_PLAN_DECODE),
    ({"n": 512, "d": 64, "n_q_heads": 32, "n_kv_heads": 8}, cb.CTOPK_PLAN_DECODE_FUSED),
    ({"n": 1024, "out_err": A16 * 7}, cb.CTOPK_PLAN_DECODE),
    ({"n": 1024, "out_dense": A16 * 7}, cb.CTOPK_PLAN_DECODE),
    ({"n": 1024, "out_var": A16 * 7}, cb.CTOPK_PLAN_DECODE),
])
def test_plan_choice(lib, kw, plan):
    assert ct.ctopk_plan(good_args(**kw)) == plan


def test_plan_reports_validation_status(lib):
    assert ct.ctopk_plan(good_args(eps=1.5)) == cb.CTOPK_ERR_EPS
    assert ct.ctopk_plan(good_args(q=None)) == cb.CTOPK_ERR_NULL
    assert ct.ctopk_plan(good_args(n_kv_heads=5)) == cb.CTOPK_ERR_SHAPE


def test_bound_flag_plan_and_limits(lib):
    assert ct.ctopk_plan(good_args(flags=cb.CTOPK_FLAG_BOUND)) == cb.CTOPK_PLAN_DECODE_BOUND
    # the bound takes precedence over the encoder-shaped and overlapped plans
    assert ct.ctopk_plan(good_args(n=512, d=64, n_q_heads=512, n_kv_heads=8,
                                   flags=cb.CTOPK_FLAG_BOUND)) == cb.CTOPK_PLAN_DECODE_BOUND
    assert ct.ctopk_plan(good_args(n=262144, flags=cb.CTOPK_FLAG_BOUND)) == cb.CTOPK_PLAN_DECODE_BOUND
    assert ct.ctopk_plan(good_args(n=1024, flags=cb.CTOPK_FLAG_BOUND)) == cb.CTOPK_PLAN_DECODE_BOUND
    assert ct.ctopk_validate(good_args(n=262145, flags=cb.CTOPK_FLAG_BOUND)) == cb.CTOPK_ERR_UNSUPPORTED
    assert ct.ctopk_validate(good_args(flags=2)) == cb.CTOPK_ERR_UNSUPPORTED


def good_k4_args(**kw):
    a = cb.CtopkK4Args()
    a.q, a.K = A16, A16 * 2
    a.dtype = cb.CTOPK_BF16
    a.n, a.d, a.n_q_heads, a.n_kv_heads = 32768, 128, 32, 8
    a.K4, a.kscale, a.kres, a.threshold = A16 * 3, A16 * 4, A16 * 5, A16 * 6
    a.sel_mask, a.count = A16 * 7, A16 * 8
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_k4_struct_layout_matches_header():
    text = open(HEADER).read()
    body = text[text.index("ctopk_candidates_k4 -- "):text.index("} ctopk_k4_args;")]
    body = body[body.index("typedef struct {") + len("typedef struct {"):]
    names = re.findall(r"\b(\w+);", re.sub(r"/\*.*?\*/", "", body, flags=re.S))
    assert names == [f for f, _ in cb.CtopkK4Args._fields_]


def test_k4_validation(lib):
    v = ct.ctopk_validate_k4
    assert v(good_k4_args()) == cb.CTOPK_OK
    assert v(good_k4_args(rescored=A16 * 9, bounds=A16 * 10, head_scale=A16 * 11)) == cb.CTOPK_OK
    for f in ("q", "K", "K4", "kscale", "kres", "threshold", "sel_mask", "count"):
        assert v(good_k4_args(**{f: 0})) == cb.CTOPK_ERR_NULL, f
    assert v(good_k4_args(d=96)) == cb.CTOPK_ERR_SHAPE
    assert v(good_k4_args(n=0)) == cb.CTOPK_ERR_SHAPE
    assert v(good_k4_args(n_q_heads=30)) == cb.CTOPK_ERR_SHAPE
    assert v(good_k4_args(n_kv_heads=0)) == cb.CTOPK_ERR_SHAPE
    assert v(good_k4_args(dtype=7)) == cb.CTOPK_ERR_UNSUPPORTED
    assert v(good_k4_args(q=A16 + 4)) == cb.CTOPK_ERR_ALIGN
    assert v(good_k4_args(K=A16 + 8)) == cb.CTOPK_ERR_ALIGN
    assert v(good_k4_args(K4=A16 + 2)) == cb.CTOPK_ERR_ALIGN
    assert v(good_k4_args(bounds=A16 + 4)) == cb.CTOPK_ERR_ALIGN
    need = ct.ctopk_k4_workspace_bytes(32768, 32, 8)
    assert need >= 8 * 512 * 8  # one straddle word per (KV head, tile)
    assert v(good_k4_args(workspace=A16 * 12, workspace_bytes=need)) == cb.CTOPK_OK
    assert v(good_k4_args(workspace=A16 * 12, workspace_bytes=need - 1)) == cb.CTOPK_ERR_WORKSPACE
    assert v(good_k4_args(workspace=A16 * 12 + 16, workspace_bytes=need)) == cb.CTOPK_ERR_ALIGN
    assert ct.ctopk_k4_workspace_bytes(0, 32, 8) == 0
    assert ct.ctopk_k4_workspace_bytes(100, 30, 8) == 0
    # groups wider than 8 heads keep one straddle word per block of 8
    assert ct.ctopk_k4_workspace_bytes(32768, 128, 8) >= 2 * need


def test_k4_entry_points_reject_before_any_gpu_call(lib):
    vp = ctypes.c_void_p
    assert lib.ctopk_candidates_k4(ctypes.byref(good_k4_args(d=96)), None) == cb.CTOPK_ERR_SHAPE
    assert lib.ctopk_quantize_k4(vp(A16), cb.CTOPK_BF16, 4096, 96, 8, vp(A16), vp(A16), vp(A16),
                                 None) == cb.CTOPK_ERR_SHAPE
    assert lib.ctopk_quantize_k4(None, cb.CTOPK_BF16, 4096, 128, 8, vp(A16), vp(A16), vp(A16),
                                 None) == cb.CTOPK_ERR_NULL
    assert lib.ctopk_quantize_k4(vp(A16 + 8), cb.CTOPK_BF16, 4096, 128, 8, vp(A16), vp(A16),
                                 vp(A16), None) == cb.CTOPK_ERR_ALIGN
    assert lib.ctopk_quantize_k4(vp(A16), 5, 4096, 128, 8, vp(A16), vp(A16), vp(A16),
                                 None) == cb.CTOPK_ERR_UNSUPPORTED
    assert lib.ctopk_quantize_k4(vp(A16), cb.CTOPK_BF16, 1 << 30, 128, 32, vp(A16), vp(A16),
                                 vp(A16), None) == cb.CTOPK_ERR_UNSUPPORTED


def test_noalloc_rejects_sizes_beyond_its_array_on_the_host(lib):
    # the fixed scratch array of ctopk_certify_noalloc is checked before any
    # HIP call, so this runs without a GPU
    n_q, n_kv, n, d = 128, 32, 131072, 128
    assert ct.ctopk_workspace_bytes(n, d, n_q, n_kv) > ct.CTOPK_NOALLOC_SCRATCH_BYTES
    vp = ctypes.c_void_p
    rc = lib.ctopk_certify_noalloc(vp(A16), vp(A16 * 2), vp(A16 * 3), n, d, n_q, n_kv, 0.01, None,
                                   vp(A16 * 4), vp(A16 * 5), vp(A16 * 6))
    assert rc == cb.CTOPK_ERR_WORKSPACE
    assert "scratch" in ct.ctopk_last_error_string()
    # and the usual argument checks come first
    rc = lib.ctopk_certify_noalloc(vp(A16), vp(A16 * 2), vp(A16 * 3), n, d, n_q, n_kv, 1.5, None,
                                   vp(A16 * 4), vp(A16 * 5), vp(A16 * 6))
    assert rc == cb.CTOPK_ERR_EPS


def test_noalloc_array_size_matches_the_header(lib):
    text = open(HEADER).read()
    m = re.search(r"#define CTOPK_NOALLOC_SCRATCH_BYTES \((\d+)u \* 1024u \* 1024u\)", text)
    assert m and int(m.group(1)) * 1024 * 1024 == ct.CTOPK_NOALLOC_SCRATCH_BYTES
