"""Device parity: libctopk (through its C ABI) against the fp64 oracle.

Every test here needs an MI355X; each prints the case it runs before the GPU
step so a failing run names it.
"""
import math
import sys

import numpy as np
import pytest

import oracle
import workloads
from parity import (OUT_RTOL_BF16, OUT_RTOL_F32, compare, rel_l2, score_band, unpack_mask)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def ct():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import certified_top_sparse_amd as c
    c.load()
    return c


def dev(x):
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def to_np(res):
    out = {k: v.cpu().numpy() for k, v in res.items()}
    return out


def run_decode(ct, wl, eps, want_scores=False, want_lse=False, workspace=None, scale=True):
    q, K, V = dev(wl["q"]), dev(wl["K"]), dev(wl["V"])
    hs = dev(wl["head_scale"]) if scale else None
    res = ct.ctopk_certify_ex(q, K, V, eps, head_scale=hs, want_mask=True,
                              want_scores=want_scores, want_lse=want_lse, workspace=workspace)
    torch.cuda.synchronize()
    g = to_np(res)
    g["sel_mask"] = unpack_mask(g["sel_mask"], wl["n"])
    return g


def check_decode(ct, wl, eps, label, rows=None, **kw):
    _say(f"{label} eps={eps} n={wl['n']} Hq={wl['n_q_heads']} Hkv={wl['n_kv_heads']} d={wl['d']}")
    g = run_decode(ct, wl, eps, **kw)
    n_q, n_kv = wl["n_q_heads"], wl["n_kv_heads"]
    G = n_q // n_kv
    if rows is None:
        rows = np.arange(n_q)
    q64 = oracle.as_f64(wl["q"])
    K64 = oracle.as_f64(wl["K"])
    V64 = oracle.as_f64(wl["V"])
    sc = np.asarray(wl["head_scale"], dtype=np.float32).astype(np.float64)
    S = np.stack([sc[h] * (K64[h // G] @ q64[h]) for h in rows])
    row_to_v = np.arange(n_q) // G
    ref = oracle.certify_scores(S, V64, eps, row_to_v[rows])
    band = np.array([score_band(q64[h], K64[h // G], sc[h], wl["d"]) for h in rows])
    out_rtol = OUT_RTOL_BF16 if wl["dtype"] == "bf16" else OUT_RTOL_F32
    rep = compare(g, ref, S, V64, row_to_v, eps, out_rtol, rows=rows, score_band=band, label=label)
    print(rep, flush=True)
    return g, ref, S


# ---------------------------------------------------------------------------
# single-query fp32 workload
# ---------------------------------------------------------------------------
def test_single_query_full(ct):
    wl = workloads.single_query()
    check_decode(ct, wl, 0.01, "single_query n=1024 fp32")


@pytest.mark.parametrize("variant", range(16))
def test_single_query_bruteforce_variants(ct, variant):
    wl = workloads.single_query(n=16, seed_extra=(variant,))
    eps = (0.01, 0.05, 0.2, 0.5)[variant % 4]
    g, ref, S = check_decode(ct, wl, eps, f"single_query n=16 variant {variant}")
    # exhaustive check of minimality on the device's own answer
    P = oracle.softmax(S[0])
    k = int(g["k_eps"][0])
    head = g["sel_mask"][0]
    assert head.sum() == k
    assert 1.0 - P[head].sum() <= eps + 1e-6
    if k > 1:
        best = np.sort(P)[::-1][: k - 1].sum()
        assert 1.0 - best > eps - 1e-6


@pytest.mark.parametrize("n", [1, 2, 63, 257, 1000, 4097])
def test_single_query_ragged(ct, n):
    wl = workloads.single_query(n=n, seed_extra=(n,))
    check_decode(ct, wl, 0.01, f"single_query ragged n={n}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("G", [1, 3, 4, 8, 16])
def test_decode_shapes(ct, d, dtype, G):
    n_kv = 2
    wl = workloads.gqa_decode(n=3001, n_q=G * n_kv, n_kv=n_kv, d=d, planted=5)
    if dtype == "f32":
        wl = dict(wl, q=workloads.bf16_to_f32(wl["q"]), K=workloads.bf16_to_f32(wl["K"]),
                  V=workloads.bf16_to_f32(wl["V"]), dtype="f32")
    check_decode(ct, wl, 0.05, f"decode d={d} {dtype} G={G}")


# ---------------------------------------------------------------------------
# GQA decode workloads
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("eps", [0.01, 0.1])
def test_gqa_decode_small(ct, eps):
    wl = workloads.gqa_decode(n=5000)
    check_decode(ct, wl, eps, "gqa_decode n=5000")


@pytest.mark.parametrize("eps", [0.01, 0.1])
def test_gqa_decode_full(ct, eps):
    wl = workloads.gqa_decode()
    check_decode(ct, wl, eps, "gqa_decode n=32768 (full)")


def test_gqa_decode_default_call(ct):
    """ctopk_certify (bf16, scale 1/sqrt(d)) equals ctopk_certify_ex with the same scale."""
    wl = workloads.gqa_decode(n=8192)
    _say("gqa_decode n=8192 via ctopk_certify")
    q, K, V = dev(wl["q"]), dev(wl["K"]), dev(wl["V"])
    out, k, tau = ct.ctopk_certify(q, K, V, 0.01)
    res = ct.ctopk_certify_ex(q, K, V, 0.01)
    torch.cuda.synchronize()
    assert torch.equal(k, res["k_eps"]) and torch.equal(out, res["out"])
    check_decode(ct, wl, 0.01, "gqa_decode n=8192 default scale", scale=False)


@pytest.mark.parametrize("eps", [0.01, 0.1])
def test_long_decode_full(ct, eps):
    wl = workloads.long_decode()
    check_decode(ct, wl, eps, "long_decode n=131072 Hq=128 (full)")


def test_scores_and_lse(ct):
    wl = workloads.gqa_decode(n=4000)
    _say("scores/lse gqa_decode n=4000")
    g = run_decode(ct, wl, 0.01, want_scores=True, want_lse=True)
    G = wl["n_q_heads"] // wl["n_kv_heads"]
    q64 = oracle.as_f64(wl["q"])
    K64 = oracle.as_f64(wl["K"])
    sc = wl["head_scale"].astype(np.float64)
    for h in range(wl["n_q_heads"]):
        s_ref = sc[h] * (K64[h // G] @ q64[h])
        bound = 2.0 * wl["d"] * 2.0 ** -24 * sc[h] * (np.abs(K64[h // G]) @ np.abs(q64[h])) + 1e-30
        assert np.all(np.abs(g["scores"][h] - s_ref) <= bound + np.abs(s_ref) * 2.0 ** -23)
        m = s_ref.max()
        lse_ref = m + math.log(np.exp(s_ref - m).sum())
        assert abs(g["lse"][h] - lse_ref) < 1e-5


def test_caller_workspace_matches_cached(ct):
    wl = workloads.gqa_decode(n=6000)
    _say("caller workspace gqa_decode n=6000")
    nbytes = ct.ctopk_workspace_bytes(6000, 128, 32, 8, ct.CTOPK_BF16)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a = run_decode(ct, wl, 0.01)
    b = run_decode(ct, wl, 0.01, workspace=ws)
    for key in ("k_eps", "out", "sel_mask"):
        assert np.array_equal(a[key], b[key])
    assert np.allclose(a["tau"], b["tau"], rtol=1e-14, atol=0)


def test_determinism(ct):
    wl = workloads.gqa_decode(n=20000)
    _say("determinism gqa_decode n=20000")
    a = run_decode(ct, wl, 0.01)
    b = run_decode(ct, wl, 0.01)
    for key in ("k_eps", "out", "sel_mask"):
        assert np.array_equal(a[key], b[key])
    assert np.allclose(a["tau"], b["tau"], rtol=1e-13, atol=0)


# ---------------------------------------------------------------------------
# overlapped plan: the select beside a dense value stream, then the tail
# correction (dense minus tail, or the head directly, per chunk)
# ---------------------------------------------------------------------------
def plan_of(ct, wl):
    q, K, V = dev(wl["q"][:1]), dev(wl["K"][:1, :1]), dev(wl["V"][:1, :1])
    a = ct.make_args(q, K, V, 0.01, out=q, k_eps=q, tau=q)
    a.n, a.n_q_heads, a.n_kv_heads = wl["n"], wl["n_q_heads"], wl["n_kv_heads"]
    a.d = wl["d"]
    return ct.ctopk_plan(a)


def as_f32(wl):
    return dict(wl, q=workloads.bf16_to_f32(wl["q"]), K=workloads.bf16_to_f32(wl["K"]),
                V=workloads.bf16_to_f32(wl["V"]), dtype="f32")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_overlap_shapes(ct, d, dtype, G):
    # every head-group width (1, 2, 4, 8, and 16 as two groups of 8); n is not
    # a multiple of the 256-key tile
    wl = workloads.gqa_decode(n=20000, n_q=2 * G, n_kv=2, d=d, planted=5, temp_range=(0.5, 2.0))
    if dtype == "f32":
        wl = as_f32(wl)
    assert plan_of(ct, wl) == ct.CTOPK_PLAN_DECODE_OVERLAP
    check_decode(ct, wl, 0.05, f"overlap d={d} {dtype} G={G}")


@pytest.mark.parametrize("eps", [0.001, 0.3, 0.9])
def test_overlap_eps(ct, eps):
    # small eps: short tails (chunks subtract the tail from the dense sums);
    # large eps: small heads (chunks sum the head directly)
    wl = workloads.gqa_decode(n=24577, temp_range=(0.5, 4.0))
    assert plan_of(ct, wl) == ct.CTOPK_PLAN_DECODE_OVERLAP
    check_decode(ct, wl, eps, "overlap gqa_decode n=24577")


def test_overlap_smallest_row(ct):
    wl = workloads.gqa_decode(n=16385, n_q=64, n_kv=8, d=64)
    assert plan_of(ct, wl) == ct.CTOPK_PLAN_DECODE_OVERLAP
    check_decode(ct, wl, 0.01, "overlap gqa_decode n=16385 Hq=64")
    wl = workloads.gqa_decode(n=16384, n_q=64, n_kv=8, d=64)
    assert plan_of(ct, wl) == ct.CTOPK_PLAN_DECODE
    check_decode(ct, wl, 0.01, "serial gqa_decode n=16384 Hq=64")


# ---------------------------------------------------------------------------
# output-level certificate: ||Attn - Attn_k||_2 and the untruncated output
# ---------------------------------------------------------------------------
def _certificate_case(ct, wl, eps, label, rtol, same_path=True, same_select=True):
    _say(f"certificate {label} eps={eps} n={wl['n']} Hq={wl['n_q_heads']} d={wl['d']}")
    q, K, V = dev(wl["q"]), dev(wl["K"]), dev(wl["V"])
    hs = dev(wl["head_scale"])
    plain = ct.ctopk_certify_ex(q, K, V, eps, head_scale=hs)
    res = ct.ctopk_certify_ex(q, K, V, eps, head_scale=hs, want_err=True, want_dense=True)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in res.items()}
    p = {k: v.cpu().numpy() for k, v in plain.items()}
    if same_select:  # the certificate does not change the select
        assert np.array_equal(g["k_eps"], p["k_eps"])
        assert np.array_equal(g["tau"], p["tau"])
    if same_path:  # nor, on one plan, the output
        assert np.array_equal(g["out"], p["out"])
    else:  # the plain call's plan may sum the head in another order
        assert rel_l2(p["out"], g["out"]).max() <= rtol
    n_q, n_kv = wl["n_q_heads"], wl["n_kv_heads"]
    G = n_q // n_kv
    q64, K64, V64 = oracle.as_f64(wl["q"]), oracle.as_f64(wl["K"]), oracle.as_f64(wl["V"])
    sc = np.asarray(wl["head_scale"], dtype=np.float32).astype(np.float64)
    S = np.stack([sc[h] * (K64[h // G] @ q64[h]) for h in range(n_q)])
    ref = oracle.certify_scores(S, V64, eps, np.arange(n_q) // G)
    kok = g["k_eps"] == ref["k_eps"]
    assert kok.sum() >= n_q - int(ref["near_boundary"].sum())
    dense_err = rel_l2(g["out_dense"], ref["out_dense"])
    assert dense_err.max() <= rtol, f"dense output rel L2 {dense_err.max():.3e}"
    e_ref = ref["out_err"][kok]
    e_gpu = g["out_err"][kok]
    rel = np.abs(e_gpu - e_ref) / np.maximum(e_ref, 1e-12)
    assert rel.max() <= rtol, f"output error off by {rel.max():.3e} (relative)"
    print(f"{label}: dense rel L2 max {dense_err.max():.2e}, ||Attn - Attn_k|| rel err max "
          f"{rel.max():.2e}, mean ||Attn - Attn_k|| {e_ref.mean():.3e}", flush=True)


@pytest.mark.parametrize("eps", [0.01, 0.1])
def test_certificate_gqa_decode(ct, eps):
    _certificate_case(ct, workloads.gqa_decode(n=6000), eps, "gqa_decode n=6000", 1e-3)


def test_certificate_gqa_decode_full(ct):
    # the plain call runs the overlapped plan, the certificate the serial one
    _certificate_case(ct, workloads.gqa_decode(), 0.01, "gqa_decode n=32768 (full)", 1e-3,
                      same_path=False)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_certificate_fp32(ct, d, G):
    wl = workloads.gqa_decode(n=2500, n_q=2 * G, n_kv=2, d=d, planted=3)
    wl = dict(wl, q=workloads.bf16_to_f32(wl["q"]), K=workloads.bf16_to_f32(wl["K"]),
              V=workloads.bf16_to_f32(wl["V"]), dtype="f32")
    _certificate_case(ct, wl, 0.05, f"fp32 d={d} G={G}", 1e-5)


def test_certificate_on_encoder_shape(ct):
    # all-queries shapes take the general path when the certificate is asked for
    wl = workloads.encoder(batch=1, heads=2)
    _certificate_case(ct, wl, 0.01, "encoder shape 1x2x512x64", 1e-3, same_path=False,
                      same_select=False)


# ---------------------------------------------------------------------------
# adversarial select inputs
# ---------------------------------------------------------------------------
def _logits_case(ct, L, V, eps, label, n_v=1, out_rtol=OUT_RTOL_F32):
    _say(f"{label} rows={L.shape[0]} n={L.shape[1]} eps={eps}")
    res = ct.ctopk_certify_logits(dev(L), dev(V), eps, n_v=n_v, want_mask=True, want_lse=True)
    torch.cuda.synchronize()
    g = to_np(res)
    g["sel_mask"] = unpack_mask(g["sel_mask"], L.shape[1])
    R = L.shape[0]
    row_to_v = np.arange(R) // (R // n_v)
    V64 = oracle.as_f64(V)
    ref = oracle.certify_scores(L.astype(np.float64), V64, eps, row_to_v)
    rep = compare(g, ref, L.astype(np.float64), V64, row_to_v, eps, out_rtol, label=label)
    print(rep, flush=True)
    return g, ref


def test_all_equal_scores(ct):
    n = 20000  # more ties than fit in LDS: exercises full-row re-read levels
    L = np.zeros((3, n), dtype=np.float32)
    L[1] = 1.5
    L[2] = -7.25
    V = np.random.default_rng(1).standard_normal((1, n, 64)).astype(np.float32)
    g, ref = _logits_case(ct, L, V, 0.01234, "all equal scores")
    k = math.ceil(n * (1 - 0.01234))
    assert (g["k_eps"] == k).all()
    assert g["sel_mask"][:, :k].all() and not g["sel_mask"][:, k:].any()


def test_signed_zeros_and_ties(ct):
    n = 4096
    rng = np.random.default_rng(4)
    L = rng.choice(np.array([-0.0, 0.0, 1.0, -1.0], dtype=np.float32), size=(4, n))
    V = rng.standard_normal((1, n, 64)).astype(np.float32)
    for eps in (0.05, 0.3):
        _logits_case(ct, L, V, eps, "signed zeros and ties")


def test_wide_dynamic_range(ct):
    rng = np.random.default_rng(6)
    n = 10000
    L = (rng.standard_normal((8, n)) * 25.0).astype(np.float32)  # range ~ 200
    L[:, 17] = 90.0
    V = rng.standard_normal((1, n, 64)).astype(np.float32)
    for eps in (1e-3, 0.2):
        _logits_case(ct, L, V, eps, "dynamic range")


@pytest.mark.parametrize("n", [30000, 70000])
def test_cut_bin_straddles_zero(ct, n):
    """Thousands of scores in the first-level bin that contains 0, on both
    sides of it: the candidates' keys share no leading bit (the sign flips), so
    the descent starts from an empty prefix.  n = 30000 keeps the row in the
    select's registers, n = 70000 streams it."""
    rng = np.random.default_rng(n)
    L = rng.uniform(-0.01, 0.01, size=(4, n)).astype(np.float32)
    L[:, 5] = 5.0
    L[:, 9] = -5.0
    V = rng.standard_normal((1, n, 64)).astype(np.float32)
    for eps in (0.3, 0.5, 0.7):
        _logits_case(ct, L, V, eps, f"cut bin straddles zero n={n}")


def test_single_key_rows(ct):
    L = np.array([[3.0], [-2.0]], dtype=np.float32)
    V = np.ones((1, 1, 64), dtype=np.float32)
    g, _ = _logits_case(ct, L, V, 0.5, "n=1")
    assert (g["k_eps"] == 1).all() and (g["tau"] == 0).all()


def test_bf16_values_on_logits_path(ct):
    rng = np.random.default_rng(8)
    L = (2.0 * rng.standard_normal((16, 3000))).astype(np.float32)
    V = workloads.bf16_rne(rng.standard_normal((4, 3000, 128)).astype(np.float32))
    _logits_case(ct, L, V, 0.01, "bf16 V, 4 value heads", n_v=4, out_rtol=1e-5)


@pytest.mark.parametrize("seq", [600, 1000])
def test_all_queries_beyond_the_encoder(ct, seq):
    # every query of a head against more than 512 keys: the general path with
    # groups of `seq` rows per KV head (the MFMA value stream); sampled rows
    wl = workloads.encoder(batch=1, heads=2, seq=seq)
    rows = np.concatenate([np.arange(0, 2 * seq, 7), [2 * seq - 1]])
    check_decode(ct, wl, 0.01, f"all queries, {seq} keys", rows=rows)


@pytest.mark.parametrize("dv,vdt", [(64, "f32"), (128, "bf16"), (128, "f32")])
def test_logits_wide_groups(ct, dv, vdt):
    # groups of 100 rows per V take the MFMA value stream: ragged row tiles,
    # an odd key count (no 16-byte logit loads) and both value types
    rng = np.random.default_rng(77)
    R, n, n_v = 200, 4097, 2
    L = (rng.standard_normal((R, n)) * 2.0).astype(np.float32)
    V = rng.standard_normal((n_v, n, dv)).astype(np.float32)
    if vdt == "bf16":
        V = workloads.bf16_rne(V)
    _logits_case(ct, L, V, 0.05, f"wide groups dv={dv} {vdt}", n_v=n_v,
                 out_rtol=OUT_RTOL_F32 if vdt == "f32" else OUT_RTOL_BF16)


def test_wide_group_stream_is_deterministic(ct):
    rng = np.random.default_rng(78)
    L = dev((rng.standard_normal((256, 3000)) * 2.0).astype(np.float32))
    V = dev(rng.standard_normal((1, 3000, 64)).astype(np.float32))
    _say("wide-group value stream determinism")
    a = ct.ctopk_certify_logits(L, V, 0.02)
    b = ct.ctopk_certify_logits(L, V, 0.02)
    torch.cuda.synchronize()
    assert torch.equal(a["out"], b["out"]) and torch.equal(a["k_eps"], b["k_eps"])


# ---------------------------------------------------------------------------
# logit sweep workloads
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("sigma", workloads.LOGIT_SIGMAS)
@pytest.mark.parametrize("n", [4096, 65536])
def test_logit_sweep(ct, sigma, n):
    wl = workloads.logit_sweep(sigma, n)
    L = dev(wl["logits"])
    V = dev(wl["V"])
    rows = np.arange(0, 1024, 16)
    S = wl["logits"][rows].astype(np.float64)
    V64 = wl["V"].astype(np.float64)
    for eps in workloads.LOGIT_EPS:
        _say(f"logit_sweep sigma={sigma} n={n} eps={eps}")
        res = ct.ctopk_certify_logits(L, V, eps, want_mask=True)
        torch.cuda.synchronize()
        g = to_np(res)
        g["sel_mask"] = unpack_mask(g["sel_mask"], n)
        ref = oracle.certify_scores(S, V64, eps)
        rep = compare(g, ref, S, V64, np.zeros(1024, dtype=np.int64), eps, OUT_RTOL_F32,
                      rows=rows, label=f"logit sweep sigma={sigma} n={n} eps={eps}")
        print(rep, flush=True)
        frac = g["k_eps"].mean() / n
        pred = oracle.gaussian_design_rule(sigma, eps)
        print(f"k/n={frac:.4f} rule={pred:.4f}", flush=True)


def test_logit_sweep_largest(ct):
    n = 1048576
    wl = workloads.logit_sweep(2.0, n)
    _say("logit_sweep sigma=2 n=2^20 rows=1024 eps=0.01 (full size)")
    res = ct.ctopk_certify_logits(dev(wl["logits"]), dev(wl["V"]), 0.01, want_mask=True)
    torch.cuda.synchronize()
    g = to_np(res)
    g["sel_mask"] = unpack_mask(g["sel_mask"], n)
    rows = np.array([0, 311, 777, 1023])
    S = wl["logits"][rows].astype(np.float64)
    V64 = wl["V"].astype(np.float64)
    ref = oracle.certify_scores(S, V64, 0.01)
    rep = compare(g, ref, S, V64, np.zeros(1024, dtype=np.int64), 0.01, OUT_RTOL_F32, rows=rows,
                  label="logit sweep n=2^20")
    print(rep, flush=True)
    frac = g["k_eps"].mean() / n
    assert abs(frac - oracle.gaussian_design_rule(2.0, 0.01)) < 0.005
