"""Device parity of the blockwise-bound certificate (CTOPK_FLAG_BOUND)
against the fp64 oracle (oracle.certify_bound and the truncation's exact TV).

The bound keeps every key scoring at or above a threshold, so the checks are
exact properties of the certificate plus agreement with the oracle's bound:
tau <= eps; the exact TV of the kept set is at most tau; the kept set is a
top set of the device's scores; k equals the kept count and is never below
the minimal k_eps; tau and k agree with the oracle's; out is the oracle's
renormalised output over the kept set.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads
from parity import OUT_RTOL_BF16, OUT_RTOL_F32, rel_l2, unpack_mask

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


def check_bound(ct, wl, eps, label, certificate=False):
    n, n_q, n_kv, d = wl["n"], wl["n_q_heads"], wl["n_kv_heads"], wl["d"]
    _say(f"bound {label} eps={eps} n={n} Hq={n_q} Hkv={n_kv} d={d}")
    res = ct.ctopk_certify_ex(dev(wl["q"]), dev(wl["K"]), dev(wl["V"]), eps,
                              head_scale=dev(wl["head_scale"]), want_mask=True, want_scores=True,
                              want_lse=True, want_err=certificate, bound=True)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in res.items()}
    kept = unpack_mask(g["sel_mask"], n)
    G = n_q // n_kv
    q64, K64, V64 = oracle.as_f64(wl["q"]), oracle.as_f64(wl["K"]), oracle.as_f64(wl["V"])
    sc = np.asarray(wl["head_scale"], dtype=np.float32).astype(np.float64)
    S = np.stack([sc[h] * (K64[h // G] @ q64[h]) for h in range(n_q)])
    ref = oracle.certify_bound(S, V64, eps, np.arange(n_q) // G)
    # The oracle's bound on the device's own fp32 scores: only the arithmetic
    # of U(t) (fp32 block masses rounded up) and the fp32 threshold differ.
    ref_dev = oracle.certify_bound(g["scores"].astype(np.float64), V64, eps, np.arange(n_q) // G)
    exact = oracle.certify_scores(S, V64, eps, np.arange(n_q) // G, with_diagnostics=False)
    out_rtol = OUT_RTOL_BF16 if wl["dtype"] == "bf16" else OUT_RTOL_F32
    worst_out, worst_tau, worst_dk = 0.0, 0.0, 0
    for h in range(n_q):
        keep = kept[h]
        assert g["k_eps"][h] == keep.sum(), f"row {h}: k is not the kept count"
        assert g["tau"][h] <= eps * (1 + 1e-12), f"row {h}: tau above eps"
        s_dev = g["scores"][h]
        if (~keep).any():
            assert s_dev[keep].min() >= s_dev[~keep].max(), f"row {h}: kept set is not a top set"
        P = oracle.softmax(S[h])
        tv = oracle.tv_half_l1(P, oracle.truncation(P, keep))
        assert tv <= g["tau"][h] * (1 + 1e-5) + 1e-9, f"row {h}: TV {tv} above the bound {g['tau'][h]}"
        assert g["k_eps"][h] >= exact["k_eps"][h] or exact["near_boundary"][h]
        assert abs(g["tau"][h] - ref["tau_bound"][h]) <= 1e-5
        assert abs(int(g["k_eps"][h]) - int(ref["k"][h])) <= max(2, 2e-3 * n)
        dk = abs(int(g["k_eps"][h]) - int(ref_dev["k"][h]))
        worst_dk = max(worst_dk, dk)
        assert dk == 0, f"row {h}: k {g['k_eps'][h]} vs {ref_dev['k'][h]} on the device's scores"
        w = np.exp(S[h] - S[h].max())
        out_ref = (w[keep] @ V64[h // G][keep]) / w[keep].sum()
        e = rel_l2(g["out"][h][None], out_ref[None])[0]
        assert e <= out_rtol, f"row {h}: out rel L2 {e:.2e}"
        worst_out, worst_tau = max(worst_out, e), max(worst_tau, abs(g["tau"][h] - ref["tau_bound"][h]))
        if certificate:
            dense = (w @ V64[h // G]) / w.sum()
            err = np.linalg.norm(dense - out_ref)
            assert abs(g["out_err"][h] - err) <= 1e-3 * max(err, 1e-12) + 1e-7
    print(f"{label}: mean k/n {g['k_eps'].mean() / n:.3f} (minimal {exact['k_eps'].mean() / n:.3f}), "
          f"max |tau - ref| {worst_tau:.1e}, max out rel L2 {worst_out:.1e}, "
          f"max |k - k on the device's scores| {worst_dk}", flush=True)


@pytest.mark.parametrize("eps", [0.01, 0.1, 0.5])
def test_bound_gqa_decode_small(ct, eps):
    check_bound(ct, workloads.gqa_decode(n=5000, temp_range=(0.5, 4.0)), eps, "gqa_decode")


def test_bound_gqa_decode_full(ct):
    check_bound(ct, workloads.gqa_decode(), 0.01, "gqa_decode full")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 8, 16])
def test_bound_fp32(ct, d, G):
    wl = workloads.gqa_decode(n=3001, n_q=2 * G, n_kv=2, d=d, planted=5, temp_range=(0.5, 2.0))
    wl = dict(wl, q=workloads.bf16_to_f32(wl["q"]), K=workloads.bf16_to_f32(wl["K"]),
              V=workloads.bf16_to_f32(wl["V"]), dtype="f32")
    check_bound(ct, wl, 0.05, f"fp32 d={d} G={G}")


def test_bound_long_decode(ct):
    check_bound(ct, workloads.long_decode(batch=1), 0.01, "long_decode n=131072")


def test_bound_largest_row(ct):
    wl = workloads.long_decode(n=262144, batch=1, n_q=8, n_kv=2)  # the bound's largest row
    check_bound(ct, wl, 0.01, "long_decode n=262144")


@pytest.mark.parametrize("n", [1, 63, 64, 65, 1000])
def test_bound_ragged(ct, n):
    check_bound(ct, workloads.gqa_decode(n=n, n_q=8, n_kv=2), 0.05, f"ragged n={n}")


def test_bound_equal_scores(ct):
    # q = 0: every score 0, Z = n, so every key is kept and tau is eps up to rounding
    wl = workloads.gqa_decode(n=4096, n_q=4, n_kv=1)
    wl = dict(wl, q=np.zeros_like(wl["q"]))
    check_bound(ct, wl, 0.05, "equal scores")
    res = ct.ctopk_certify_ex(dev(wl["q"]), dev(wl["K"]), dev(wl["V"]), 0.05, bound=True)
    torch.cuda.synchronize()
    assert np.all(res["k_eps"].cpu().numpy() == 4096)
    assert np.allclose(res["tau"].cpu().numpy(), 0.05, rtol=1e-5)


def test_bound_with_certificate(ct):
    check_bound(ct, workloads.gqa_decode(n=6000), 0.05, "with output error", certificate=True)


@pytest.mark.parametrize("eps", [1e-4, 0.9])
def test_bound_extreme_eps(ct, eps):
    check_bound(ct, workloads.gqa_decode(n=3000, n_q=16, n_kv=1, temp_range=(0.5, 8.0)), eps,
                f"eps={eps}, group of 16")


def test_bound_is_deterministic(ct):
    # integer atomics and fixed-order sums: two calls agree bit for bit
    wl = workloads.gqa_decode(n=9000, temp_range=(0.5, 4.0))
    _say("bound determinism n=9000")
    args = (dev(wl["q"]), dev(wl["K"]), dev(wl["V"]), 0.05)
    a = ct.ctopk_certify_ex(*args, head_scale=dev(wl["head_scale"]), want_mask=True, bound=True)
    b = ct.ctopk_certify_ex(*args, head_scale=dev(wl["head_scale"]), want_mask=True, bound=True)
    torch.cuda.synchronize()
    for key in ("out", "k_eps", "tau", "sel_mask"):
        assert torch.equal(a[key], b[key]), key


def test_bound_on_all_queries_shape(ct):
    # all queries of a head (groups of 512 rows): the bound plan's value stream
    # is the MFMA one for wide groups
    wl = workloads.encoder(batch=1, heads=1)
    check_bound(ct, wl, 0.05, "all queries, 512 keys")


def test_bound_with_caller_workspace(ct):
    wl = workloads.gqa_decode(n=5000)
    _say("bound with caller workspace")
    need = ct.ctopk_workspace_bytes(5000, 128, 32, 8)
    raw = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    off = (-raw.data_ptr()) % 256
    ws = raw[off:off + need]
    args = (dev(wl["q"]), dev(wl["K"]), dev(wl["V"]), 0.05)
    a = ct.ctopk_certify_ex(*args, head_scale=dev(wl["head_scale"]), workspace=ws, bound=True)
    b = ct.ctopk_certify_ex(*args, head_scale=dev(wl["head_scale"]), bound=True)
    torch.cuda.synchronize()
    for key in ("out", "k_eps", "tau"):
        assert torch.equal(a[key], b[key]), key
