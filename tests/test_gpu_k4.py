"""Device parity of the 4-bit key copy and the exact candidate generation
(ctopk_quantize_k4, ctopk_candidates_k4) against the fp64 oracle's copy and
bounds and against the library's own fp32 scores.

* The copy is integer work: codes (packed nibbles) and scales are compared bit
  for bit with oracle.quantize_k4 / pack_k4; the residual bound must cover the
  oracle's exact residual norm and stay within 2e-5 of it.
* The candidate set is {i : s_i >= T} with s the library's fp32 score, so it
  is compared bit for bit with a threshold on the scores ctopk_certify_ex
  returns; against the oracle's fp64 scores it may differ only on keys within
  the fp32 rounding band of T.  Every reported interval must contain both the
  device's and the oracle's score.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads
from parity import unpack_mask

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


def as_f32(wl):
    return dict(wl, q=workloads.bf16_to_f32(wl["q"]), K=workloads.bf16_to_f32(wl["K"]),
                V=workloads.bf16_to_f32(wl["V"]), dtype="f32")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_quantize_matches_oracle(ct, dtype, d):
    _say(f"quantize {dtype} d={d}")
    wl = workloads.gqa_decode(n=3001, n_q=4, n_kv=2, d=d, planted=3)
    if dtype == "f32":
        wl = as_f32(wl)
    K4, ks, kr = ct.ctopk_quantize_k4(dev(wl["K"]))
    torch.cuda.synchronize()
    c, a, rho = oracle.quantize_k4(wl["K"])
    assert np.array_equal(K4.cpu().numpy(), oracle.pack_k4(c))
    assert np.array_equal(ks.cpu().numpy(), a)
    kr = kr.cpu().numpy().astype(np.float64)
    assert np.all(kr >= rho)
    assert np.all(kr <= rho * (1 + 2e-5) + 1e-30)


def test_quantize_zero_and_exact_rows(ct):
    _say("quantize zero and exact rows")
    rng = np.random.default_rng(7)
    c0 = rng.integers(-7, 8, size=(2, 300, 64)).astype(np.float32)
    c0[..., 0] = 7.0
    K = (c0 * np.float32(0.25)).astype(np.float32)
    K[0, 5] = 0.0
    K4, ks, kr = ct.ctopk_quantize_k4(dev(K))
    torch.cuda.synchronize()
    c, a, rho = oracle.quantize_k4(K)
    assert np.array_equal(K4.cpu().numpy(), oracle.pack_k4(c))
    assert np.array_equal(ks.cpu().numpy(), a)
    assert np.all(kr.cpu().numpy() < 1e-30)  # no residual: the bound is a denormal at most


def run_k4(ct, wl, T, want_bounds=True):
    q, K = dev(wl["q"]), dev(wl["K"])
    hs = dev(wl["head_scale"])
    K4, ks, kr = ct.ctopk_quantize_k4(K)
    res = ct.ctopk_candidates_k4(q, K, K4, ks, kr, dev(np.asarray(T, dtype=np.float32)),
                                 head_scale=hs, want_bounds=want_bounds)
    ref = ct.ctopk_certify_ex(q, K, dev(wl["V"]), 0.01, head_scale=hs, want_scores=True,
                              want_mask=True)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in res.items()}, {k: v.cpu().numpy() for k, v in ref.items()}


def check_candidates(ct, wl, T, label):
    n, n_q, n_kv, d = wl["n"], wl["n_q_heads"], wl["n_kv_heads"], wl["d"]
    _say(f"candidates {label} n={n} Hq={n_q} Hkv={n_kv} d={d}")
    g, ref = run_k4(ct, wl, T)
    s_dev = ref["scores"]
    mask = unpack_mask(g["sel_mask"], n)
    T = np.asarray(T, dtype=np.float32)
    want = s_dev >= T[:, None]
    assert np.array_equal(mask, want), f"{label}: candidate set differs from the fp32 threshold"
    assert np.array_equal(g["count"], want.sum(axis=1))
    lo, hi = g["bounds"][..., 0], g["bounds"][..., 1]
    assert np.all(lo <= s_dev) and np.all(s_dev <= hi), "an interval misses the device score"
    G = n_q // n_kv
    q64, K64 = oracle.as_f64(wl["q"]), oracle.as_f64(wl["K"])
    sc = np.asarray(wl["head_scale"], dtype=np.float32).astype(np.float64)
    S = np.stack([sc[h] * (K64[h // G] @ q64[h]) for h in range(n_q)])
    assert np.all(lo <= S) and np.all(S <= hi), "an interval misses the exact score"
    # the oracle's candidate set, up to keys within the fp32 rounding band of T
    band = 4 * d * 2.0 ** -24 * np.abs(sc)[:, None] * np.max(np.abs(K64), axis=(1, 2)).repeat(G)[:, None] \
        * np.abs(q64).sum(axis=1)[:, None]
    diff = mask != (S >= T[:, None].astype(np.float64))
    assert np.all(np.abs(S - T[:, None])[diff] <= band.repeat(n, axis=1)[diff])
    groups = -(-G // 8) if G > 8 else 1
    assert np.all(g["rescored"] <= n * groups)
    frac = g["rescored"].sum() / (n * n_kv * groups)
    print(f"{label}: candidates/n {want.mean():.4f}, rescored fraction {frac:.4f}, "
          f"fp64 disagreements {int(diff.sum())}", flush=True)
    return g, ref


def quantile_thresholds(ct, wl, qs):
    _, ref = run_k4(ct, wl, np.zeros(wl["n_q_heads"], dtype=np.float32), want_bounds=False)
    s = ref["scores"]
    return np.array([np.quantile(s[h], qs[h % len(qs)]) for h in range(s.shape[0])], dtype=np.float32)


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_candidates_groups(ct, G):
    wl = workloads.gqa_decode(n=5000, n_q=2 * G, n_kv=2, planted=4, temp_range=(0.5, 4.0))
    T = quantile_thresholds(ct, wl, [0.5, 0.9, 0.99, 0.999])
    check_candidates(ct, wl, T, f"G={G}")


@pytest.mark.parametrize("d", [64, 128])
def test_candidates_fp32(ct, d):
    wl = as_f32(workloads.gqa_decode(n=3001, n_q=8, n_kv=2, d=d, planted=3, temp_range=(0.5, 2.0)))
    T = quantile_thresholds(ct, wl, [0.2, 0.95])
    check_candidates(ct, wl, T, f"fp32 d={d}")


@pytest.mark.parametrize("n", [1, 63, 64, 65, 1000])
def test_candidates_ragged(ct, n):
    wl = workloads.gqa_decode(n=n, n_q=8, n_kv=2)
    T = quantile_thresholds(ct, wl, [0.0, 0.5, 0.9])
    check_candidates(ct, wl, T, f"ragged n={n}")


def test_candidates_extreme_thresholds(ct):
    wl = workloads.gqa_decode(n=2000, n_q=4, n_kv=1)
    T = np.array([-np.inf, np.inf, -1e30, 1e30], dtype=np.float32)
    g, _ = check_candidates(ct, wl, T, "extreme thresholds")
    assert list(g["count"]) == [2000, 0, 2000, 0]
    assert g["rescored"][0] == 0  # every interval is settled


def test_candidates_are_the_certified_head(ct):
    # with each head's cut score as its threshold the candidates are the head
    # of the exact certified truncation (rows without ties at the cut)
    wl = workloads.gqa_decode()
    _say("candidates = certified head, gqa_decode n=32768")
    q, K = dev(wl["q"]), dev(wl["K"])
    ref = ct.ctopk_certify_ex(q, K, dev(wl["V"]), 0.01, want_scores=True, want_mask=True)
    torch.cuda.synchronize()
    s = ref["scores"].cpu().numpy()
    head = unpack_mask(ref["sel_mask"].cpu().numpy(), wl["n"])
    T = np.array([s[h][head[h]].min() for h in range(s.shape[0])], dtype=np.float32)
    K4, ks, kr = ct.ctopk_quantize_k4(K)
    g = ct.ctopk_candidates_k4(q, K, K4, ks, kr, dev(T))
    torch.cuda.synchronize()
    mask = unpack_mask(g["sel_mask"].cpu().numpy(), wl["n"])
    rows = [h for h in range(s.shape[0]) if (s[h] == T[h]).sum() == 1]
    assert len(rows) >= s.shape[0] - 2
    for h in rows:
        assert np.array_equal(mask[h], head[h])
    assert np.array_equal(g["count"].cpu().numpy()[rows], ref["k_eps"].cpu().numpy()[rows])
    print(f"rescored fraction {g['rescored'].cpu().numpy().sum() / (8 * wl['n']):.3f}", flush=True)


def test_candidates_caller_workspace_and_repeat(ct):
    wl = workloads.gqa_decode(n=4097, n_q=8, n_kv=2)
    _say("candidates caller workspace")
    q, K = dev(wl["q"]), dev(wl["K"])
    K4, ks, kr = ct.ctopk_quantize_k4(K)
    T = dev(np.full(8, 0.5, dtype=np.float32))
    ws = torch.empty(ct.ctopk_k4_workspace_bytes(4097, 8, 2) + 256, dtype=torch.uint8, device="cuda")
    off = (-ws.data_ptr()) % 256
    ws = ws[off:off + ct.ctopk_k4_workspace_bytes(4097, 8, 2)]
    a = ct.ctopk_candidates_k4(q, K, K4, ks, kr, T, workspace=ws)
    b = ct.ctopk_candidates_k4(q, K, K4, ks, kr, T)
    torch.cuda.synchronize()
    assert torch.equal(a["sel_mask"], b["sel_mask"]) and torch.equal(a["count"], b["count"])


def test_candidates_are_deterministic(ct):
    wl = workloads.gqa_decode(n=9000, n_q=16, n_kv=2)
    _say("candidates determinism n=9000")
    q, K = dev(wl["q"]), dev(wl["K"])
    K4, ks, kr = ct.ctopk_quantize_k4(K)
    K4b, ksb, krb = ct.ctopk_quantize_k4(K)
    T = dev(np.linspace(-1.0, 2.0, 16).astype(np.float32))
    a = ct.ctopk_candidates_k4(q, K, K4, ks, kr, T, want_bounds=True)
    b = ct.ctopk_candidates_k4(q, K, K4b, ksb, krb, T, want_bounds=True)
    torch.cuda.synchronize()
    assert torch.equal(K4, K4b) and torch.equal(ks, ksb) and torch.equal(kr, krb)
    for key in ("sel_mask", "count", "rescored", "bounds"):
        assert torch.equal(a[key], b[key]), key
