"""Pins of the fp64 oracle to what the Abstract of "A Mathematical Theory of
Top-k Sparse Attention via Total Variation Distance" (arXiv 2512.07647) and
plain mathematics fix.  CPU only.

Each test checks the oracle against something other than itself:
* hand-derived closed forms (tests/golden/closed_forms.json);
* the definition of total variation as a supremum over events (brute force);
* the TV-KL identity, the head-tail factorisation and the diameter bound;
* exhaustive search over all key subsets for the minimal certified k;
* library routines (scipy's softmax) in the special case k = n;
* the Gaussian-score closed forms and design rule.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _frac(x):
    return float(Fraction(x[0], x[1]))


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_golden_closed_forms(case):
    s = np.log(np.array(case["log_weights"], dtype=np.float64))
    V = np.array(case["V"], dtype=np.float64)[None]
    r = oracle.certify_scores(s[None], V, case["eps"])
    assert int(r["k_eps"][0]) == case["k_eps"]
    assert abs(r["tau"][0] - _frac(case["tau"])) < 1e-14
    assert sorted(np.nonzero(r["head_mask"][0])[0].tolist()) == case["head"]
    out = np.array([_frac(x) for x in case["out"]])
    np.testing.assert_allclose(r["out"][0], out, rtol=0, atol=1e-14)
    assert not r["near_boundary"][0]
    if "attn" in case:
        attn = np.array([_frac(x) for x in case["attn"]])
        P = oracle.softmax(s)
        np.testing.assert_allclose(P @ V[0], attn, atol=1e-14)
        Ph = oracle.truncation(P, r["head_mask"][0])
        assert abs(oracle.kl(Ph, P) - (-math.log(7 / 8))) < 1e-14
        assert abs(oracle.diam_head_tail(V[0], r["head_mask"][0]) ** 2 - case["diam_sq"]) < 1e-12


def _random_rows(rng, count, n, sigma):
    return sigma * rng.standard_normal((count, n))


@pytest.mark.parametrize("n,sigma,eps", [(64, 1.0, 0.01), (257, 3.0, 0.1), (1000, 2.0, 0.001),
                                         (512, 8.0, 0.01), (33, 0.1, 0.3)])
def test_tv_is_tail_mass_and_kl_identity(n, sigma, eps):
    rng = np.random.default_rng(7 + n)
    S = _random_rows(rng, 6, n, sigma)
    V = rng.standard_normal((1, n, 5))
    r = oracle.certify_scores(S, V, eps)
    for i in range(S.shape[0]):
        P = oracle.softmax(S[i])
        head = r["head_mask"][i]
        Ph = oracle.truncation(P, head)
        tv = oracle.tv_half_l1(P, Ph)
        assert abs(tv - r["tau"][i]) < 1e-12
        assert r["tau"][i] <= eps
        kl = oracle.kl(Ph, P)
        assert abs(-math.expm1(-kl) - r["tau"][i]) < 1e-12
        assert int(head.sum()) == int(r["k_eps"][i])


def test_tv_matches_supremum_over_events():
    rng = np.random.default_rng(11)
    for n in (3, 6, 9, 11):
        for eps in (0.05, 0.3):
            s = 2.0 * rng.standard_normal(n)
            r = oracle.certify_scores(s[None], rng.standard_normal((1, n, 2)), eps)
            P = oracle.softmax(s)
            Ph = oracle.truncation(P, r["head_mask"][0])
            assert abs(oracle.tv_sup_events(P, Ph) - r["tau"][0]) < 1e-12


@pytest.mark.parametrize("n,sigma,eps,dv", [(128, 1.0, 0.01, 16), (300, 4.0, 0.1, 8),
                                            (50, 0.5, 0.2, 3)])
def test_head_tail_factorisation_and_diameter_bound(n, sigma, eps, dv):
    rng = np.random.default_rng(100 + n)
    S = _random_rows(rng, 5, n, sigma)
    V = rng.standard_normal((1, n, dv))
    r = oracle.certify_scores(S, V, eps)
    for i in range(S.shape[0]):
        head = r["head_mask"][i]
        attn = sp_softmax(S[i]) @ V[0]          # library softmax, not the oracle's
        err = attn - r["out"][i]
        P = oracle.softmax(S[i])
        mu_h, mu_t = oracle.head_tail_means(P, V[0], head)
        np.testing.assert_allclose(mu_h, r["out"][i], rtol=1e-12, atol=1e-13)
        fac = r["tau"][i] * (mu_t - mu_h)
        np.testing.assert_allclose(err, fac, rtol=1e-9, atol=1e-14)
        ne = np.linalg.norm(err)
        assert abs(ne - r["tau"][i] * np.linalg.norm(mu_t - mu_h)) <= 1e-10 * max(ne, 1e-300)
        # the oracle's dense output and output error against the library softmax
        np.testing.assert_allclose(r["out_dense"][i], attn, rtol=1e-10, atol=1e-14)
        assert abs(r["out_err"][i] - ne) <= 1e-9 * max(ne, 1e-300) + 1e-15
        assert ne <= r["tau"][i] * oracle.diam_head_tail(V[0], head) * (1 + 1e-12)


def _subset_masses(P):
    n = P.shape[0]
    masks = np.arange(1 << n, dtype=np.int64)
    bits = ((masks[:, None] >> np.arange(n)) & 1).astype(np.float64)
    return masks, bits @ P, bits.sum(1).astype(np.int64)


@pytest.mark.parametrize("seed", range(40))
def test_bruteforce_minimal_k_and_topk_optimality(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 17))
    sigma = float(rng.choice([0.3, 1.0, 2.0, 5.0]))
    eps = float(rng.choice([0.001, 0.01, 0.05, 0.2, 0.5]))
    s = sigma * rng.standard_normal(n)
    r = oracle.certify_scores(s[None], rng.standard_normal((1, n, 3)), eps)
    P = oracle.softmax(s)
    masks, kept, sizes = _subset_masses(P)
    dropped = 1.0 - kept
    k_brute = None
    for k in range(1, n + 1):
        sel = sizes == k
        if dropped[sel].min() <= eps + 1e-15:
            k_brute = k
            best = masks[sel][np.argmin(dropped[sel])]
            break
    assert k_brute == int(r["k_eps"][0])
    head_bits = sum(1 << int(i) for i in np.nonzero(r["head_mask"][0])[0])
    assert head_bits == int(best)


def test_equal_scores_closed_form():
    n, eps = 1000, 0.0123
    s = np.zeros((1, n))
    rng = np.random.default_rng(3)
    V = rng.standard_normal((1, n, 4))
    r = oracle.certify_scores(s, V, eps)
    k = math.ceil(n * (1 - eps))   # T_k = (n - k)/n <= eps
    assert int(r["k_eps"][0]) == k
    assert abs(r["tau"][0] - (n - k) / n) < 1e-12
    np.testing.assert_allclose(r["out"][0], V[0, :k].mean(0), rtol=1e-12, atol=1e-13)
    assert r["head_mask"][0, :k].all() and not r["head_mask"][0, k:].any()


def test_equal_scores_exact_boundary_is_flagged():
    n, eps = 100, 0.25           # T_75 = 25/100 = eps up to rounding
    r = oracle.certify_scores(np.zeros((1, n)), np.ones((1, n, 2)), eps)
    assert r["near_boundary"][0]
    assert int(r["k_eps"][0]) in (75, 76)


def _scores_from_probs(p):
    # scores whose softmax is p (up to rounding of log and exp, ~1e-16)
    return np.log(np.asarray(p, dtype=np.float64))[None]


def test_near_boundary_flag_from_the_previous_tail_only():
    # P = (3/4 - d, 1/4 + d, ...) with eps = 1/4: T_1 = 1/4 + d > eps, so k_eps = 2,
    # and T_2 = 0.05 is far from eps; only T_{k_eps - 1} lies within 1e-6 eps
    # of eps, so the flag must come from that side (an index slip that reads
    # T_{k_eps} or T_{k_eps + 1} there leaves the row unflagged)
    d = 1e-8
    eps = 0.25
    r = oracle.certify_scores(_scores_from_probs([0.75 - d, 0.2 + d, 0.03, 0.02]),
                              np.ones((1, 4, 1)), eps)
    assert int(r["k_eps"][0]) == 2
    assert abs(r["tau"][0] - 0.05) < 1e-14
    assert abs(r["T_prev"][0] - (0.25 + d)) < 1e-14
    assert r["near_boundary"][0]


def test_near_boundary_flag_from_the_certified_tail_only():
    # T_1 = 1/4 - d <= eps = 1/4 gives k_eps = 1 with tau within 1e-6 eps of eps,
    # while T_0 = 1 is far away
    d = 1e-8
    r = oracle.certify_scores(_scores_from_probs([0.75 + d, 0.2 - d, 0.03, 0.02]),
                              np.ones((1, 4, 1)), 0.25)
    assert int(r["k_eps"][0]) == 1
    assert abs(r["T_prev"][0] - 1.0) < 1e-14
    assert r["near_boundary"][0]


def test_rows_away_from_the_boundary_are_not_flagged():
    # T_1 = 0.3 and T_2 = 0.1 around eps = 0.25: both sides far from eps
    r = oracle.certify_scores(_scores_from_probs([0.7, 0.2, 0.06, 0.04]), np.ones((1, 4, 1)), 0.25)
    assert int(r["k_eps"][0]) == 2
    assert abs(r["T_prev"][0] - 0.3) < 1e-14 and abs(r["tau"][0] - 0.1) < 1e-14
    assert not r["near_boundary"][0]
    # a relative gap just above the 1e-6 band on the previous side is not flagged either
    d = 3e-7
    r = oracle.certify_scores(_scores_from_probs([0.75 - d, 0.2 + d, 0.03, 0.02]),
                              np.ones((1, 4, 1)), 0.25)
    assert int(r["k_eps"][0]) == 2 and not r["near_boundary"][0]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_cut_score_of_the_golden_cases(case):
    # s* is the score of the last key the certified head keeps: the smallest
    # weight among the case's hand-derived head, as a log
    w = np.array(case["log_weights"], dtype=np.float64)
    r = oracle.certify_scores(np.log(w)[None], np.array(case["V"], dtype=np.float64)[None],
                              case["eps"])
    assert r["s_star"][0] == math.log(min(w[case["head"]]))


def test_cut_score_two_level_closed_form():
    # m keys at a and n - m at b: the cut score is a while k_eps <= m and b after;
    # eps = 0.44 puts the cut on exactly the m-th key (T_{m-1} > eps >= T_m), where
    # the next key in the order scores b
    n, m, a, b = 200, 13, 2.0, -1.0
    rng = np.random.default_rng(5)
    s = np.full(n, b)
    s[rng.permutation(n)[:m]] = a
    Z = m * math.exp(a) + (n - m) * math.exp(b)
    assert ((n - m) * math.exp(b) / Z <= 0.44 < (math.exp(a) + (n - m) * math.exp(b)) / Z)
    V = np.zeros((1, n, 1))
    for eps, k_cf, s_cf in ((0.44, m, a), (0.6, None, a), (0.3, None, b)):
        r = oracle.certify_scores(s[None], V, eps)
        if k_cf is not None:
            assert int(r["k_eps"][0]) == k_cf
        assert r["s_star"][0] == s_cf


def test_signed_zero_scores_tie():
    s = np.array([[-0.0, 0.0, -0.0, 0.0]])
    r = oracle.certify_scores(s, np.eye(4)[None], 0.3)
    assert int(r["k_eps"][0]) == 3
    assert r["head_mask"][0].tolist() == [True, True, True, False]


def test_two_level_closed_form():
    n, m, a, b = 200, 13, 2.0, -1.0
    rng = np.random.default_rng(5)
    pos = rng.permutation(n)[:m]
    s = np.full(n, b)
    s[pos] = a
    Z = m * math.exp(a) + (n - m) * math.exp(b)
    for eps in (0.001, 0.05, 0.3, 0.6, 0.9):
        def T(k):
            if k <= m:
                return ((m - k) * math.exp(a) + (n - m) * math.exp(b)) / Z
            return (n - k) * math.exp(b) / Z
        k_cf = min(k for k in range(1, n + 1) if T(k) <= eps)
        r = oracle.certify_scores(s[None], rng.standard_normal((1, n, 2)), eps)
        assert int(r["k_eps"][0]) == k_cf
        assert abs(r["tau"][0] - T(k_cf)) < 1e-12
        head = np.nonzero(r["head_mask"][0])[0]
        hi = np.sort(pos)
        lo = np.setdiff1d(np.arange(n), pos)
        expect = np.sort(np.concatenate([hi[:min(k_cf, m)], lo[:max(0, k_cf - m)]]))
        assert head.tolist() == expect.tolist()


def test_one_dominant_key():
    n, a, b = 300, 12.0, 0.0
    s = np.full(n, b)
    s[17] = a
    r = oracle.certify_scores(s[None], np.random.default_rng(1).standard_normal((1, n, 3)), 0.01)
    assert int(r["k_eps"][0]) == 1
    tau = (n - 1) * math.exp(b) / (math.exp(a) + (n - 1) * math.exp(b))
    assert abs(r["tau"][0] - tau) < 1e-15
    assert r["head_mask"][0, 17]


def test_keep_all_reduces_to_dense_attention():
    rng = np.random.default_rng(9)
    n, d = 40, 6
    s = rng.standard_normal(n)
    V = rng.standard_normal((1, n, d))
    P = sp_softmax(s)
    eps = 0.5 * float(P.min())        # every key is needed
    r = oracle.certify_scores(s[None], V, eps)
    assert int(r["k_eps"][0]) == n and r["tau"][0] == 0.0
    np.testing.assert_allclose(r["out"][0], P @ V[0], rtol=1e-12, atol=1e-14)


def test_scores_and_gqa_mapping():
    rng = np.random.default_rng(2)
    n_q, n_kv, n, d = 8, 2, 50, 16
    K = rng.standard_normal((n_kv, n, d)).astype(np.float32)
    V = rng.standard_normal((n_kv, n, d)).astype(np.float32)
    q = np.zeros((n_q, d), dtype=np.float32)
    for h in range(n_q):
        q[h, h] = 1.0                    # q_h = e_h picks column h of K
    scale = np.full(n_q, 0.5, dtype=np.float32)
    r = oracle.certify(q, K, V, 0.1, n_q, n_kv, head_scale=scale)
    for h in range(n_q):
        g = h // (n_q // n_kv)
        np.testing.assert_array_equal(r["S"][h], 0.5 * K[g, :, h].astype(np.float64))
        assert oracle.gqa_kv_head(h, n_q, n_kv) == g


def test_bf16_decode():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F7F, 0x0001, 0x3FC0], dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, 3.3895313892515355e38, 9.183549615799121e-41, 1.5]
    got = oracle.bf16_bits_to_f64(bits)
    assert got.tolist() == want
    assert math.copysign(1.0, got[3]) == -1.0


def test_gaussian_tail_mass_closed_form():
    rng = np.random.default_rng(21)
    n = 2_000_000
    for sigma in (0.5, 1.0, 2.0):
        s = sigma * rng.standard_normal(n)
        w = np.exp(s - s.max())
        for z in (-1.0, 0.0, 1.5):
            frac = w[s <= z * sigma].sum() / w.sum()
            assert abs(frac - oracle.gaussian_tail_fraction(sigma, z)) < 6e-3


@pytest.mark.parametrize("sigma", [1.0, 2.0])
@pytest.mark.parametrize("n", [4096, 65536])
@pytest.mark.parametrize("eps", [0.01, 0.1])
def test_gaussian_design_rule(sigma, n, eps):
    rows = 64 if n == 4096 else 16
    wl = workloads.logit_sweep(sigma, n, rows=rows, dv=2)
    r = oracle.certify_scores(wl["logits"], wl["V"], eps)
    frac = float(np.mean(r["k_eps"] / n))
    pred = oracle.gaussian_design_rule(sigma, eps)
    assert abs(frac - pred) <= 0.005, (frac, pred)


@pytest.mark.parametrize("sigma", [3.0, 4.0])
def test_gaussian_design_rule_gap_closes_with_n(sigma):
    eps = 0.01
    pred = oracle.gaussian_design_rule(sigma, eps)
    gaps = []
    for n, rows in ((4096, 64), (262144, 4)):
        wl = workloads.logit_sweep(sigma, n, rows=rows, dv=2)
        r = oracle.certify_scores(wl["logits"], wl["V"], eps)
        gaps.append(abs(float(np.mean(r["k_eps"] / n)) - pred))
    assert gaps[1] < gaps[0]


def test_design_rule_values():
    # Phi_c(sigma + Phi^{-1}(eps)) evaluated with the error function directly.
    def phi(x):
        return 0.5 * (1.0 + math.erf(x / math.sqrt(2.0)))

    def phi_inv(p):
        lo, hi = -40.0, 40.0
        for _ in range(200):
            mid = 0.5 * (lo + hi)
            if phi(mid) < p:
                lo = mid
            else:
                hi = mid
        return 0.5 * (lo + hi)

    for sigma in (1.0, 2.0, 3.0, 4.0):
        for eps in (0.001, 0.01, 0.1):
            want = 1.0 - phi(sigma + phi_inv(eps))
            assert abs(oracle.gaussian_design_rule(sigma, eps) - want) < 1e-9


def test_eps_outside_open_interval_rejected():
    for eps in (0.0, 1.0, -0.1, 1.5):
        with pytest.raises(ValueError):
            oracle.certify_scores(np.zeros((1, 4)), np.ones((1, 4, 1)), eps)


# ---------------------------------------------------------------------------
# blockwise deterministic bound (Abstract: "blockwise variants")
# ---------------------------------------------------------------------------
def _bound_rows(seed, n, sigma, count=3):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((count, n)) * sigma


@pytest.mark.parametrize("block", [1, 7, 64])
@pytest.mark.parametrize("sigma", [0.5, 2.0, 4.0])
def test_block_bound_dominates_tail_mass(block, sigma):
    # U(t) >= the brute-force mass of the keys below t, at random thresholds
    for s in _bound_rows(11, 700, sigma):
        m = s.max()
        M, sizes = oracle.block_maxima(s, block)
        w = np.exp(s - m)
        for t in np.random.default_rng(1).uniform(s.min() - 1, m + 1, 50):
            assert w[s < t].sum() <= oracle.block_bound(M, sizes, m, t) * (1 + 1e-12) + 1e-300


def test_block_bound_is_monotone():
    s = _bound_rows(12, 900, 2.0, 1)[0]
    M, sizes = oracle.block_maxima(s, 64)
    ts = np.sort(np.concatenate([np.linspace(s.min() - 1, s.max() + 1, 400), M]))
    U = np.array([oracle.block_bound(M, sizes, s.max(), t) for t in ts])
    assert np.all(np.diff(U) >= -1e-12 * U[1:])


@pytest.mark.parametrize("eps", [0.001, 0.01, 0.1, 0.5])
def test_bound_threshold_is_the_largest_feasible(eps):
    # against a dense grid of thresholds: no grid point above t keeps U <= eps Z
    for s in _bound_rows(13, 1500, 2.0):
        t, U, Z, m = oracle.bound_threshold(s, eps)
        assert U <= eps * Z * (1 + 1e-12)
        M, sizes = oracle.block_maxima(s)
        grid = np.linspace(t, s.max() + 1, 3000)[1:]
        feas = [g for g in grid if oracle.block_bound(M, sizes, m, g) <= eps * Z]
        assert not feas or max(feas) - t <= 1e-9 * max(1.0, abs(t))


@pytest.mark.parametrize("eps", [0.01, 0.1])
@pytest.mark.parametrize("sigma", [1.0, 3.0])
def test_bound_certificate_properties(eps, sigma):
    S = _bound_rows(14, 3000, sigma, 4)
    V = np.random.default_rng(2).standard_normal((1, 3000, 8))
    b = oracle.certify_bound(S, V, eps)
    e = oracle.certify_scores(S, V, eps)
    assert np.all(b["tv"] <= b["tau_bound"] * (1 + 1e-12))
    assert np.all(b["tau_bound"] <= eps * (1 + 1e-12))
    assert np.all(b["k"] >= e["k_eps"])  # a valid certificate is never smaller than the minimal one
    for r in range(S.shape[0]):  # H_t is a top set: every kept key outscores every dropped key
        h = b["head_mask"][r]
        if (~h).any():  # the bound may also keep every key
            assert S[r][h].min() > S[r][~h].max()
        assert b["k"][r] == h.sum()


def test_bound_closed_form_equal_scores():
    # all scores equal: every block maximum is 0, Z = n, and on (-inf, 0] the
    # bound is (n - nb) e^t, so t = log(eps n / (n - nb)), every key is kept
    # and the certified bound is exactly eps
    n, eps = 1000, 0.05
    nb = -(-n // 64)
    t, U, Z, m = oracle.bound_threshold(np.zeros(n), eps)
    assert Z == n and m == 0.0
    assert t == pytest.approx(math.log(eps * n / (n - nb)), rel=1e-13)
    assert U / Z == pytest.approx(eps, rel=1e-13)
    b = oracle.certify_bound(np.zeros((1, n)), np.ones((1, n, 2)), eps)
    assert b["k"][0] == n and b["tv"][0] == 0.0


@pytest.mark.parametrize("eps", [0.001, 0.01, 0.2])
def test_bound_with_unit_blocks_is_the_minimal_topk(eps):
    # blocks of one key make the bound exact (U(t) is the mass below t), so the
    # certified head is the minimal Top-k head
    rng = np.random.default_rng(15)
    S = rng.standard_normal((5, 800)) * 2.0
    V = rng.standard_normal((1, 800, 4))
    b = oracle.certify_bound(S, V, eps, block=1)
    e = oracle.certify_scores(S, V, eps)
    assert np.array_equal(b["k"], e["k_eps"])
    assert np.array_equal(b["head_mask"], e["head_mask"])


# ---------------------------------------------------------------------------
# 4-bit key copy and score bounds ("Certified Sparse Attention via Perturbed
# Retrieval", arXiv 2610.24991, Abstract)
# ---------------------------------------------------------------------------
def _bf16_keys(seed, n, d, spread=1.0):
    rng = np.random.default_rng(seed)
    return workloads.bf16_rne(rng.standard_normal((n, d), dtype=np.float32) * np.float32(spread))


def test_k4_reconstruction_error_and_range():
    K = _bf16_keys(40, 2000, 128, 3.0)
    c, a, rho = oracle.quantize_k4(K)
    Kf = oracle.as_f64(K)
    assert c.min() >= -7 and c.max() <= 7
    err = np.abs(Kf - a.astype(np.float64)[:, None] * c)
    assert np.all(err <= a.astype(np.float64)[:, None] * 0.5 * (1 + 1e-6))  # nearest code
    # the largest element of each row maps to the end code
    top = np.argmax(np.abs(Kf), axis=1)
    assert np.all(np.abs(c[np.arange(len(top)), top]) == 7)
    # rho is the residual norm, which the elementwise error bounds
    assert np.all(rho <= np.sqrt(128) * a * 0.5 * (1 + 1e-6))
    assert np.allclose(rho, np.linalg.norm(Kf - a.astype(np.float64)[:, None] * c, axis=1), rtol=1e-12)


def test_k4_pack_layout_and_roundtrip():
    # element 2j in the low nibble of byte j, two's complement
    assert list(oracle.pack_k4(np.array([1, -1, 7, -7], dtype=np.int8))) == [0xF1, 0x97]
    rng = np.random.default_rng(41)
    c = rng.integers(-8, 8, size=(3, 50, 64)).astype(np.int8)
    assert np.array_equal(oracle.unpack_k4(oracle.pack_k4(c), 64), c)


@pytest.mark.parametrize("d", [64, 128])
def test_k4_bounds_contain_every_exact_score(d):
    rng = np.random.default_rng(42 + d)
    K = _bf16_keys(43 + d, 3000, d, 2.0)
    c, a, rho = oracle.quantize_k4(K)
    for r in range(5):
        q = workloads.bf16_rne(rng.standard_normal(d, dtype=np.float32))
        scale = np.float32(rng.uniform(0.05, 0.5))
        s = float(scale) * (oracle.as_f64(K) @ oracle.as_f64(q))
        shat, R = oracle.k4_score_bounds(q, c, a, rho, scale)
        assert np.all(np.abs(s - shat) <= R * (1 + 1e-12) + 1e-12)
        # classification against a threshold agrees with the exact candidate set
        T = float(np.quantile(s, 0.9))
        cand = oracle.candidates(q, K, scale, T)
        assert np.all(cand[shat - R >= T]) and not np.any(cand[shat + R < T])


def test_k4_exact_when_the_residual_vanishes():
    # keys that are integer multiples of a power of two with largest entry 7 units
    rng = np.random.default_rng(44)
    c0 = rng.integers(-7, 8, size=(200, 64)).astype(np.float32)
    c0[:, 0] = 7.0
    K = (c0 * np.float32(0.125)).astype(np.float32)
    c, a, rho = oracle.quantize_k4(K)
    assert np.all(a == np.float32(0.125)) and np.array_equal(c, c0.astype(np.int8))
    assert np.all(rho == 0.0)
    q = rng.standard_normal(64)
    shat, R = oracle.k4_score_bounds(q, c, a, rho, 0.3)
    assert np.all(R == 0.0)
    assert np.allclose(shat, 0.3 * (K.astype(np.float64) @ q), rtol=0, atol=1e-12)
    # a zero row: scale 0, codes 0, no residual
    c, a, rho = oracle.quantize_k4(np.zeros((1, 64), dtype=np.float32))
    assert a[0] == 0 and not c.any() and rho[0] == 0


def test_k4_bound_is_attained_for_a_query_along_the_residual():
    # Cauchy-Schwarz is tight when q is parallel to the residual: |s - shat| = R
    K = _bf16_keys(45, 10, 128)
    c, a, rho = oracle.quantize_k4(K)
    Kf = oracle.as_f64(K)
    for i in range(10):
        e = Kf[i] - float(a[i]) * c[i]
        q = 3.0 * e / np.linalg.norm(e)
        s = 0.2 * (Kf[i] @ q)
        shat, R = oracle.k4_score_bounds(q, c[i:i + 1], a[i:i + 1], rho[i:i + 1], 0.2)
        assert s - shat[0] == pytest.approx(R[0], rel=1e-12)


# ---------------------------------------------------------------------------
# gap bounds and the Var_P(V) refinement (Abstract: deterministic bounds from
# a single boundary gap and from several gaps; refinements of the output
# error by Var_P(V))
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("sigma", [0.5, 2.0, 6.0])
def test_gap_bounds_dominate_the_tail_mass(sigma):
    rng = np.random.default_rng(71)
    n = 40
    for _ in range(5):
        s = rng.standard_normal(n) * sigma
        _, _, _, T = oracle.tail_masses(s)
        for k in range(1, n + 1):
            single = oracle.gap_bound(s, k)
            assert T[k] <= single * (1 + 1e-12) + 1e-300
            if k < n - 1:
                inner = np.sort(rng.choice(np.arange(k + 1, n), size=min(3, n - k - 1),
                                           replace=False))
                multi = oracle.gap_bound(s, k, inner)
                # more gaps never loosen the bound, and it still holds
                assert T[k] <= multi * (1 + 1e-12) + 1e-300
                assert multi <= single * (1 + 1e-12)


def test_single_gap_bound_is_exact_on_two_levels():
    # k keys at a and n - k at b < a: every inequality of the bound is tight,
    # TV = (n - k) e^{b} / (k e^{a} + (n - k) e^{b}).
    n, a, b = 23, 1.25, -0.75
    for k in range(1, n):
        s = np.full(n, b)
        s[np.random.default_rng(k).choice(n, size=k, replace=False)] = a
        exact = (n - k) * math.exp(b) / (k * math.exp(a) + (n - k) * math.exp(b))
        assert abs(oracle.gap_bound(s, k) - exact) <= 1e-15
        _, _, _, T = oracle.tail_masses(s)
        assert abs(T[k] - exact) <= 1e-14


def test_multi_gap_bound_with_every_rank_is_exact_for_one_head_key():
    # k = 1: the head is the top key itself, and with a gap at every rank the
    # bound sums each tail key's exact weight.
    rng = np.random.default_rng(5)
    for n in (2, 7, 31):
        s = rng.standard_normal(n) * 3.0
        _, _, _, T = oracle.tail_masses(s)
        b = oracle.gap_bound(s, 1, list(range(2, n)))
        assert abs(b - T[1]) <= 1e-13 * max(T[1], 1e-300)


def test_gap_bound_closed_form_values():
    # s = (3, 1, 0, 0, -2): k = 2, Delta = s_(2) - s_(3) = 1.
    s = np.array([0.0, 3.0, -2.0, 1.0, 0.0])
    single = 3 * math.exp(-1.0) / (2 + 3 * math.exp(-1.0))
    assert abs(oracle.gap_bound(s, 2) - single) <= 1e-15
    # ranks (2, 4, 5): ranks 3-4 score at most s_(3) = 0, rank 5 at most -2.
    B = 2 * math.exp(-1.0) + math.exp(-3.0)
    assert abs(oracle.gap_bound(s, 2, [4]) - B / (2 + B)) <= 1e-15
    assert oracle.gap_bound(s, 5) == 0.0
    with pytest.raises(ValueError):
        oracle.gap_bound(s, 2, [2])


@pytest.mark.parametrize("sigma,eps", [(1.0, 0.01), (2.5, 0.1), (4.0, 0.3)])
def test_variance_bound_holds(sigma, eps):
    rng = np.random.default_rng(17)
    n, dv = 300, 8
    S = _random_rows(rng, 4, n, sigma)
    V = rng.standard_normal((1, n, dv)) * rng.uniform(0.5, 2.0, size=dv)
    r = oracle.certify_scores(S, V, eps)
    for i in range(S.shape[0]):
        P = sp_softmax(S[i])
        var = oracle.variance_p(P, V[0])
        # Var_P against its definition through a library mean and variance
        mu = np.average(V[0], axis=0, weights=P)
        assert abs(var - float(np.sum(np.average((V[0] - mu) ** 2, axis=0, weights=P)))) \
            <= 1e-12 * var
        assert r["out_err"][i] <= oracle.variance_bound(r["tau"][i], var) * (1 + 1e-12)
        assert abs(r["out_var"][i] - var) <= 1e-11 * var


def test_variance_bound_is_attained_by_two_value_rows():
    # head rows all equal to A and tail rows all equal to B: Var_P(V) is the
    # between-group part tau (1 - tau) ||A - B||^2 alone, so the bound is met
    # with equality: sqrt(tau Var / (1 - tau)) = tau ||A - B|| = ||Attn - Attn_k||.
    rng = np.random.default_rng(3)
    n, dv = 64, 5
    s = rng.standard_normal(n) * 1.5
    r = oracle.certify_scores(s[None], np.zeros((1, n, dv)), 0.1)
    head = r["head_mask"][0]
    A, B = rng.standard_normal(dv), rng.standard_normal(dv)
    V = np.where(head[:, None], A[None, :], B[None, :])
    r = oracle.certify_scores(s[None], V[None], 0.1)
    tau = r["tau"][0]
    var = oracle.variance_p(sp_softmax(s), V)
    assert abs(var - tau * (1 - tau) * float(np.sum((A - B) ** 2))) <= 1e-12 * var
    assert abs(oracle.variance_bound(tau, var) - tau * np.linalg.norm(A - B)) <= 1e-12
    assert abs(r["out_err"][0] - tau * np.linalg.norm(A - B)) <= 1e-12
