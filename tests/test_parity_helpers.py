"""CPU checks of the comparison helpers the device tests rely on: the
sort-free minimality check accepts the oracle's own answers and rejects each
kind of wrong answer (a non-minimal k, a head that is not a top set, a wrong
tau, a wrong tie order, an output off its head)."""
import numpy as np
import pytest

import oracle
from parity import check_topk_properties


def _case(seed, R=16, n=3000, sigma=2.0, eps=0.01, ties=False):
    rng = np.random.default_rng(seed)
    S = (rng.standard_normal((R, n)) * sigma).astype(np.float32).astype(np.float64)
    if ties:
        S = np.round(S * 2.0) / 2.0
    V = rng.standard_normal((1, n, 8))
    ref = oracle.certify_scores(S, V, eps)
    gpu = {"k_eps": ref["k_eps"].copy(), "tau": ref["tau"].copy(),
           "sel_mask": ref["head_mask"].copy(), "out": ref["out"].copy()}
    return S, V, gpu, eps


@pytest.mark.parametrize("ties", [False, True])
@pytest.mark.parametrize("eps", [0.001, 0.01, 0.3])
def test_accepts_the_oracle(ties, eps):
    S, V, gpu, eps = _case(1, eps=eps, ties=ties)
    rep = check_topk_properties(gpu, S, eps, V64=V, out_rtol=1e-10)
    assert rep["rows"] == S.shape[0]


def _order(S, r):
    return np.lexsort((np.arange(S.shape[1]), -S[r]))


def test_rejects_a_larger_k():
    S, V, gpu, eps = _case(2)
    o = _order(S, 3)
    gpu["sel_mask"][3, o[gpu["k_eps"][3]]] = True  # one key too many
    gpu["k_eps"][3] += 1
    with pytest.raises(AssertionError, match="minimal"):
        check_topk_properties(gpu, S, eps)


def test_rejects_a_smaller_k():
    S, V, gpu, eps = _case(3)
    o = _order(S, 5)
    gpu["sel_mask"][5, o[gpu["k_eps"][5] - 1]] = False
    gpu["k_eps"][5] -= 1
    with pytest.raises(AssertionError, match="minimal"):
        check_topk_properties(gpu, S, eps)


def test_rejects_a_head_that_is_not_a_top_set():
    S, V, gpu, eps = _case(4)
    o = _order(S, 7)
    k = gpu["k_eps"][7]
    gpu["sel_mask"][7, o[k - 1]] = False    # swap the last kept key
    gpu["sel_mask"][7, o[k + 5]] = True     # for a lower one
    with pytest.raises(AssertionError, match="top set"):
        check_topk_properties(gpu, S, eps)


def test_rejects_the_wrong_tie_order():
    # equal scores: the lower index must be kept first
    n = 100
    S = np.zeros((1, n))
    V = np.ones((1, n, 2))
    ref = oracle.certify_scores(S, V, 0.25)
    gpu = {"k_eps": ref["k_eps"].copy(), "tau": ref["tau"].copy(),
           "sel_mask": ref["head_mask"][:, ::-1].copy()}  # the highest indices instead
    with pytest.raises(AssertionError, match="top set"):
        check_topk_properties(gpu, S, 0.25)


def test_rejects_a_wrong_tau_and_output():
    S, V, gpu, eps = _case(5)
    bad = dict(gpu, tau=gpu["tau"] + 2e-5)
    with pytest.raises(AssertionError, match="tau"):
        check_topk_properties(bad, S, eps)
    out = gpu["out"].copy()
    out[2] *= 1.01
    with pytest.raises(AssertionError, match="out"):
        check_topk_properties(dict(gpu, out=out), S, eps, V64=V, out_rtol=1e-5)


def test_near_boundary_rows_are_counted():
    # equal scores with n * eps integral: T_k equals eps, either k is accepted
    n, eps = 100, 0.25
    S = np.zeros((1, n))
    for k in (75, 76):
        mask = np.zeros((1, n), dtype=bool)
        mask[0, :k] = True
        gpu = {"k_eps": np.array([k]), "tau": np.array([(n - k) / n]), "sel_mask": mask}
        rep = check_topk_properties(gpu, S, eps)
        assert rep["near_boundary"] == 1
