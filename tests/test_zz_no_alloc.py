"""ctopk_certify_noalloc (the entry point that allocates nothing) through the
C ABI: two calls in a row on one GPU, the second on a smaller input, each
against ctopk_certify on the same inputs; and the size limit."""
import ctypes
import sys

import numpy as np
import pytest

import workloads
from parity import OUT_RTOL_BF16, TAU_ATOL, rel_l2

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import certified_top_sparse_amd as ct
    return ct.load()


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()


def _outputs(n_q, d):
    return (torch.full((n_q, d), float("nan"), dtype=torch.float32, device="cuda"),
            torch.full((n_q,), -1, dtype=torch.int32, device="cuda"),
            torch.full((n_q,), float("nan"), dtype=torch.float64, device="cuda"))


def _call(fn, q, K, V, eps, outs):
    vp = ctypes.c_void_p
    n_q, d = q.shape
    n_kv, n, _ = K.shape
    stream = vp(torch.cuda.current_stream().cuda_stream)
    out, k, tau = outs
    rc = fn(vp(q.data_ptr()), vp(K.data_ptr()), vp(V.data_ptr()), n, d, n_q, n_kv, float(eps),
            stream, vp(out.data_ptr()), vp(k.data_ptr()), vp(tau.data_ptr()))
    return rc


def test_noalloc_matches_certify_twice(lib):
    cases = [("gqa_decode n=32768 32/8 heads", workloads.gqa_decode(), 0.01),
             ("gqa_decode n=5000 8/2 heads", workloads.gqa_decode(n=5000, n_q=8, n_kv=2), 0.1)]
    for label, wl, eps in cases:
        _say(f"no-alloc vs certify: {label} eps={eps}")
        q, K, V = _dev(wl["q"]), _dev(wl["K"]), _dev(wl["V"])
        n_q, d = q.shape
        a, b = _outputs(n_q, d), _outputs(n_q, d)
        assert _call(lib.ctopk_certify_noalloc, q, K, V, eps, a) == 0
        assert _call(lib.ctopk_certify, q, K, V, eps, b) == 0
        torch.cuda.synchronize()
        ka, kb = a[1].cpu().numpy(), b[1].cpu().numpy()
        assert np.array_equal(ka, kb), (ka, kb)
        assert np.abs(a[2].cpu().numpy() - b[2].cpu().numpy()).max() <= TAU_ATOL
        err = rel_l2(a[0].cpu().numpy(), b[0].cpu().numpy())
        assert err.max() <= OUT_RTOL_BF16, err.max()
        print(f"{label}: k equal, max |dtau| "
              f"{np.abs(a[2].cpu().numpy() - b[2].cpu().numpy()).max():.2e}, max rel L2 {err.max():.2e}",
              flush=True)


def test_noalloc_rejects_sizes_beyond_its_array(lib):
    import certified_top_sparse_amd as ct
    from certified_top_sparse_amd import ctopk as cb
    n_q, n_kv, n, d = 128, 32, 131072, 128
    assert ct.ctopk_workspace_bytes(n, d, n_q, n_kv) > ct.CTOPK_NOALLOC_SCRATCH_BYTES
    _say("no-alloc size limit (host-side rejection)")
    fake = 1 << 20  # never dereferenced: the call returns before any HIP call
    vp = ctypes.c_void_p
    rc = lib.ctopk_certify_noalloc(vp(fake), vp(fake), vp(fake), n, d, n_q, n_kv, 0.01, None,
                                   vp(fake), vp(fake), vp(fake))
    assert rc == cb.CTOPK_ERR_WORKSPACE
    assert "scratch" in ct.ctopk_last_error_string()
