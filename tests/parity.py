"""Comparison protocol between the device path and the fp64 oracle.

* k_eps must match exactly, except on rows the oracle flags near-boundary (its
  tail mass within 1e-6 * eps of eps at k_eps or k_eps - 1); such mismatches
  are counted and reported.
* tau must match to 1e-5 absolute on every row whose k_eps matches.
* out must match per row to a relative L2 tolerance (2e-3 for bf16 inputs,
  1e-5 for fp32).  A row whose device head set differs from the oracle's
  (fp32 scores can swap keys whose fp64 scores differ by rounding) passes if
  every key in the symmetric difference scores within the fp32 rounding band
  of the cut score and the oracle's output recomputed on the device's head set
  matches; such rows are counted.
"""
from __future__ import annotations

import numpy as np

TAU_ATOL = 1e-5
OUT_RTOL_BF16 = 2e-3
OUT_RTOL_F32 = 1e-5


def unpack_mask(words: np.ndarray, n: int) -> np.ndarray:
    w = np.ascontiguousarray(words.astype(np.int32)).view(np.uint8)
    bits = np.unpackbits(w.reshape(words.shape[0], -1), axis=1, bitorder="little")
    return bits[:, :n].astype(bool)


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b, axis=-1)
    num = np.linalg.norm(a - b, axis=-1)
    return num / np.maximum(den, 1e-300)


def compare(gpu: dict, ref: dict, S: np.ndarray, V64: np.ndarray, row_to_v: np.ndarray,
            eps: float, out_rtol: float, rows=None, score_band=None, label=""):
    """Check device results against the oracle on the given rows.

    gpu: numpy arrays k_eps, tau, out and optionally sel_mask (bool [R, n]) for
    all rows; ref: oracle dict for the same rows (in `rows` order); S: oracle
    fp64 scores of those rows; V64: fp64 values [Hv, n, dv]; score_band: per
    row tolerance on scores for the tie adjudication.
    """
    if rows is None:
        rows = np.arange(len(ref["k_eps"]))
    rows = np.asarray(rows)
    kg = gpu["k_eps"][rows].astype(np.int64)
    kr = ref["k_eps"].astype(np.int64)
    near = ref["near_boundary"]
    kmis = kg != kr
    bad_k = kmis & ~near
    report = {"label": label, "rows": int(len(rows)), "k_mismatch_near_boundary": int((kmis & near).sum()),
              "set_adjudicated": 0}
    assert not bad_k.any(), (
        f"{label}: k_eps mismatch on rows {rows[bad_k][:10]}: gpu {kg[bad_k][:10]} ref {kr[bad_k][:10]}")
    tg = gpu["tau"][rows]
    tdiff = np.abs(tg - ref["tau"])
    okrow = ~kmis
    assert (tdiff[okrow] <= TAU_ATOL).all(), (
        f"{label}: tau off by {tdiff[okrow].max():.3e}")
    report["tau_max_abs_err"] = float(tdiff[okrow].max()) if okrow.any() else 0.0
    og = gpu["out"][rows]
    err = rel_l2(og, ref["out"])
    report["out_max_rel_l2"] = float(err[okrow].max()) if okrow.any() else 0.0
    badout = okrow & (err > out_rtol)
    for j in np.nonzero(badout)[0]:
        assert "sel_mask" in gpu, f"{label}: out rel L2 {err[j]:.3e} on row {rows[j]} (no mask to adjudicate)"
        hg = gpu["sel_mask"][rows[j]]
        hr = ref["head_mask"][j]
        diff = hg ^ hr
        assert diff.any(), f"{label}: out rel L2 {err[j]:.3e} on row {rows[j]} with identical head sets"
        band = score_band[j] if score_band is not None else 0.0
        s = S[j]
        assert np.all(np.abs(s[diff] - ref["s_star"][j]) <= band), (
            f"{label}: head sets differ away from the cut on row {rows[j]}")
        w = np.exp(s - s.max()) * hg
        o2 = (w @ V64[row_to_v[rows[j]]]) / w.sum()
        e2 = rel_l2(og[j], o2)
        assert e2 <= out_rtol, f"{label}: out rel L2 {e2:.3e} on row {rows[j]} even on the device head set"
        report["set_adjudicated"] += 1
    if "sel_mask" in gpu:
        hg = gpu["sel_mask"][rows]
        assert (hg.sum(1) == kg).all(), f"{label}: mask popcount differs from k_eps"
    return report


def score_band(q64: np.ndarray, K64: np.ndarray, scale: float, d: int) -> float:
    """Bound on |s_fp32 - s_fp64| over the keys of one query head for the
    device's fp32 dot product: 4 * d * 2^-24 * |scale| * max_i sum_j |q_j k_ij|
    (a loose Higham-style bound)."""
    mag = np.abs(K64) @ np.abs(q64)
    return float(4.0 * d * 2.0 ** -24 * abs(scale) * mag.max())


def check_topk_properties(gpu: dict, S: np.ndarray, eps: float, V64=None, row_to_v=None,
                          out_rtol=None, label=""):
    """Sort-free check, on every row of S (fp64 scores that the device used
    exactly, e.g. given fp32 logits), that the device's (k_eps, tau, sel_mask)
    is the certified minimal Top-k: the mask holds k_eps keys and is a top set
    in the order (score descending, index ascending among equal scores); its
    dropped mass T equals tau to TAU_ATOL and is <= eps; putting back the last
    kept key would exceed eps (T + P_last > eps), so no smaller k qualifies.
    These three facts determine k_eps and the head uniquely, so they are the
    definition restated without a sort.  Rows within 1e-6 eps of the boundary
    on either side are counted, not failed.  With V64, out must equal the
    renormalised output over the device's own head to out_rtol.  Returns a
    report dict."""
    S = np.asarray(S, dtype=np.float64)
    R, n = S.shape
    k = np.asarray(gpu["k_eps"]).astype(np.int64)
    mask = np.asarray(gpu["sel_mask"], dtype=bool)
    assert mask.shape == (R, n), (mask.shape, S.shape)
    assert (mask.sum(1) == k).all(), f"{label}: mask popcount differs from k_eps"
    assert (k >= 1).all() and (k <= n).all(), f"{label}: k_eps out of range"
    m = S.max(1, keepdims=True)
    w = np.exp(S - m)
    Z = w.sum(1)
    T = np.where(mask, 0.0, w).sum(1) / Z
    smin = np.where(mask, S, np.inf).min(1)
    dmax = np.where(mask, -np.inf, S).max(1)
    idx = np.arange(n)[None, :]
    at_min = S == smin[:, None]
    kept_tie_last = np.where(mask & at_min, idx, -1).max(1)
    drop_tie_first = np.where(~mask & at_min, idx, n).min(1)
    top = (dmax < smin) | ((dmax == smin) & (drop_tie_first > kept_tie_last))
    assert top.all(), f"{label}: device head is not a top set on rows {np.nonzero(~top)[0][:10]}"
    T_prev = T + np.exp(smin - m[:, 0]) / Z
    band = 1e-6 * eps
    near = (np.abs(T - eps) <= band) | (np.abs(T_prev - eps) <= band)
    bad = ~near & ~((T <= eps) & (T_prev > eps))
    assert not bad.any(), (
        f"{label}: not the minimal certified k on rows {np.nonzero(bad)[0][:10]}: "
        f"T={T[bad][:5]} T_prev={T_prev[bad][:5]}")
    tdiff = np.abs(np.asarray(gpu["tau"], dtype=np.float64) - T)
    assert (tdiff <= TAU_ATOL).all(), f"{label}: tau off by {tdiff.max():.3e}"
    rep = {"label": label, "rows": int(R), "near_boundary": int(near.sum()),
           "tau_max_abs_err": float(tdiff.max())}
    if V64 is not None:
        if row_to_v is None:
            row_to_v = np.zeros(R, dtype=np.int64)
        wh = np.where(mask, w, 0.0)
        o = np.empty((R, V64.shape[-1]))
        for g in np.unique(row_to_v):
            sel = row_to_v == g
            o[sel] = wh[sel] @ V64[g]
        o /= wh.sum(1)[:, None]
        err = rel_l2(gpu["out"], o)
        assert (err <= out_rtol).all(), f"{label}: out rel L2 {err.max():.3e} on its own head"
        rep["out_max_rel_l2_own_head"] = float(err.max())
    return rep
