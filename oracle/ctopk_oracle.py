"""Plain fp64 CPU oracle for certified Top-k attention truncation.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry point and the
benchmark's CPU-baseline leg may import this module.  The library under
``certified_top_sparse_amd`` never imports it, and this module imports nothing
from the library: the two share no code.

Source of every definition below: "A Mathematical Theory of Top-k Sparse
Attention via Total Variation Distance" (Tzachristas, Deng, Tzachristas,
Zhang, Chen; arXiv 2512.07647), Abstract.  The abstract defines:

* P, the softmax attention distribution of one query over its keys;
* the Top-k truncation P_hat, which keeps the k largest-score keys (the head H)
  and renormalises them, giving zero weight to the tail T;
* TV(P, P_hat), which equals the softmax mass of the discarded tail, and the
  identity TV = 1 - exp(-KL(P_hat || P));
* the head-only output Attn_k, its exact head/tail decomposition with
  tau = TV, and the bound by tau times the head/tail diameter;
* the minimal k_eps with TV <= eps, and its Gaussian-score design rule
  k_eps / n ~ Phi_c(sigma + Phi^{-1}(eps)).

Readings where the page leaves a step open:

* the certificate is inclusive, TV <= eps, and k ranges over 1..n;
* keys are ordered by score descending and, among equal scores, by index
  ascending, so the lower index enters the head first;
* the tail mass is summed directly from the smallest term upward, never as
  1 - head mass;
* diam_{H,T} is the largest Euclidean distance between a head value row and a
  tail value row;
* a row is "near-boundary" when T_{k_eps} or T_{k_eps - 1} lies within
  1e-6 * eps of eps; such rows are reported, not failed, on a k_eps mismatch;
* the blockwise deterministic bound (the Abstract names "blockwise variants"
  of bounds that control TV from the ordered logits, without printing one):
  with the keys cut into consecutive blocks B of `block` keys, block maxima
  M_B and m = max s, the softmax mass of the keys scoring below a threshold t
  is at most U(t) = sum_{M_B < t} |B| e^{M_B - m} + sum_{M_B >= t} (|B| - 1)
  e^{t - m} (a block whose maximum is below t has all its keys below t; any
  other block has at most |B| - 1 keys below t, each of weight below
  e^{t - m}); the certified truncation keeps H_t = {i : s_i >= t} for the
  largest t with U(t) <= eps * Z, so TV(P, P_hat_{H_t}) <= U(t) / Z <= eps.

4-bit key copy and score bounds.  A second page ("Certified Sparse
Attention via Perturbed Retrieval", arXiv 2610.24991: its Abstract, and the
"Limitations and Discussion" figure quoted on the paperfoot.com page)
describes a pass over all keys in a 4-bit form, with a deterministic bound on
each score's error and one pass per grouped-query group, from which the exact
candidate set follows; it gives no formula.  Readings taken:

* each key k_i (a row of d values) gets a scale a_i = amax_i / 7 and codes
  c_ij = clamp(rint(k_ij / a_i), -7, 7), computed in float32 as written (the
  codes are integers, so a copy made elsewhere must match them exactly);
  a_i = 0 and all codes 0 when the row is zero;
* the residual e_i = k_i - a_i c_i is summarised by its Euclidean norm rho_i;
* the score s_i = scale (q . k_i) then lies in
  [shat_i - R_i, shat_i + R_i] with shat_i = scale a_i (q . c_i) and
  R_i = scale ||q||_2 rho_i (Cauchy-Schwarz on q . e_i);
* the candidates for a threshold T are exactly {i : s_i >= T}: keys whose
  interval lies at or above T are in, keys whose interval lies below T are
  out, and only the keys whose interval straddles T need their full score.

Everything is computed in float64.  bf16 and fp32 inputs convert to float64
exactly.  The score scale is applied as the float64 value of the float32 the
device receives.

Parity status: every function here is pinned by the tests in
``tests/test_oracle_pins.py`` (identities, brute force, closed forms, the
Gaussian design rule, the blockwise bound's validity, monotonicity and
optimality, and the 4-bit copy's reconstruction error, interval containment
on every key, and the exact cases where the residual vanishes).  The pages print no worked example, so no specific
(q, K, V) -> (k_eps, tau, out) triple is pinned by a printed value.
"""
from __future__ import annotations

import itertools
import math

import numpy as np

NEAR_BOUNDARY_REL = 1e-6


# ---------------------------------------------------------------------------
# input decoding (the oracle's own; shares nothing with the device path)
# ---------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of bfloat16 bit patterns (uint16 array)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def as_f64(x) -> np.ndarray:
    """float64 view of an input array: uint16 is taken as bf16 bits."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    return x.astype(np.float64)


# ---------------------------------------------------------------------------
# scores
# ---------------------------------------------------------------------------
def scores(q, K, scale) -> np.ndarray:
    """s_i = scale * <q, k_i> for every key row k_i (Abstract: P is the softmax
    of these scores).  q: [d]; K: [n, d]; returns float64 [n]."""
    q64 = as_f64(q)
    K64 = as_f64(K)
    return float(scale) * (K64 @ q64)


def gqa_kv_head(h: int, n_q_heads: int, n_kv_heads: int) -> int:
    """KV head read by query head h: consecutive query heads share a KV head
    (the grouped-query layout the second page's scan shares across)."""
    return h // (n_q_heads // n_kv_heads)


# ---------------------------------------------------------------------------
# certified Top-k on given scores
# ---------------------------------------------------------------------------
def order_desc(s: np.ndarray) -> np.ndarray:
    """Key order: score descending, index ascending among equal scores.
    -0.0 and +0.0 compare equal here, as numpy compares them."""
    s = np.asarray(s, dtype=np.float64)
    idx = np.arange(s.shape[-1])
    idx = np.broadcast_to(idx, s.shape)
    return np.lexsort((idx, -s), axis=-1)


def tail_masses(s: np.ndarray):
    """For scores s [..., n]: returns (order, w, Z, T) where w = exp(s - max),
    Z = sum(w) and T[..., k] is the softmax mass left out when the first k keys
    of ``order`` are kept (k = 0..n).  T is accumulated from the smallest term
    upward (Abstract: TV equals the discarded tail mass)."""
    s = np.asarray(s, dtype=np.float64)
    m = np.max(s, axis=-1, keepdims=True)
    w = np.exp(s - m)
    Z = np.sum(w, axis=-1, keepdims=True)
    P = w / Z
    order = order_desc(s)
    Ps = np.take_along_axis(P, order, axis=-1)
    rev = np.cumsum(Ps[..., ::-1], axis=-1)[..., ::-1]  # rev[k] = sum_{j>=k} Ps[j]
    zeros = np.zeros(s.shape[:-1] + (1,), dtype=np.float64)
    T = np.concatenate([rev, zeros], axis=-1)
    return order, w, Z[..., 0], T


def minimal_k(T: np.ndarray, eps: float) -> np.ndarray:
    """k_eps = min{k in 1..n : T[k] <= eps} (Abstract: the minimal k that keeps
    TV(P, P_hat) <= eps).  T has n+1 entries with T[n] = 0."""
    ok = T[..., 1:] <= eps
    return np.argmax(ok, axis=-1) + 1


def certify_scores(S, V, eps: float, row_to_v=None, with_diagnostics: bool = True):
    """Certified Top-k truncation for every row of the score matrix S.

    S: [R, n] scores; V: [Hv, n, dv] value rows; row r reads V[row_to_v[r]]
    (default: all rows read V[0]).  Returns a dict of float64/int64 arrays:
    k_eps [R], tau [R], out [R, dv], out_dense [R, dv] (untruncated softmax
    output), out_err [R] (= ||out_dense - out||_2), out_var [R] (= Var_P(V)),
    lse [R], T_prev [R] (= T_{k_eps - 1}),
    near_boundary [R] (bool), head_mask [R, n] (bool), and, with diagnostics,
    s_star [R] (score of the last kept key).
    """
    S = np.atleast_2d(np.asarray(S, dtype=np.float64))
    V = as_f64(V)
    if V.ndim == 2:
        V = V[None]
    R, n = S.shape
    if row_to_v is None:
        row_to_v = np.zeros(R, dtype=np.int64)
    row_to_v = np.asarray(row_to_v, dtype=np.int64)
    if not (0.0 < eps < 1.0):
        raise ValueError("eps must lie in (0, 1)")

    order, w, Z, T = tail_masses(S)
    k = minimal_k(T, eps)
    rows = np.arange(R)
    tau = T[rows, k]
    T_prev = T[rows, k - 1]
    near = (np.abs(tau - eps) <= NEAR_BOUNDARY_REL * eps) | (
        np.abs(T_prev - eps) <= NEAR_BOUNDARY_REL * eps)

    rank = np.empty_like(order)
    np.put_along_axis(rank, order, np.broadcast_to(np.arange(n), order.shape), axis=-1)
    head = rank < k[:, None]

    # Attn_k: renormalised head-only output (Abstract).
    wh = np.where(head, w, 0.0)
    num = np.empty((R, V.shape[-1]), dtype=np.float64)
    for g in np.unique(row_to_v):
        sel = row_to_v == g
        num[sel] = wh[sel] @ V[g]
    den = np.sum(wh, axis=-1)
    out = num / den[:, None]

    # Attn: the untruncated softmax output, and the output error of the
    # truncation, ||Attn - Attn_k||_2 (the quantity the Abstract factorises
    # as tau * ||mu_tail - mu_head||_2), here straight from its definition.
    dense = np.empty((R, V.shape[-1]), dtype=np.float64)
    for g in np.unique(row_to_v):
        sel = row_to_v == g
        dense[sel] = w[sel] @ V[g]
    dense /= Z[:, None]
    out_err = np.linalg.norm(dense - out, axis=-1)
    # Var_P(V) = sum_i P_i ||v_i - Attn||^2 (the spread the Abstract's
    # refinement of the output error is stated in; see variance_bound)
    var_p = np.empty(R, dtype=np.float64)
    for g in np.unique(row_to_v):
        sel = np.nonzero(row_to_v == g)[0]
        for r in sel:
            var_p[r] = (w[r] / Z[r]) @ np.sum((V[g] - dense[r]) ** 2, axis=1)

    res = {
        "k_eps": k.astype(np.int64),
        "tau": tau,
        "out": out,
        "out_dense": dense,
        "out_err": out_err,
        "out_var": var_p,
        "lse": np.log(Z) + np.max(S, axis=-1),
        "T_prev": T_prev,
        "near_boundary": near,
        "head_mask": head,
    }
    if with_diagnostics:
        last = np.take_along_axis(order, (k - 1)[:, None], axis=-1)[:, 0]
        res["s_star"] = S[rows, last]
    return res


def certify(q, K, V, eps: float, n_q_heads: int, n_kv_heads: int, head_scale=None):
    """Decode-shaped entry: q [Hq, d], K/V [Hkv, n, d] (float or bf16 bits).

    head_scale: per-query-head float32 scale; default float32(1/sqrt(d)).
    Returns the dict of ``certify_scores`` plus the fp64 scores "S".
    """
    q64 = as_f64(q).reshape(n_q_heads, -1)
    K64 = as_f64(K)
    d = q64.shape[1]
    if head_scale is None:
        head_scale = np.full(n_q_heads, np.float32(1.0 / math.sqrt(d)), dtype=np.float32)
    sc = np.asarray(head_scale, dtype=np.float32).astype(np.float64)
    G = n_q_heads // n_kv_heads
    n = K64.shape[1]
    S = np.empty((n_q_heads, n), dtype=np.float64)
    for g in range(n_kv_heads):
        hs = slice(g * G, (g + 1) * G)
        S[hs] = sc[hs, None] * (q64[hs] @ K64[g].T)
    row_to_v = np.arange(n_q_heads) // G
    res = certify_scores(S, V, eps, row_to_v)
    res["S"] = S
    return res


def certify_logits(logits, V, eps: float, n_v: int = 1):
    """Select-only entry on given logits [rows, n]; row r reads V head
    r // (rows / n_v) of V [n_v, n, dv]."""
    L = np.asarray(logits, dtype=np.float64)
    R = L.shape[0]
    row_to_v = np.arange(R) // (R // n_v)
    return certify_scores(L, V, eps, row_to_v)


# ---------------------------------------------------------------------------
# quantities the Abstract relates to one another (used by the pins)
# ---------------------------------------------------------------------------
def softmax(s) -> np.ndarray:
    s = np.asarray(s, dtype=np.float64)
    w = np.exp(s - np.max(s))
    return w / np.sum(w)


def truncation(P: np.ndarray, head: np.ndarray) -> np.ndarray:
    """P_hat: P restricted to the head and renormalised (Abstract)."""
    Ph = np.where(head, P, 0.0)
    return Ph / np.sum(Ph)


def tv_half_l1(P: np.ndarray, Q: np.ndarray) -> float:
    """Total variation distance as half the L1 distance."""
    return 0.5 * float(np.sum(np.abs(P - Q)))


def tv_sup_events(P: np.ndarray, Q: np.ndarray) -> float:
    """Total variation distance as the largest gap |P(A) - Q(A)| over all
    events A; brute force, so only for tiny supports."""
    n = P.shape[0]
    best = 0.0
    for r in range(n + 1):
        for A in itertools.combinations(range(n), r):
            A = list(A)
            best = max(best, abs(float(P[A].sum() - Q[A].sum())))
    return best


def kl(Q: np.ndarray, P: np.ndarray) -> float:
    """KL(Q || P) over the support of Q."""
    m = Q > 0
    return float(np.sum(Q[m] * np.log(Q[m] / P[m])))


def head_tail_means(P: np.ndarray, V: np.ndarray, head: np.ndarray):
    """mu_head and mu_tail: P-weighted means of the value rows over H and T."""
    V = as_f64(V)
    PH = np.where(head, P, 0.0)
    PT = np.where(head, 0.0, P)
    mu_h = PH @ V / PH.sum()
    mu_t = PT @ V / PT.sum() if PT.sum() > 0 else np.zeros(V.shape[1])
    return mu_h, mu_t


def diam_head_tail(V: np.ndarray, head: np.ndarray) -> float:
    """diam_{H,T}: largest distance between a head value row and a tail value
    row (reading of the Abstract's head-tail diameter)."""
    V = as_f64(V)
    VH = V[head]
    VT = V[~head]
    if VT.shape[0] == 0:
        return 0.0
    d2 = (np.sum(VH * VH, 1)[:, None] + np.sum(VT * VT, 1)[None, :]
          - 2.0 * VH @ VT.T)
    return float(np.sqrt(max(0.0, float(np.max(d2)))))


def variance_p(P: np.ndarray, V: np.ndarray) -> float:
    """Var_P(V) = sum_i P_i ||v_i - Attn||_2^2, the spread of the value rows
    under the attention distribution P (Attn = sum_i P_i v_i)."""
    V = as_f64(V)
    mu = P @ V
    return float(P @ np.sum((V - mu) ** 2, axis=1))


def variance_bound(tau: float, var_p: float) -> float:
    """Refinement of the output error by Var_P(V) (reading of the Abstract's
    "refinements linking the error to Var_P(V)"): Attn is the mixture
    (1 - tau) mu_head + tau mu_tail, so the law of total variance gives
    Var_P(V) >= tau (1 - tau) ||mu_tail - mu_head||^2, and with the
    factorisation ||Attn - Attn_k|| = tau ||mu_tail - mu_head|| this is
    ||Attn - Attn_k||_2 <= sqrt(tau Var_P(V) / (1 - tau)).  Equality holds
    when every head row equals mu_head and every tail row equals mu_tail."""
    if tau <= 0.0:
        return 0.0
    return math.sqrt(tau * var_p / (1.0 - tau))


def gap_bound(s, k: int, ranks=None) -> float:
    """Deterministic bound on TV(P, P_hat) of the Top-k truncation from the
    ordered logits (reading of the Abstract's "single boundary gap" and
    "multi-gap" bounds, whose formulas the page does not print).

    With s_(1) >= ... >= s_(n) the ordered scores, every head key has weight at
    least e^{s_(k)}, and a tail key of rank in (r_j, r_{j+1}] has weight at
    most e^{s_(r_j + 1)}.  For ranks k = r_0 < r_1 < ... < r_J = n and the
    gaps G_j = s_(k) - s_(r_j + 1) >= 0, the tail mass relative to e^{s_(k)}
    is at most B = sum_j (r_{j+1} - r_j) e^{-G_j} and the head's at least k,
    and since x / (a + x) grows with x and falls with a,
        TV <= B / (k + B).
    ranks=None takes the single boundary gap (J = 1, r_1 = n), which reads
    (n - k) e^{-Delta} / (k + (n - k) e^{-Delta}) with Delta = s_(k) - s_(k+1);
    `ranks` lists r_1 < ... < r_{J-1} strictly between k and n for the
    multi-gap bound.  k = n returns 0."""
    s = np.asarray(s, dtype=np.float64)
    n = s.shape[0]
    if not (1 <= k <= n):
        raise ValueError("k must lie in 1..n")
    if k == n:
        return 0.0
    ss = s[order_desc(s)]
    r = [k] + ([] if ranks is None else [int(x) for x in ranks]) + [n]
    if any(b <= a for a, b in zip(r[:-1], r[1:])):
        raise ValueError("ranks must increase strictly between k and n")
    sk = ss[k - 1]
    B = 0.0
    for a, b in zip(r[:-1], r[1:]):
        B += (b - a) * math.exp(ss[a] - sk)  # ss[a] is s_(a + 1)
    return B / (k + B)


def gaussian_design_rule(sigma: float, eps: float) -> float:
    """k_eps / n ~ Phi_c(sigma + Phi^{-1}(eps)) for i.i.d. N(mu, sigma^2)
    scores (Abstract), with Phi_c = 1 - Phi."""
    from scipy.special import ndtr, ndtri
    return float(1.0 - ndtr(sigma + ndtri(eps)))


def gaussian_tail_fraction(sigma: float, z: float) -> float:
    """Closed-form softmax mass below mu + z*sigma for N(mu, sigma^2) scores in
    the large-n limit: E[e^s 1{s <= t}] / E[e^s] = Phi(z - sigma)."""
    from scipy.special import ndtr
    return float(ndtr(z - sigma))


# ---------------------------------------------------------------------------
# blockwise deterministic bound (Abstract: "blockwise variants" of the
# deterministic bounds that control TV from the ordered logits)
# ---------------------------------------------------------------------------
BOUND_BLOCK = 64


def block_maxima(s, block: int = BOUND_BLOCK):
    """Maxima and sizes of the consecutive blocks of `block` keys of one row."""
    s = np.asarray(s, dtype=np.float64)
    n = s.shape[-1]
    nb = -(-n // block)
    M = np.array([s[b * block:(b + 1) * block].max() for b in range(nb)])
    sizes = np.array([min(block, n - b * block) for b in range(nb)], dtype=np.float64)
    return M, sizes


def block_bound(M, sizes, m: float, t: float) -> float:
    """U(t) * e^{-m} scale: sum_{M_B < t} |B| e^{M_B - m} + sum_{M_B >= t} (|B| - 1) e^{t - m},
    an upper bound on the softmax mass (unnormalised, relative to e^m) of the
    keys scoring below t."""
    below = M < t
    return float(np.sum(sizes[below] * np.exp(M[below] - m))
                 + np.sum(sizes[~below] - 1.0) * math.exp(t - m))


def bound_threshold(s, eps: float, block: int = BOUND_BLOCK):
    """The largest t with U(t) <= eps * Z, and U(t).

    U is non-decreasing in t and equal to A_j + c_j e^{t - m} on the interval
    (M_(j-1), M_(j)] between consecutive sorted block maxima (A_j sums
    |B| e^{M_B - m} over the j blocks with the smallest maxima, c_j sums
    |B| - 1 over the others), so the largest feasible t of each interval is
    min(M_(j), m + log((eps Z - A_j) / c_j)); the answer is the one of the
    last interval where that exceeds M_(j-1).  Returns (t, U(t), Z, m)."""
    s = np.asarray(s, dtype=np.float64)
    m = float(s.max())
    Z = float(np.sum(np.exp(s - m)))
    M, sizes = block_maxima(s, block)
    order = np.argsort(M, kind="stable")
    Ms, szs = M[order], sizes[order]
    nb = len(Ms)
    A = np.concatenate([[0.0], np.cumsum(szs * np.exp(Ms - m))])
    c = np.concatenate([np.cumsum((szs - 1.0)[::-1])[::-1], [0.0]])
    budget = eps * Z
    best = -math.inf
    for j in range(nb):
        lo = Ms[j - 1] if j > 0 else -math.inf
        if A[j] > budget:
            break
        if c[j] > 0.0:
            room = budget - A[j]
            tj = min(Ms[j], m + math.log(room / c[j])) if room > 0.0 else -math.inf
        else:
            tj = Ms[j]
        if tj > lo:
            best = tj
    return best, block_bound(M, sizes, m, best), Z, m


def certify_bound(S, V, eps: float, row_to_v=None, block: int = BOUND_BLOCK):
    """Certified truncation from the blockwise bound, for every row of S.

    Keeps H_t = {i : s_i >= t} at the threshold of bound_threshold.  Returns
    a dict: t [R], k [R] (= |H_t|, never below the minimal k_eps), tau_bound
    [R] (= U(t) / Z <= eps), tv [R] (the exact TV of the truncation,
    <= tau_bound), out [R, dv] (head-only renormalised output over H_t) and
    head_mask [R, n]."""
    S = np.atleast_2d(np.asarray(S, dtype=np.float64))
    V = as_f64(V)
    if V.ndim == 2:
        V = V[None]
    R, n = S.shape
    if row_to_v is None:
        row_to_v = np.zeros(R, dtype=np.int64)
    if not (0.0 < eps < 1.0):
        raise ValueError("eps must lie in (0, 1)")
    ts, tb, tv, ks = np.empty(R), np.empty(R), np.empty(R), np.empty(R, dtype=np.int64)
    head = np.zeros((R, n), dtype=bool)
    out = np.empty((R, V.shape[-1]))
    for r in range(R):
        t, U, Z, m = bound_threshold(S[r], eps, block)
        w = np.exp(S[r] - m)
        h = S[r] >= t
        head[r] = h
        ks[r] = int(h.sum())
        ts[r], tb[r] = t, U / Z
        tv[r] = float(np.sort(w[~h]).sum()) / Z
        out[r] = (w[h] @ V[row_to_v[r]][h]) / w[h].sum()
    return {"t": ts, "k": ks, "tau_bound": tb, "tv": tv, "out": out, "head_mask": head}



# ---------------------------------------------------------------------------
# 4-bit key copy with deterministic score bounds (reading of the Abstract of
# "Certified Sparse Attention via Perturbed Retrieval", arXiv 2610.24991)
# ---------------------------------------------------------------------------
K4_LEVEL = 7  # codes in [-7, 7]


def quantize_k4(K):
    """Per-key symmetric 4-bit copy of K [..., n, d] (float or bf16 bits).

    Returns (codes int8 [..., n, d], a float32 [..., n], rho float64 [..., n]):
    a = float32(amax) / float32(7) and codes = clamp(rint(float32(k) / a), -7, 7)
    in float32 arithmetic (a zero row gets a = 0 and codes 0); rho is the
    exact Euclidean norm of k - a * codes."""
    Kf = as_f64(K).astype(np.float32)  # bf16 and fp32 values are exact in fp32
    amax = np.max(np.abs(Kf), axis=-1)
    a = (amax / np.float32(K4_LEVEL)).astype(np.float32)
    safe = np.where(a > 0, a, np.float32(1.0)).astype(np.float32)
    c = np.rint((Kf / safe[..., None]).astype(np.float32))
    c = np.clip(c, -K4_LEVEL, K4_LEVEL)
    c = np.where(a[..., None] > 0, c, 0).astype(np.int8)
    resid = Kf.astype(np.float64) - a.astype(np.float64)[..., None] * c.astype(np.float64)
    rho = np.sqrt(np.sum(resid * resid, axis=-1))
    return c, a, rho


def pack_k4(codes):
    """Two's-complement nibbles, element 2j in the low half of byte j."""
    c = np.asarray(codes, dtype=np.int16) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_k4(packed, d: int):
    """Inverse of pack_k4."""
    p = np.asarray(packed, dtype=np.uint8).astype(np.int16)
    lo, hi = p & 0xF, (p >> 4) & 0xF
    out = np.empty(p.shape[:-1] + (d,), dtype=np.int16)
    out[..., 0::2], out[..., 1::2] = lo, hi
    return np.where(out >= 8, out - 16, out).astype(np.int8)


def k4_score_bounds(q, codes, a, rho, scale):
    """Score intervals of one query row q [d] against every key of a 4-bit
    copy: shat = scale * a * (q . codes) and R = scale * ||q||_2 * rho, so
    the exact score scale * (q . k) lies in [shat - R, shat + R]."""
    q = as_f64(q)
    sc = float(scale)
    shat = sc * np.asarray(a, dtype=np.float64) * (codes.astype(np.float64) @ q)
    R = abs(sc) * float(np.linalg.norm(q)) * np.asarray(rho, dtype=np.float64)
    return shat, R


def candidates(q, K, scale, T):
    """The candidate set the scan generates: {i : scale * (q . k_i) >= T}."""
    s = float(scale) * (as_f64(K) @ as_f64(q))
    return s >= T
