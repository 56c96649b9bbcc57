"""Seeded synthetic inputs for certified Top-k attention truncation.

This module only draws inputs.  It holds none of the method's arithmetic (no
scores, softmax, selection or output), so both the fp64 oracle and the device
path can be fed from it without sharing any computation.

Every generator returns host numpy arrays.  bf16 tensors are returned as
uint16 bit patterns, rounded from float32 with round-to-nearest-even.

Workloads (sizes are the defaults; tests pass smaller ones with the same
recipe):

* ``single_query``   one head, n = 1024, d = 64, fp32, q/K/V iid N(0,1),
                     scale 2/sqrt(d) = 0.25 (so logits ~ N(0,4)).
* ``encoder``        batch 8 x 12 heads x 512 tokens, d = 64, bf16, iid N(0,1);
                     a temperature c in {0.5,1,2,4,8} per (batch, head) gives
                     the scale c/sqrt(d) for all 512 query rows of that head.
* ``gqa_decode``     32 query heads / 8 KV heads, d = 128, n = 32768, bf16;
                     K, V iid N(0,1); key 0 (the sink) and the last 64 keys
                     are shifted by 3 * u_g toward the group's queries; 16
                     planted keys per KV head are aimed at one query head each.
* ``long_decode``    batch 4 folded into heads: 128 query / 32 KV heads,
                     n = 131072, 64 planted keys per KV head and a per-query-
                     head temperature t ~ U[0.5, 2] (scale t/sqrt(d)).
* ``logit_sweep``    rows of iid N(0, sigma^2) fp32 logits with one fp32 value
                     matrix [n, 64] shared by all rows.
"""
from __future__ import annotations

import math

import numpy as np

BASE_SEED = 1000


def bf16_rne(x) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def _rng(cfg: int, rotation: int = 0, extra=()):
    return np.random.default_rng((BASE_SEED + cfg + 100 * rotation,) + tuple(extra))


def single_query(n: int = 1024, d: int = 64, rotation: int = 0, seed_extra=()):
    """fp32 single-head workload; returns q [1,d], K/V [1,n,d], head_scale [1]."""
    rng = _rng(0, rotation, seed_extra)
    q = rng.standard_normal((1, d), dtype=np.float32)
    K = rng.standard_normal((1, n, d), dtype=np.float32)
    V = rng.standard_normal((1, n, d), dtype=np.float32)
    scale = np.array([2.0 / math.sqrt(d)], dtype=np.float32)
    return {"q": q, "K": K, "V": V, "head_scale": scale, "n_q_heads": 1,
            "n_kv_heads": 1, "n": n, "d": d, "dtype": "f32"}


TEMPERATURES = (0.5, 1.0, 2.0, 4.0, 8.0)


def encoder(batch: int = 8, heads: int = 12, seq: int = 512, d: int = 64, rotation: int = 0):
    """bf16 all-queries workload, folded to q [B*H*L, d], K/V [B*H, L, d]."""
    rng = _rng(1, rotation)
    Q = rng.standard_normal((batch * heads, seq, d), dtype=np.float32)
    K = rng.standard_normal((batch * heads, seq, d), dtype=np.float32)
    V = rng.standard_normal((batch * heads, seq, d), dtype=np.float32)
    temp = rng.choice(np.array(TEMPERATURES, dtype=np.float32), size=batch * heads)
    scale = (temp / np.float32(math.sqrt(d))).astype(np.float32)
    head_scale = np.repeat(scale, seq).astype(np.float32)
    return {"q": bf16_rne(Q.reshape(batch * heads * seq, d)), "K": bf16_rne(K),
            "V": bf16_rne(V), "head_scale": head_scale, "temperature": temp,
            "n_q_heads": batch * heads * seq, "n_kv_heads": batch * heads,
            "n": seq, "d": d, "dtype": "bf16"}


def _decode_common(rng, n_q, n_kv, n, d, planted, temp_range):
    G = n_q // n_kv
    q = rng.standard_normal((n_q, d), dtype=np.float32)
    qn = q / np.linalg.norm(q, axis=1, keepdims=True)
    Kb = np.empty((n_kv, n, d), dtype=np.uint16)
    Vb = np.empty((n_kv, n, d), dtype=np.uint16)
    tail = min(64, max(n - 1, 0))
    for g in range(n_kv):
        Kg = rng.standard_normal((n, d), dtype=np.float32)
        Vg = rng.standard_normal((n, d), dtype=np.float32)
        u = qn[g * G:(g + 1) * G].sum(axis=0)
        u = u / np.linalg.norm(u)
        Kg[0] += 3.0 * u
        if tail > 0:
            Kg[n - tail:] += 3.0 * u
        lo_hi = n - tail - 1  # planted positions lie in [1, n - tail - 1]
        n_pl = min(planted, max(lo_hi, 0))
        if n_pl > 0:
            pos = rng.choice(lo_hi, size=n_pl, replace=False) + 1
            for j, p in enumerate(pos):
                h = g * G + (j % G)
                Kg[p] = 2.5 * qn[h] + rng.standard_normal(d, dtype=np.float32)
        Kb[g] = bf16_rne(Kg)
        Vb[g] = bf16_rne(Vg)
    if temp_range is None:
        head_scale = np.full(n_q, np.float32(1.0 / math.sqrt(d)), dtype=np.float32)
    else:
        t = rng.uniform(temp_range[0], temp_range[1], size=n_q).astype(np.float32)
        head_scale = (t / np.float32(math.sqrt(d))).astype(np.float32)
    return {"q": bf16_rne(q), "K": Kb, "V": Vb, "head_scale": head_scale,
            "n_q_heads": n_q, "n_kv_heads": n_kv, "n": n, "d": d, "dtype": "bf16"}


def gqa_decode(n: int = 32768, n_q: int = 32, n_kv: int = 8, d: int = 128,
               planted: int = 16, rotation: int = 0, temp_range=None):
    """bf16 GQA decode step (batch 1); temp_range (lo, hi) multiplies each query
    head's 1/sqrt(d) scale by a uniform draw from it (None: plain 1/sqrt(d))."""
    return _decode_common(_rng(2, rotation), n_q, n_kv, n, d, planted, temp_range)


def long_decode(n: int = 131072, batch: int = 4, n_q: int = 32, n_kv: int = 8,
                d: int = 128, planted: int = 64, rotation: int = 0):
    """bf16 long-context GQA decode, batch folded into heads."""
    return _decode_common(_rng(3, rotation), batch * n_q, batch * n_kv, n, d,
                          planted, (0.5, 2.0))


LOGIT_SIGMAS = (1.0, 2.0, 3.0, 4.0)
LOGIT_NS = (4096, 65536, 1048576)
LOGIT_EPS = (0.001, 0.01, 0.1)


def logit_sweep(sigma: float, n: int, rows: int = 1024, dv: int = 64, rotation: int = 0):
    """fp32 logits [rows, n] = sigma * N(0,1) and one shared V [1, n, dv]."""
    si = LOGIT_SIGMAS.index(sigma) if sigma in LOGIT_SIGMAS else 99
    rng = _rng(4, rotation, (si, int(n)))
    L = rng.standard_normal((rows, n), dtype=np.float32)
    L *= np.float32(sigma)
    V = rng.standard_normal((1, n, dv), dtype=np.float32)
    return {"logits": L, "V": V, "rows": rows, "n": n, "dv": dv, "n_v": 1,
            "sigma": sigma}
