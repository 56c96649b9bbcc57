#!/usr/bin/env python3
"""Benchmark of certified Top-k attention truncation on one MI355X.

Workload (one step = one ctopk_certify call = the whole path: score scan,
global log-sum-exp, mass-weighted radix select, head-only value stream):
GQA decode, batch 1, 32 query heads / 8 KV heads, d = 128, n = 32768 keys,
bf16 KV cache, eps = 0.01, scale 1/sqrt(d); keys iid N(0,1) with the sink and
last 64 keys shifted toward the group's queries and 16 planted keys per KV
head.  Inputs are synthetic and seeded, generated on the host and resident in
HBM before timing.  Steps rotate over R independent input sets (R * 128 MiB
of K and V, above the 256 MB Infinity Cache) so that K and V come from HBM.

Prints one JSON line.  `value` is query-heads/s; the roofline block is for
the dominant kernel (the one with the longest average duration):
algorithmic bytes of one launch (kernel_bytes) divided by its average
duration, timed live with HIP events that the library attaches to each
kernel's dispatch (ctopk_record_kernel_events), over the same rotating steps
as the headline loop; `rooflines` gives the same figures for every kernel.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "certified top-k decode query-heads/s + achieved HBM GB/s (% peak), n=32K GQA"
PEAK_HBM_GBPS = 8000.0
# Kernel names per decode plan, in launch order (ctopk_plan).  The level-0
# histogram runs only for rows longer than the select holds in registers;
# otherwise its event pair is recorded back to back and times no kernel.
KERNELS_BY_PLAN = {
    2: ("score_scan", "hist0", "resolve", "vsum", "finalize"),
    3: ("score_scan", "hist0", "select_dense", "tail", "finalize"),
    4: ("score_scan", "hist0", "bound", "vsum", "finalize"),
}
PLAN_NAMES = {1: "encoder", 2: "decode", 3: "decode_overlap", 4: "decode_bound"}
# Rows of at most this many keys are resolved in registers, without the
# separate level-0 histogram kernel (whose event pair then times no kernel).
REGISTER_ROW_KEYS = 32768
PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_gqa_decode_n32768.md")
CSRC = os.path.join(ROOT, "certified_top_sparse_amd", "csrc")
_COMMON = ("kernels.h", "device_common.h")
# Sources each kernel is built from: a counter figure applies only while they
# are unchanged.
KERNEL_SOURCES = {
    "score_scan": ("score_scan.hip", "scan_dot.h") + _COMMON,
    "k4_scan": ("k4.hip", "scan_dot.h") + _COMMON,
    "k4_rescore": ("k4.hip", "scan_dot.h") + _COMMON,
    "select_dense": ("select.hip", "vsum_body.h") + _COMMON,
    "resolve": ("select.hip", "vsum_body.h") + _COMMON,
    "tail": ("vsum.hip", "vsum_body.h") + _COMMON,
    "vsum": ("vsum.hip", "vsum_body.h") + _COMMON,
    "bound": ("bound.hip",) + _COMMON,
}


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle as it stands, on the host's cores
# ---------------------------------------------------------------------------
_CPU = {}


def _cpu_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _cpu_head(h):
    import oracle
    wl, eps = _CPU["wl"], _CPU["eps"]
    G = wl["n_q_heads"] // wl["n_kv_heads"]
    g = h // G
    r = oracle.certify(wl["q"][h:h + 1], wl["K"][g:g + 1], wl["V"][g:g + 1], eps, 1, 1,
                       head_scale=wl["head_scale"][h:h + 1])
    return int(r["k_eps"][0])


def cpu_baseline(wl, eps, seconds):
    import multiprocessing as mp
    _CPU["wl"], _CPU["eps"] = wl, eps
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    procs = max(1, min(16, avail))
    heads = 0
    ctx = mp.get_context("fork")
    with ctx.Pool(procs, initializer=_cpu_init) as pool:
        pool.map(_cpu_head, range(procs))  # start-up, untimed
        t0 = time.perf_counter()
        while True:
            pool.map(_cpu_head, range(wl["n_q_heads"]))
            heads += wl["n_q_heads"]
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": heads / dt, "unit": "query-heads/s", "cores": procs, "kind": "oracle",
            "sample": (f"{heads} query heads ({heads // wl['n_q_heads']} full steps of the same "
                       f"workload, n={wl['n']}, eps={eps}) in {dt:.1f} s, fp64 numpy, "
                       f"{procs} single-threaded worker processes"),
            "cpu_model": model}


# ---------------------------------------------------------------------------
# HIP events through the runtime torch loaded
# ---------------------------------------------------------------------------
class Hip:
    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return e.value

    def elapsed_ms(self, a, b):
        out = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(out.value)

    def destroy(self, e):
        self.lib.hipEventDestroy(ctypes.c_void_p(e))


def sources_digest(names):
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel):
    """HBM bytes per dispatch of `kernel` from the committed rocprofv3 --pmc
    summary, if it was taken on the kernel's current sources."""
    try:
        with open(PMC_SUMMARY) as f:
            text = f.read()
    except OSError:
        return None
    m = re.search(r"```json\s*(\{.*?\})\s*```", text, re.S)
    if not m or kernel not in KERNEL_SOURCES:
        return None
    entry = json.loads(m.group(1)).get("kernels", {}).get(kernel)
    if not entry or entry.get("sources_sha256_16") != sources_digest(KERNEL_SOURCES[kernel]):
        return None
    return entry.get("traffic_bytes_per_dispatch")


def copy_stream_gbps(torch, bufs, reps=60):
    """Achievable streaming rate on this machine: a plain device copy from the
    same rotating 64 MiB K buffers the decode steps read into one 64 MiB
    destination, counted as bytes read plus bytes written (timed with events)."""
    dst = torch.empty_like(bufs[0])
    for b in bufs:
        dst.copy_(b)
    torch.cuda.synchronize()
    a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(reps):
        dst.copy_(bufs[i % len(bufs)])
    e.record()
    torch.cuda.synchronize()
    nbytes = 2 * dst.numel() * dst.element_size()
    return nbytes * reps / (a.elapsed_time(e) * 1e-3) / 1e9


def group_heads(G):
    """Query heads per workgroup of the value passes (bf16 values)."""
    return 1 if G == 1 else (2 if G == 2 else (4 if G <= 4 else 8))


def tail_pass_rows(bits, k, n_kv, G, n):
    """V rows the tail pass gathers: per head group, the keys outside some
    head's set (tail mode: the tails together hold no more keys than the
    largest head) or inside some head's set (head mode)."""
    gb = group_heads(G)
    rows = 0
    for g in range(n_kv):
        for z in range(0, G, gb):
            hs = slice(g * G + z, g * G + min(G, z + gb))
            kk = k[hs].astype(np.int64)
            hb = bits[hs]
            if (n - kk).sum() <= kk.max():
                rows += int((~hb).any(axis=0).sum())
            else:
                rows += int(hb.any(axis=0).sum())
    return rows


def bound_leg(lib, ct, torch, hip, Q, Kd, Vd, steps, eps):
    """The same decode workload certified by the blockwise bound
    (CTOPK_FLAG_BOUND): per-call time, per-kernel times and the keys kept,
    against the exact select's."""
    sets = len(Q)
    n_q, d = Q[0].shape
    n = Kd[0].shape[1]
    out = torch.empty((n_q, d), dtype=torch.float32, device="cuda")
    k_eps = torch.empty(n_q, dtype=torch.int32, device="cuda")
    tau = torch.empty(n_q, dtype=torch.float64, device="cuda")
    args = [ct.make_args(Q[r], Kd[r], Vd[r], eps, out=out, k_eps=k_eps, tau=tau,
                         flags=ct.CTOPK_FLAG_BOUND) for r in range(sets)]
    assert ct.ctopk_plan(args[0]) == ct.CTOPK_PLAN_DECODE_BOUND
    names = KERNELS_BY_PLAN[ct.CTOPK_PLAN_DECODE_BOUND]
    sptr = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    call = lib.ctopk_certify_ex

    def step(i):
        rc = call(ctypes.byref(args[i % sets]), sptr)
        if rc != 0:
            raise RuntimeError(ct.ctopk_last_error_string())

    kmean, taumax = [], 0.0
    for i in range(sets):
        step(i)
        torch.cuda.synchronize()
        kmean.append(float(k_eps.double().mean().item()))
        taumax = max(taumax, float(tau.max().item()))
    for i in range(20):
        step(i)
    e0, e1 = hip.event(), hip.event()
    torch.cuda.synchronize()
    hip.lib.hipEventRecord(ctypes.c_void_p(e0), sptr)
    for i in range(steps):
        step(i)
    hip.lib.hipEventRecord(ctypes.c_void_p(e1), sptr)
    torch.cuda.synchronize()
    us = hip.elapsed_ms(e0, e1) * 1e3 / steps
    hip.destroy(e0)
    hip.destroy(e1)
    n_ev = 2 * len(names)
    evs = [[hip.event() for _ in range(n_ev)] for _ in range(steps)]
    arrs = [(ctypes.c_void_p * n_ev)(*[ctypes.c_void_p(e) for e in row]) for row in evs]
    torch.cuda.synchronize()
    for i in range(steps):
        lib.ctopk_record_kernel_events(arrs[i], n_ev)
        step(i)
    torch.cuda.synchronize()
    per = np.array([[hip.elapsed_ms(row[2 * j], row[2 * j + 1]) for j in range(len(names))]
                    for row in evs])
    kern = {name: (None if name == "hist0" else round(float(per[:, j].mean()) * 1e3, 3))
            for j, name in enumerate(names)}
    for row in evs:
        for e in row:
            hip.destroy(e)
    return {"eps": eps, "steps": steps, "us_per_call": round(us, 3),
            "query_heads_per_s": round(n_q / (us * 1e-6), 1), "kernel_us": kern,
            "mean_k_over_n": round(float(np.mean(kmean)) / n, 4), "max_tau": taumax,
            "bound_kernel_traffic_bytes": read_traffic("bound")}


def k4_leg(lib, ct, torch, hip, Q, Kd, T_cut, T_top, steps):
    """The 4-bit key copy on the decode inputs: exact candidate generation
    (ctopk_candidates_k4) at two thresholds per head -- the certified cut
    score (candidates = the exact head) and the 64th largest score (a
    retrieval-sized set) -- with per-kernel times, keys rescored at full
    width, and the scan's bytes against the full-width score scan's."""
    sets = len(Q)
    n_q, d = Q[0].shape
    n_kv, n, _ = Kd[0].shape
    copies = [ct.ctopk_quantize_k4(K) for K in Kd]
    torch.cuda.synchronize()
    ev0, ev1 = hip.event(), hip.event()
    sptr = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    hip.lib.hipEventRecord(ctypes.c_void_p(ev0), sptr)
    for r in range(sets):
        ct.ctopk_quantize_k4(Kd[r])
    hip.lib.hipEventRecord(ctypes.c_void_p(ev1), sptr)
    torch.cuda.synchronize()
    quant_us = hip.elapsed_ms(ev0, ev1) * 1e3 / sets
    mask = torch.empty((n_q, (n + 31) // 32), dtype=torch.int32, device="cuda")
    count = torch.empty(n_q, dtype=torch.int32, device="cuda")
    resc = torch.empty(n_kv, dtype=torch.int32, device="cuda")
    names = ("k4_scan", "k4_rescore")
    out = {"quantize_us_per_call": round(quant_us, 3),
           "scan_bytes_per_call": n_kv * n * (d // 2 + 8),
           "full_width_scan_bytes": n_kv * n * d * 2}
    for label, Ts in (("cut_score", T_cut), ("top64", T_top)):
        thr = [torch.from_numpy(np.ascontiguousarray(t, dtype=np.float32)).cuda() for t in Ts]
        args = [ct.make_k4_args(Q[r], Kd[r], *copies[r], thr[r], sel_mask=mask, count=count,
                                rescored=resc) for r in range(sets)]
        call = lib.ctopk_candidates_k4

        def step(i):
            rc = call(ctypes.byref(args[i % sets]), sptr)
            if rc != 0:
                raise RuntimeError(ct.ctopk_last_error_string())

        fr, cnt = [], []
        for r in range(sets):
            step(r)
            torch.cuda.synchronize()
            fr.append(float(resc.double().sum().item()) / (n_kv * n))
            cnt.append(float(count.double().mean().item()))
        for i in range(20):
            step(i)
        e0, e1 = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.lib.hipEventRecord(ctypes.c_void_p(e0), sptr)
        for i in range(steps):
            step(i)
        hip.lib.hipEventRecord(ctypes.c_void_p(e1), sptr)
        torch.cuda.synchronize()
        us = hip.elapsed_ms(e0, e1) * 1e3 / steps
        hip.destroy(e0)
        hip.destroy(e1)
        n_ev = 2 * len(names)
        evs = [[hip.event() for _ in range(n_ev)] for _ in range(steps)]
        arrs = [(ctypes.c_void_p * n_ev)(*[ctypes.c_void_p(e) for e in row]) for row in evs]
        torch.cuda.synchronize()
        for i in range(steps):
            lib.ctopk_record_kernel_events(arrs[i], n_ev)
            step(i)
        torch.cuda.synchronize()
        per = np.array([[hip.elapsed_ms(row[2 * j], row[2 * j + 1]) for j in range(len(names))]
                        for row in evs])
        for row in evs:
            for e in row:
                hip.destroy(e)
        kern = {nm: round(float(per[:, j].mean()) * 1e3, 3) for j, nm in enumerate(names)}
        scan_gbps = out["scan_bytes_per_call"] / (kern["k4_scan"] * 1e-6) / 1e9
        out[label] = {"us_per_call": round(us, 3), "kernel_us": kern,
                      "mean_candidates": round(float(np.mean(cnt)), 1),
                      "rescored_fraction": round(float(np.mean(fr)), 4),
                      "k4_scan_gbps": round(scan_gbps, 1),
                      "k4_scan_roofline": {"bound": "hbm", "achieved": round(scan_gbps, 1),
                                           "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                           "frac": round(scan_gbps / PEAK_HBM_GBPS, 4),
                                           "traffic": read_traffic("k4_scan")},
                      "bytes_per_call": round(out["scan_bytes_per_call"] + float(np.mean(fr)) * n_kv * n * d * 2)}
    hip.destroy(ev0)
    hip.destroy(ev1)
    return out


def long_leg(lib, ct, torch, hip, steps, eps):
    """Long-context decode: batch 4 folded into 128 query / 32 KV heads,
    n = 131072, d = 128, bf16, per-head temperature in [0.5, 2] (1 GiB each of
    K and V, far above the 256 MB Infinity Cache, so no rotation is needed).
    Per-call time, per-kernel times, and the score scan's rate against the
    8 TB/s peak."""
    wl = workloads.long_decode(batch=4)
    n_q, d = wl["q"].shape
    n_kv, n, _ = wl["K"].shape

    def dev(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    q, K, V, hs = dev(wl["q"]), dev(wl["K"]), dev(wl["V"]), dev(wl["head_scale"])
    del wl
    out = torch.empty((n_q, d), dtype=torch.float32, device="cuda")
    k_eps = torch.empty(n_q, dtype=torch.int32, device="cuda")
    tau = torch.empty(n_q, dtype=torch.float64, device="cuda")
    mask = torch.empty((n_q, (n + 31) // 32), dtype=torch.int32, device="cuda")
    res = ct.ctopk_certify_ex(q, K, V, eps, head_scale=hs, want_mask=True)
    torch.cuda.synchronize()
    words = res["sel_mask"].cpu().numpy().astype(np.int32).view(np.uint8)
    bits = np.unpackbits(words.reshape(n_q, -1), axis=1, bitorder="little")[:, :n].astype(bool)
    union = int(bits.reshape(n_kv, n_q // n_kv, n).any(axis=1).sum())
    kmean = float(res["k_eps"].double().mean().item()) / n
    args = ct.make_args(q, K, V, eps, head_scale=hs, out=out, k_eps=k_eps, tau=tau)
    plan = ct.ctopk_plan(args)
    names = KERNELS_BY_PLAN[plan]
    sptr = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    call = lib.ctopk_certify_ex

    def step():
        rc = call(ctypes.byref(args), sptr)
        if rc != 0:
            raise RuntimeError(ct.ctopk_last_error_string())

    for _ in range(5):
        step()
    e0, e1 = hip.event(), hip.event()
    torch.cuda.synchronize()
    hip.lib.hipEventRecord(ctypes.c_void_p(e0), sptr)
    for _ in range(steps):
        step()
    hip.lib.hipEventRecord(ctypes.c_void_p(e1), sptr)
    torch.cuda.synchronize()
    us = hip.elapsed_ms(e0, e1) * 1e3 / steps
    hip.destroy(e0)
    hip.destroy(e1)
    n_ev = 2 * len(names)
    evs = [[hip.event() for _ in range(n_ev)] for _ in range(steps)]
    arrs = [(ctypes.c_void_p * n_ev)(*[ctypes.c_void_p(e) for e in row]) for row in evs]
    torch.cuda.synchronize()
    for i in range(steps):
        lib.ctopk_record_kernel_events(arrs[i], n_ev)
        step()
    torch.cuda.synchronize()
    per = np.array([[hip.elapsed_ms(row[2 * j], row[2 * j + 1]) for j in range(len(names))]
                    for row in evs])
    for row in evs:
        for e in row:
            hip.destroy(e)
    kern = {nm: round(float(per[:, j].mean()) * 1e3, 3) for j, nm in enumerate(names)}
    k_bytes = n_kv * n * d * 2
    scan_gbps = k_bytes / (kern["score_scan"] * 1e-6) / 1e9
    e2e_gbps = (k_bytes + union * d * 2) / (us * 1e-6) / 1e9
    return {"workload": "long_decode batch 4: 128 query / 32 KV heads, n=131072, d=128, bf16",
            "eps": eps, "steps": steps, "plan": PLAN_NAMES.get(plan, plan),
            "us_per_call": round(us, 3), "query_heads_per_s": round(n_q / (us * 1e-6), 1),
            "kernel_us": kern, "scan_gbps": round(scan_gbps, 1),
            "scan_frac_of_peak": round(scan_gbps / PEAK_HBM_GBPS, 4),
            "hbm_gbps_end_to_end": round(e2e_gbps, 1), "v_union_fraction": round(union / (n_kv * n), 4),
            "mean_k_over_n": round(kmean, 4)}


def logits_leg(lib, ct, torch, hip, steps, eps):
    """The select and output on given logits (ctopk_certify_logits): 1024 rows
    of sigma = 2 Gaussian fp32 logits, n = 65536, one shared fp32 V [n, 64]
    (256 MiB of logits, above the 256 MB Infinity Cache).  Per-call and
    per-kernel times, rows/s and the logits' read rate."""
    wl = workloads.logit_sweep(2.0, 65536)
    rows, n, dv = wl["rows"], wl["n"], wl["dv"]
    L = torch.from_numpy(wl["logits"]).cuda()
    V = torch.from_numpy(wl["V"]).cuda()
    del wl
    out = torch.empty((rows, dv), dtype=torch.float32, device="cuda")
    k_eps = torch.empty(rows, dtype=torch.int32, device="cuda")
    tau = torch.empty(rows, dtype=torch.float64, device="cuda")
    sptr = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    vp = ctypes.c_void_p
    argv = (vp(L.data_ptr()), vp(V.data_ptr()), ct.CTOPK_F32, n, dv, rows, 1, float(eps), None, 0,
            sptr, vp(out.data_ptr()), vp(k_eps.data_ptr()), vp(tau.data_ptr()), None, None)

    def step():
        rc = lib.ctopk_certify_logits(*argv)
        if rc != 0:
            raise RuntimeError(ct.ctopk_last_error_string())

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    kmean = float(k_eps.double().mean().item()) / n
    e0, e1 = hip.event(), hip.event()
    hip.lib.hipEventRecord(ctypes.c_void_p(e0), sptr)
    for _ in range(steps):
        step()
    hip.lib.hipEventRecord(ctypes.c_void_p(e1), sptr)
    torch.cuda.synchronize()
    us = hip.elapsed_ms(e0, e1) * 1e3 / steps
    hip.destroy(e0)
    hip.destroy(e1)
    names = ("resolve", "vsum", "finalize")
    n_ev = 2 * len(names)
    evs = [[hip.event() for _ in range(n_ev)] for _ in range(steps)]
    arrs = [(ctypes.c_void_p * n_ev)(*[ctypes.c_void_p(e) for e in row]) for row in evs]
    torch.cuda.synchronize()
    for i in range(steps):
        lib.ctopk_record_kernel_events(arrs[i], n_ev)
        step()
    torch.cuda.synchronize()
    per = np.array([[hip.elapsed_ms(row[2 * j], row[2 * j + 1]) for j in range(len(names))]
                    for row in evs])
    for row in evs:
        for e in row:
            hip.destroy(e)
    kern = {nm: round(float(per[:, j].mean()) * 1e3, 3) for j, nm in enumerate(names)}
    lbytes = rows * n * 4
    return {"workload": "logit sweep: 1024 rows x 65536 fp32 logits, sigma=2, shared fp32 V [65536, 64]",
            "eps": eps, "steps": steps, "us_per_call": round(us, 3),
            "rows_per_s": round(rows / (us * 1e-6), 1), "kernel_us": kern,
            "select_logit_gbps": round(lbytes / (kern["resolve"] * 1e-6) / 1e9, 1),
            "mean_k_over_n": round(kmean, 4)}


def encoder_leg(lib, ct, torch, hip, steps, eps, sets=16):
    """All-queries (encoder-shaped) workload: batch 8, 12 heads, 512 queries and
    512 keys per head, d = 64, bf16, per-head temperature; every query row of a
    head is one certified row.  Rotates over `sets` input sets (16 x 18.9 MB,
    above the 256 MB Infinity Cache).  Returns per-call time and rates."""
    wls = [workloads.encoder(rotation=r) for r in range(sets)]
    w0 = wls[0]
    n, d, n_q, n_kv = w0["n"], w0["d"], w0["n_q_heads"], w0["n_kv_heads"]

    def dev(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    ins = [(dev(w["q"]), dev(w["K"]), dev(w["V"]), dev(w["head_scale"])) for w in wls]
    out = torch.empty((n_q, d), dtype=torch.float32, device="cuda")
    k_eps = torch.empty(n_q, dtype=torch.int32, device="cuda")
    tau = torch.empty(n_q, dtype=torch.float64, device="cuda")
    args = [ct.make_args(q, K, V, eps, head_scale=hs, out=out, k_eps=k_eps, tau=tau)
            for (q, K, V, hs) in ins]
    sptr = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    call = lib.ctopk_certify_ex

    def step(i):
        rc = call(ctypes.byref(args[i % sets]), sptr)
        if rc != 0:
            raise RuntimeError(ct.ctopk_last_error_string())

    kmean = []
    for i in range(sets):
        step(i)
        torch.cuda.synchronize()
        kmean.append(float(k_eps.double().mean().item()))
    for i in range(20):
        step(i)
    # kernel duration: an event pair attached to each call's one kernel
    pairs = [(hip.event(), hip.event()) for _ in range(steps)]
    arrs = [(ctypes.c_void_p * 2)(ctypes.c_void_p(a), ctypes.c_void_p(b)) for a, b in pairs]
    torch.cuda.synchronize()
    for i in range(steps):
        lib.ctopk_record_kernel_events(arrs[i], 2)
        step(i)
    torch.cuda.synchronize()
    kern_us = float(np.mean([hip.elapsed_ms(a, b) for a, b in pairs])) * 1e3
    for a, b in pairs:
        hip.destroy(a)
        hip.destroy(b)
    e0, e1 = hip.event(), hip.event()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    hip.lib.hipEventRecord(ctypes.c_void_p(e0), sptr)
    for i in range(steps):
        step(i)
    hip.lib.hipEventRecord(ctypes.c_void_p(e1), sptr)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = hip.elapsed_ms(e0, e1) * 1e3 / steps
    hip.destroy(e0)
    hip.destroy(e1)
    in_bytes = 3 * n_kv * n * d * 2
    qk_flops = 2.0 * n_kv * (n_q // n_kv) * n * d
    return {"workload": "encoder batch 8 x 12 heads, 512 queries x 512 keys, d=64, bf16",
            "eps": eps, "steps": steps, "rotating_sets": sets,
            "us_per_call": round(us, 3), "us_per_call_wall": round(wall * 1e6 / steps, 3),
            "kernel_us": round(kern_us, 3),
            "query_rows_per_s": round(n_q / (us * 1e-6), 1),
            "qk_mfma_tflops": round(qk_flops / (us * 1e-6) / 1e12, 2),
            "input_gbps": round(in_bytes / (us * 1e-6) / 1e9, 1),
            "mean_k_over_n": round(float(np.mean(kmean)) / n, 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--eps", type=float, default=0.01)
    ap.add_argument("--sets", type=int, default=6, help="rotating input sets (128 MiB each)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline leg")
    ap.add_argument("--no-kernel-events", action="store_true")
    ap.add_argument("--bound-steps", type=int, default=1000,
                    help="calls of the blockwise-bound leg on the decode workload; 0 skips it")
    ap.add_argument("--logits-steps", type=int, default=20,
                    help="calls of the given-logits leg (1024 x 65536 fp32); 0 skips it")
    ap.add_argument("--long-steps", type=int, default=40,
                    help="calls of the long-context decode leg (n = 131072, 1 GiB of K); 0 skips it")
    ap.add_argument("--k4-steps", type=int, default=500,
                    help="calls per threshold of the 4-bit candidate leg; 0 skips it")
    ap.add_argument("--encoder-steps", type=int, default=500,
                    help="calls of the all-queries (encoder-shaped) leg; 0 skips it")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the decode path shards by KV head with no exchange, so every GPU would run this "
              "same one-GPU step on its own heads.", file=sys.stderr)
        sys.exit(2)

    t_gen = time.perf_counter()
    sets = [workloads.gqa_decode(rotation=r) for r in range(args.sets)]
    wl0 = sets[0]
    n, d, n_q, n_kv = wl0["n"], wl0["d"], wl0["n_q_heads"], wl0["n_kv_heads"]
    print(f"[bench] generated {args.sets} input sets in {time.perf_counter() - t_gen:.1f} s",
          file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu:
        print(f"[bench] CPU baseline (~{args.cpu_seconds:.0f} s)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl0, args.eps, args.cpu_seconds)

    import torch
    import certified_top_sparse_amd as ct

    lib = ct.load()
    hip = Hip()
    torch.cuda.set_device(0)

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()

    Q = [dev(s["q"]) for s in sets]
    Kd = [dev(s["K"]) for s in sets]
    Vd = [dev(s["V"]) for s in sets]
    out = torch.empty((n_q, d), dtype=torch.float32, device="cuda")
    k_eps = torch.empty(n_q, dtype=torch.int32, device="cuda")
    tau = torch.empty(n_q, dtype=torch.float64, device="cuda")

    # Union of the group's head sets per input set: the V rows the path must read.
    G = n_q // n_kv
    union_rows = []
    tail_rows = []
    kmean = []
    T_cut, T_top = [], []
    for r in range(args.sets):
        res = ct.ctopk_certify_ex(Q[r], Kd[r], Vd[r], args.eps, want_mask=True, want_scores=True)
        torch.cuda.synchronize()
        words = res["sel_mask"].cpu().numpy().astype(np.int32).view(np.uint8)
        bits = np.unpackbits(words.reshape(n_q, -1), axis=1, bitorder="little")[:, :n].astype(bool)
        sc = res["scores"].cpu().numpy()
        T_cut.append(np.array([sc[h][bits[h]].min() for h in range(n_q)], dtype=np.float32))
        T_top.append(np.sort(sc, axis=1)[:, -64].astype(np.float32))
        union_rows.append(int(bits.reshape(n_kv, G, n).any(axis=1).sum()))
        kr = res["k_eps"].cpu().numpy()
        tail_rows.append(tail_pass_rows(bits, kr, n_kv, G, n))
        kmean.append(float(kr.astype(np.float64).mean()))
    k_bytes = n_kv * n * d * 2
    v_bytes = float(np.mean(union_rows)) * d * 2
    score_bytes = n_q * n * 4
    # Algorithmic bytes of one launch of each kernel: what it must read.
    kernel_bytes = {
        "score_scan": k_bytes,                                   # K
        "resolve": score_bytes,                                  # the scores
        "vsum": v_bytes + score_bytes,                           # head-union V rows, scores
        "select_dense": k_bytes + 2 * score_bytes,               # all of V, scores twice
        "tail": float(np.mean(tail_rows)) * d * 2 + score_bytes,  # gathered V rows, scores
    }

    # A plain copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters.
    src = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst

    plan_args = ct.make_args(Q[0], Kd[0], Vd[0], args.eps, out=out, k_eps=k_eps, tau=tau)
    plan = ct.ctopk_plan(plan_args)
    KERNELS = KERNELS_BY_PLAN[plan]

    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    qp = [ctypes.c_void_p(t.data_ptr()) for t in Q]
    kp = [ctypes.c_void_p(t.data_ptr()) for t in Kd]
    vp = [ctypes.c_void_p(t.data_ptr()) for t in Vd]
    op, kep, tp = (ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(k_eps.data_ptr()),
                   ctypes.c_void_p(tau.data_ptr()))
    eps = float(args.eps)

    def step(i):
        r = i % args.sets
        rc = lib.ctopk_certify(qp[r], kp[r], vp[r], n, d, n_q, n_kv, eps, sptr, op, kep, tp)
        if rc != 0:
            raise RuntimeError(ct.ctopk_last_error_string())

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: exactly `steps` calls, bracketed by device synchronisation.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    value = n_q * args.steps / wall

    # Instrumented pass over the same steps: the library attaches a (start,
    # stop) event pair to each kernel's dispatch, so each pair times one kernel.
    n_ev = 2 * len(KERNELS)
    kernel_us = {}
    ms_events = None
    if not args.no_kernel_events:
        evs = [[hip.event() for _ in range(n_ev)] for _ in range(args.steps)]
        arm = lib.ctopk_record_kernel_events
        ev_arrays = [(ctypes.c_void_p * n_ev)(*[ctypes.c_void_p(e) for e in row]) for row in evs]
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(args.steps):
            arm(ev_arrays[i], n_ev)
            step(i)
        torch.cuda.synchronize()
        ms_events = (time.perf_counter() - t1) * 1e3 / args.steps
        per = np.array([[hip.elapsed_ms(row[2 * j], row[2 * j + 1]) for j in range(len(KERNELS))]
                        for row in evs])
        for j, name in enumerate(KERNELS):
            kernel_us[name] = round(float(per[:, j].mean()) * 1e3, 3)
        if n <= REGISTER_ROW_KEYS:  # no level-0 histogram kernel is launched
            kernel_us["hist0"] = None
        for row in evs:
            for e in row:
                hip.destroy(e)

    rooflines = {}
    for name, us in kernel_us.items():
        if us is None or name not in kernel_bytes:
            continue
        achieved = kernel_bytes[name] / (us * 1e-6) / 1e9
        rooflines[name] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                           "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                           "traffic": read_traffic(name), "kernel": name,
                           "algorithmic_bytes_per_launch": round(kernel_bytes[name]),
                           "avg_launch_us": us}
    roofline = max(rooflines.values(), key=lambda r: r["avg_launch_us"]) if rooflines else None

    bound = None
    if args.bound_steps > 0:
        bound = bound_leg(lib, ct, torch, hip, Q, Kd, Vd, args.bound_steps, eps)

    logits = None
    if args.logits_steps > 0:
        logits = logits_leg(lib, ct, torch, hip, args.logits_steps, eps)

    long_decode = None
    if args.long_steps > 0:
        long_decode = long_leg(lib, ct, torch, hip, args.long_steps, eps)

    k4 = None
    if args.k4_steps > 0:
        k4 = k4_leg(lib, ct, torch, hip, Q, Kd, T_cut, T_top, args.k4_steps)

    encoder = None
    if args.encoder_steps > 0:
        encoder = encoder_leg(lib, ct, torch, hip, args.encoder_steps, eps)

    e2e_gbps = (k_bytes + v_bytes) / (ms_per_step * 1e-3) / 1e9
    stream_gbps = copy_stream_gbps(torch, Kd)
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "query-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gqa_decode", "batch": 1, "n": n, "n_q_heads": n_q,
                   "n_kv_heads": n_kv, "d": d, "eps": eps, "kv_dtype": "bf16",
                   "rotating_sets": args.sets},
        "roofline": roofline,
        "rooflines": rooflines,
        "cpu_baseline": cpu,
        "hbm_gbps_end_to_end": round(e2e_gbps, 1),
        "hbm_frac_end_to_end": round(e2e_gbps / PEAK_HBM_GBPS, 4),
        "copy_stream_gbps": round(stream_gbps, 1),
        "bytes_per_step": {"K": k_bytes, "V_union": round(v_bytes)},
        "v_union_fraction": round(v_bytes / k_bytes, 4),
        "mean_k_eps": round(float(np.mean(kmean)), 1),
        "plan": PLAN_NAMES.get(plan, plan),
        "kernel_us": kernel_us,
        "ms_per_step_with_kernel_events": None if ms_events is None else round(ms_events, 5),
        "bound_certificate": bound,
        "k4_candidates": k4,
        "long_decode": long_decode,
        "logits_select": logits,
        "encoder": encoder,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
