#!/usr/bin/env python3
"""Benchmark of certified Top-k attention truncation on one MI355X.

Headline workload (one step = one ctopk_certify call = the whole path: score
scan, global log-sum-exp, mass-weighted radix select, head-only value
stream): GQA decode, batch 1, 32 query heads / 8 KV heads, d = 128,
n = 32768 keys, bf16 KV cache, eps = 0.01, scale 1/sqrt(d); keys iid N(0,1)
with the sink and last 64 keys shifted toward the group's queries and 16
planted keys per KV head.  Inputs are synthetic and seeded, generated on the
host and resident in HBM before timing.  Steps rotate over R independent
input sets (R * 128 MiB of K and V, above the 256 MB Infinity Cache) so that
K and V come from HBM.

Prints one JSON line.  `value` is query-heads/s.  Algorithmic bytes follow
the path's definition: the K scan (every key row once) plus the V rows of
the union of the head sets of each KV group (each such row once).  They are
assigned to the kernel that must move them -- K to the score scan, the
V-union to the kernel that streams V -- and every other byte a kernel moves
(the fp32 score buffer, partial sums, V rows read a second time) is
overhead, reported under `traffic` from the committed rocprofv3 counters.
`roofline` is the dominant kernel (longest average duration among those with
algorithmic bytes): those bytes divided by its average duration, timed live
with HIP events that the library attaches to each kernel's dispatch
(ctopk_record_kernel_events) over the same rotating steps.
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
    3: ("score_scan", "hist0", "select_spec"),
    4: ("score_scan", "hist0", "bound", "vsum", "finalize"),
    5: ("short_row",),
}
# The kernel of each plan that streams the V rows of the head sets.
V_KERNEL = {2: "vsum", 3: "select_spec", 4: "vsum"}
PLAN_NAMES = {1: "encoder", 2: "decode", 3: "decode_overlap", 4: "decode_bound",
              5: "decode_fused"}
PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_gqa_decode_n32768.md")
CSRC = os.path.join(ROOT, "certified_top_sparse_amd", "csrc")
_COMMON = ("kernels.h", "device_common.h")
# Sources each kernel is built from: a counter figure applies only while they
# are unchanged.
KERNEL_SOURCES = {
    "score_scan": ("score_scan.hip", "scan_dot.h") + _COMMON,
    "k4_scan": ("k4.hip", "scan_dot.h") + _COMMON,
    "k4_rescore": ("k4.hip", "scan_dot.h") + _COMMON,
    "select_spec": ("select.hip", "vsum_body.h") + _COMMON,
    "resolve": ("select.hip", "vsum_body.h") + _COMMON,
    "vsum": ("vsum.hip", "vsum_body.h") + _COMMON,
    "bound": ("bound.hip",) + _COMMON,
}
# Worker processes the CPU baseline may start: the GPU machine's host share for
# one GPU (the box limits processes per call).
CPU_PROCS_MAX = 16


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


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


def cpu_model():
    model, sockets = "", set()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name") and not model:
                    model = line.split(":", 1)[1].strip()
                elif line.startswith("physical id"):
                    sockets.add(line.split(":", 1)[1].strip())
    except OSError:
        pass
    return model, len(sockets)


def cpu_baseline(wl, eps, seconds):
    import multiprocessing as mp
    _CPU["wl"], _CPU["eps"] = wl, eps
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    procs = max(1, min(CPU_PROCS_MAX, avail))
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
    model, sockets = cpu_model()
    return {"value": heads / dt, "unit": "query-heads/s", "cores": procs, "kind": "oracle",
            "sample": (f"{heads} query heads ({heads // wl['n_q_heads']} full steps of the same "
                       f"workload, n={wl['n']}, eps={eps}) in {dt:.1f} s, fp64 numpy, "
                       f"{procs} single-threaded worker processes, one query head per task"),
            "cpu_model": model, "sockets": sockets, "affinity_cores": avail,
            "os_cpu_count": os.cpu_count()}


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

    def record(self, e, sptr):
        self.lib.hipEventRecord(ctypes.c_void_p(e), sptr)

    def elapsed_ms(self, a, b):
        out = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(out.value)

    def destroy(self, e):
        self.lib.hipEventDestroy(ctypes.c_void_p(e))


class Timer:
    """Per-call and per-kernel timing of a library call `step(i)` on the
    current stream."""

    def __init__(self, lib, torch, hip):
        self.lib, self.torch, self.hip = lib, torch, hip
        self.sptr = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def per_call_us(self, step, steps, warmup=10):
        for i in range(warmup):
            step(i)
        e0, e1 = self.hip.event(), self.hip.event()
        self.torch.cuda.synchronize()
        self.hip.record(e0, self.sptr)
        for i in range(steps):
            step(i)
        self.hip.record(e1, self.sptr)
        self.torch.cuda.synchronize()
        us = self.hip.elapsed_ms(e0, e1) * 1e3 / steps
        self.hip.destroy(e0)
        self.hip.destroy(e1)
        return us

    def per_kernel_us(self, step, steps, names):
        """Mean duration of each kernel of the call (event pairs attached to
        the dispatches); None for a pair that times no kernel."""
        n_ev = 2 * len(names)
        evs = [[self.hip.event() for _ in range(n_ev)] for _ in range(steps)]
        arrs = [(ctypes.c_void_p * n_ev)(*[ctypes.c_void_p(e) for e in row]) for row in evs]
        self.torch.cuda.synchronize()
        for i in range(steps):
            self.lib.ctopk_record_kernel_events(arrs[i], n_ev)
            step(i)
        self.torch.cuda.synchronize()
        per = np.array([[self.hip.elapsed_ms(row[2 * j], row[2 * j + 1]) for j in range(len(names))]
                        for row in evs])
        for row in evs:
            for e in row:
                self.hip.destroy(e)
        return {nm: round(float(per[:, j].mean()) * 1e3, 3) for j, nm in enumerate(names)}


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


def roofline_entry(name, nbytes, us, traffic=True):
    achieved = nbytes / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": read_traffic(name) if traffic else None, "kernel": name,
            "algorithmic_bytes_per_launch": int(round(nbytes)), "avg_launch_us": us}


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


def to_dev(torch, x):
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def unpack_bits(words, n):
    w = words.cpu().numpy().astype(np.int32).view(np.uint8)
    return np.unpackbits(w.reshape(words.shape[0], -1), axis=1, bitorder="little")[:, :n].astype(bool)


# ---------------------------------------------------------------------------
# decode legs
# ---------------------------------------------------------------------------
def decode_leg(ct, lib, torch, timer, ins, eps, steps, warmup, wall=False, kernel_events=True):
    """One decode workload at one eps: `ins` is a list of rotating input sets
    (q, K, V, head_scale or None) on the device.  Returns per-call time,
    query-heads/s, per-kernel times, the plan, mean k/n, the V-union and the
    rooflines of the kernels with algorithmic bytes."""
    q0, K0, V0, _ = ins[0]
    n_q, d = q0.shape
    n_kv, n, _ = K0.shape
    G = n_q // n_kv
    out = torch.empty((n_q, d), dtype=torch.float32, device="cuda")
    k_eps = torch.empty(n_q, dtype=torch.int32, device="cuda")
    tau = torch.empty(n_q, dtype=torch.float64, device="cuda")
    union, kmean = [], []
    for (q, K, V, hs) in ins:
        res = ct.ctopk_certify_ex(q, K, V, eps, head_scale=hs, want_mask=True)
        torch.cuda.synchronize()
        bits = unpack_bits(res["sel_mask"], n)
        union.append(int(bits.reshape(n_kv, G, n).any(axis=1).sum()))
        kmean.append(float(res["k_eps"].double().mean().item()) / n)
        del res, bits
    args = [ct.make_args(q, K, V, eps, head_scale=hs, out=out, k_eps=k_eps, tau=tau)
            for (q, K, V, hs) in ins]
    plan = ct.ctopk_plan(args[0])
    names = KERNELS_BY_PLAN[plan]
    sptr = timer.sptr
    call = lib.ctopk_certify_ex
    sets = len(ins)

    def step(i):
        rc = call(ctypes.byref(args[i % sets]), sptr)
        if rc != 0:
            raise RuntimeError(ct.ctopk_last_error_string())

    res = {"eps": eps, "plan": PLAN_NAMES.get(plan, plan), "rotating_sets": sets}
    if wall:
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) * 1e6 / steps
        res["timing"] = "wall clock between device synchronisations"
    else:
        us = timer.per_call_us(step, steps, warmup)
        res["timing"] = "HIP events around the loop"
    k_bytes = n_kv * n * d * K0.element_size()
    v_bytes = float(np.mean(union)) * d * V0.element_size()
    res.update({"steps": steps, "us_per_call": round(us, 3),
                "query_heads_per_s": round(n_q / (us * 1e-6), 1),
                "hbm_gbps_end_to_end": round((k_bytes + v_bytes) / (us * 1e-6) / 1e9, 1),
                "hbm_frac_end_to_end": round((k_bytes + v_bytes) / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
                "bytes_per_call": {"K": k_bytes, "V_union": int(round(v_bytes))},
                "v_union_fraction": round(v_bytes / (n_kv * n * d * V0.element_size()), 4),
                "mean_k_over_n": round(float(np.mean(kmean)), 4)})
    if kernel_events:
        kern = timer.per_kernel_us(step, steps, names)
        if n <= 32768:
            kern["hist0"] = None  # no level-0 kernel is launched for register rows
        res["kernel_us"] = kern
        algo = {"score_scan": k_bytes, V_KERNEL[plan]: v_bytes}
        rl = {nm: roofline_entry(nm, b, kern[nm]) for nm, b in algo.items() if kern.get(nm)}
        res["rooflines"] = rl
        res["roofline"] = max(rl.values(), key=lambda r: r["avg_launch_us"]) if rl else None
        res["overhead_kernels_us"] = {nm: v for nm, v in kern.items() if nm not in algo and v}
    return res


def single_query_leg(ct, lib, torch, timer, steps):
    """C0: one fp32 head, n = 1024, d = 64, scale 0.25: latency per call."""
    wl = workloads.single_query()
    q, K, V, hs = (to_dev(torch, wl[k]) for k in ("q", "K", "V", "head_scale"))
    out = torch.empty((1, 64), dtype=torch.float32, device="cuda")
    k_eps = torch.empty(1, dtype=torch.int32, device="cuda")
    tau = torch.empty(1, dtype=torch.float64, device="cuda")
    args = ct.make_args(q, K, V, 0.01, head_scale=hs, out=out, k_eps=k_eps, tau=tau)
    plan = ct.ctopk_plan(args)
    names = KERNELS_BY_PLAN[plan]

    def step(i):
        rc = lib.ctopk_certify_ex(ctypes.byref(args), timer.sptr)
        if rc != 0:
            raise RuntimeError(ct.ctopk_last_error_string())

    us = timer.per_call_us(step, steps, 20)
    kern = timer.per_kernel_us(step, min(steps, 200), names)
    if "hist0" in kern:
        kern["hist0"] = None
    return {"workload": "single query: 1 head, n=1024, d=64, fp32, scale 0.25", "eps": 0.01,
            "plan": PLAN_NAMES.get(plan, plan), "steps": steps, "us_per_call": round(us, 3),
            "kernel_us": kern, "k_eps": int(k_eps.item())}


def bound_leg(ct, lib, torch, timer, ins, steps, eps):
    """The decode workload certified by the blockwise bound (CTOPK_FLAG_BOUND):
    per-call time, per-kernel times and the keys kept."""
    n_q, d = ins[0][0].shape
    n = ins[0][1].shape[1]
    out = torch.empty((n_q, d), dtype=torch.float32, device="cuda")
    k_eps = torch.empty(n_q, dtype=torch.int32, device="cuda")
    tau = torch.empty(n_q, dtype=torch.float64, device="cuda")
    args = [ct.make_args(q, K, V, eps, out=out, k_eps=k_eps, tau=tau, flags=ct.CTOPK_FLAG_BOUND)
            for (q, K, V, _) in ins]
    assert ct.ctopk_plan(args[0]) == ct.CTOPK_PLAN_DECODE_BOUND
    names = KERNELS_BY_PLAN[ct.CTOPK_PLAN_DECODE_BOUND]
    sets = len(ins)

    def step(i):
        rc = lib.ctopk_certify_ex(ctypes.byref(args[i % sets]), timer.sptr)
        if rc != 0:
            raise RuntimeError(ct.ctopk_last_error_string())

    kmean, taumax = [], 0.0
    for i in range(sets):
        step(i)
        torch.cuda.synchronize()
        kmean.append(float(k_eps.double().mean().item()))
        taumax = max(taumax, float(tau.max().item()))
    us = timer.per_call_us(step, steps, 20)
    kern = timer.per_kernel_us(step, steps, names)
    kern["hist0"] = None
    return {"eps": eps, "steps": steps, "us_per_call": round(us, 3),
            "query_heads_per_s": round(n_q / (us * 1e-6), 1), "kernel_us": kern,
            "mean_k_over_n": round(float(np.mean(kmean)) / n, 4), "max_tau": taumax,
            "bound_kernel_traffic_bytes": read_traffic("bound")}


def k4_leg(ct, lib, torch, timer, hip, ins, T_cut, T_top, steps):
    """The 4-bit key copy on the decode inputs: exact candidate generation
    (ctopk_candidates_k4) at two thresholds per head -- the certified cut
    score (candidates = the exact head) and the 64th largest score (a
    retrieval-sized set) -- with per-kernel times, keys rescored at full
    width, and the scan's bytes against the full-width score scan's."""
    sets = len(ins)
    n_q, d = ins[0][0].shape
    n_kv, n, _ = ins[0][1].shape
    copies = [ct.ctopk_quantize_k4(K) for (_, K, _, _) in ins]
    torch.cuda.synchronize()
    ev0, ev1 = hip.event(), hip.event()
    hip.record(ev0, timer.sptr)
    for (_, K, _, _) in ins:
        ct.ctopk_quantize_k4(K)
    hip.record(ev1, timer.sptr)
    torch.cuda.synchronize()
    quant_us = hip.elapsed_ms(ev0, ev1) * 1e3 / sets
    hip.destroy(ev0)
    hip.destroy(ev1)
    mask = torch.empty((n_q, (n + 31) // 32), dtype=torch.int32, device="cuda")
    count = torch.empty(n_q, dtype=torch.int32, device="cuda")
    resc = torch.empty(n_kv, dtype=torch.int32, device="cuda")
    names = ("k4_scan", "k4_rescore")
    out = {"quantize_us_per_call": round(quant_us, 3),
           "scan_bytes_per_call": n_kv * n * (d // 2 + 8),
           "full_width_scan_bytes": n_kv * n * d * 2}
    for label, Ts in (("cut_score", T_cut), ("top64", T_top)):
        thr = [torch.from_numpy(np.ascontiguousarray(t, dtype=np.float32)).cuda() for t in Ts]
        args = [ct.make_k4_args(ins[r][0], ins[r][1], *copies[r], thr[r], sel_mask=mask,
                                count=count, rescored=resc) for r in range(sets)]

        def step(i):
            rc = lib.ctopk_candidates_k4(ctypes.byref(args[i % sets]), timer.sptr)
            if rc != 0:
                raise RuntimeError(ct.ctopk_last_error_string())

        fr, cnt = [], []
        for r in range(sets):
            step(r)
            torch.cuda.synchronize()
            fr.append(float(resc.double().sum().item()) / (n_kv * n))
            cnt.append(float(count.double().mean().item()))
        us = timer.per_call_us(step, steps, 20)
        kern = timer.per_kernel_us(step, steps, names)
        scan_gbps = out["scan_bytes_per_call"] / (kern["k4_scan"] * 1e-6) / 1e9
        out[label] = {"us_per_call": round(us, 3), "kernel_us": kern,
                      "mean_candidates": round(float(np.mean(cnt)), 1),
                      "rescored_fraction": round(float(np.mean(fr)), 4),
                      "k4_scan_roofline": roofline_entry("k4_scan", out["scan_bytes_per_call"],
                                                         kern["k4_scan"]),
                      "bytes_per_call": round(out["scan_bytes_per_call"]
                                              + float(np.mean(fr)) * n_kv * n * d * 2)}
    return out


def logits_leg(ct, lib, torch, timer, steps, eps):
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
    vp = ctypes.c_void_p
    argv = (vp(L.data_ptr()), vp(V.data_ptr()), ct.CTOPK_F32, n, dv, rows, 1, float(eps), None, 0,
            timer.sptr, vp(out.data_ptr()), vp(k_eps.data_ptr()), vp(tau.data_ptr()), None, None)

    def step(i):
        rc = lib.ctopk_certify_logits(*argv)
        if rc != 0:
            raise RuntimeError(ct.ctopk_last_error_string())

    step(0)
    torch.cuda.synchronize()
    kmean = float(k_eps.double().mean().item()) / n
    us = timer.per_call_us(step, steps, 3)
    kern = timer.per_kernel_us(step, steps, ("resolve", "vsum", "finalize"))
    lbytes = rows * n * 4
    return {"workload": "logit sweep: 1024 rows x 65536 fp32 logits, sigma=2, shared fp32 V [65536, 64]",
            "eps": eps, "steps": steps, "us_per_call": round(us, 3),
            "rows_per_s": round(rows / (us * 1e-6), 1), "kernel_us": kern,
            "select_roofline": roofline_entry("resolve", lbytes, kern["resolve"], traffic=False),
            "mean_k_over_n": round(kmean, 4)}


def design_rule_leg(ct, torch, seed=4004):
    """k_eps / n on the device against the Abstract's Gaussian design rule
    Phi_c(sigma + Phi^{-1}(eps)) for every (sigma, n, eps) of the logit sweep:
    1024 rows of iid N(0, sigma^2) fp32 logits per cell, drawn on the device
    from a seeded generator (the host generator takes ~20 s per 4 GiB), one
    shared fp32 V [n, 64]."""
    import oracle
    gen = torch.Generator(device="cuda")
    table = []
    for n in workloads.LOGIT_NS:
        gen.manual_seed(seed + n)
        V = torch.randn((1, n, 64), generator=gen, device="cuda", dtype=torch.float32)
        for sigma in workloads.LOGIT_SIGMAS:
            L = torch.randn((1024, n), generator=gen, device="cuda", dtype=torch.float32)
            L.mul_(sigma)
            for eps in workloads.LOGIT_EPS:
                res = ct.ctopk_certify_logits(L, V, eps)
                torch.cuda.synchronize()
                kn = res["k_eps"].double().cpu().numpy() / n
                pred = oracle.gaussian_design_rule(sigma, eps)
                table.append({"sigma": sigma, "n": n, "eps": eps, "k_over_n": round(float(kn.mean()), 5),
                              "sd": round(float(kn.std()), 5), "rule": round(pred, 5),
                              "gap": round(float(kn.mean()) - pred, 5)})
            del L
        del V
        torch.cuda.empty_cache()
    return {"rows": 1024, "cells": table}


def encoder_leg(ct, lib, torch, timer, steps, eps, sets=16):
    """All-queries (encoder-shaped) workload: batch 8, 12 heads, 512 queries and
    512 keys per head, d = 64, bf16, per-head temperature; every query row of a
    head is one certified row.  Rotates over `sets` input sets (16 x 18.9 MB,
    above the 256 MB Infinity Cache)."""
    wls = [workloads.encoder(rotation=r) for r in range(sets)]
    w0 = wls[0]
    n, d, n_q, n_kv = w0["n"], w0["d"], w0["n_q_heads"], w0["n_kv_heads"]
    ins = [tuple(to_dev(torch, w[k]) for k in ("q", "K", "V", "head_scale")) for w in wls]
    del wls
    out = torch.empty((n_q, d), dtype=torch.float32, device="cuda")
    k_eps = torch.empty(n_q, dtype=torch.int32, device="cuda")
    tau = torch.empty(n_q, dtype=torch.float64, device="cuda")
    args = [ct.make_args(q, K, V, eps, head_scale=hs, out=out, k_eps=k_eps, tau=tau)
            for (q, K, V, hs) in ins]

    def step(i):
        rc = lib.ctopk_certify_ex(ctypes.byref(args[i % sets]), timer.sptr)
        if rc != 0:
            raise RuntimeError(ct.ctopk_last_error_string())

    kmean = []
    for i in range(sets):
        step(i)
        torch.cuda.synchronize()
        kmean.append(float(k_eps.double().mean().item()))
    kern_us = timer.per_kernel_us(step, steps, ("encoder",))["encoder"]
    us = timer.per_call_us(step, steps, 20)
    in_bytes = 3 * n_kv * n * d * 2
    qk_flops = 2.0 * n_kv * (n_q // n_kv) * n * d
    return {"workload": "encoder batch 8 x 12 heads, 512 queries x 512 keys, d=64, bf16",
            "eps": eps, "steps": steps, "rotating_sets": sets,
            "us_per_call": round(us, 3), "kernel_us": round(kern_us, 3),
            "query_rows_per_s": round(n_q / (us * 1e-6), 1),
            "qk_flops_per_call": qk_flops,
            "qk_tflops_over_kernel": round(qk_flops / (kern_us * 1e-6) / 1e12, 2),
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
    ap.add_argument("--legs", default="eps01,single,long,bound,logits,k4,encoder,rule",
                    help="comma list of extra legs to run after the headline (empty: none)")
    ap.add_argument("--leg-steps", type=int, default=500, help="calls per extra decode leg")
    args = ap.parse_args()
    legs = {x for x in args.legs.split(",") if x}

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "every GPU box here has one GPU.  The decode path shards by KV head with no "
              "exchange, so each GPU would run this same one-GPU step on its own heads.",
              file=sys.stderr)
        sys.exit(2)

    t_gen = time.perf_counter()
    sets = [workloads.gqa_decode(rotation=r) for r in range(args.sets)]
    wl0 = sets[0]
    n, d, n_q, n_kv = wl0["n"], wl0["d"], wl0["n_q_heads"], wl0["n_kv_heads"]
    log(f"generated {args.sets} input sets in {time.perf_counter() - t_gen:.1f} s")

    cpu = None
    if not args.no_cpu:
        log(f"CPU baseline (~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline(wl0, args.eps, args.cpu_seconds)

    import torch
    import certified_top_sparse_amd as ct

    lib = ct.load()
    hip = Hip()
    torch.cuda.set_device(0)
    timer = Timer(lib, torch, hip)

    ins = [(to_dev(torch, s["q"]), to_dev(torch, s["K"]), to_dev(torch, s["V"]), None)
           for s in sets]
    eps = float(args.eps)

    # Headline: exactly `steps` ctopk_certify calls, wall clock between device
    # synchronisations.
    out = torch.empty((n_q, d), dtype=torch.float32, device="cuda")
    k_eps = torch.empty(n_q, dtype=torch.int32, device="cuda")
    tau = torch.empty(n_q, dtype=torch.float64, device="cuda")
    vp = ctypes.c_void_p
    ptrs = [(vp(q.data_ptr()), vp(K.data_ptr()), vp(V.data_ptr())) for (q, K, V, _) in ins]
    op, kep, tp = vp(out.data_ptr()), vp(k_eps.data_ptr()), vp(tau.data_ptr())
    sptr = timer.sptr

    def step(i):
        qp, kp, vvp = ptrs[i % args.sets]
        rc = lib.ctopk_certify(qp, kp, vvp, n, d, n_q, n_kv, eps, sptr, op, kep, tp)
        if rc != 0:
            raise RuntimeError(ct.ctopk_last_error_string())

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    value = n_q * args.steps / wall
    log(f"headline: {ms_per_step * 1e3:.2f} us per step")

    # The same workload, instrumented: per-kernel times, V-union, rooflines.
    head = decode_leg(ct, lib, torch, timer, ins, eps, args.steps, 20,
                      kernel_events=not args.no_kernel_events)
    k_bytes = head["bytes_per_call"]["K"]
    v_bytes = head["bytes_per_call"]["V_union"]

    extra = {}
    if "eps01" in legs:
        log("decode eps=0.1")
        extra["decode_eps_0.1"] = decode_leg(ct, lib, torch, timer, ins, 0.1, args.leg_steps, 20)
    if "single" in legs:
        log("single query")
        extra["single_query"] = single_query_leg(ct, lib, torch, timer, 2000)
    if "bound" in legs:
        log("bound")
        extra["bound_certificate"] = bound_leg(ct, lib, torch, timer, ins, args.leg_steps, eps)
    if "k4" in legs:
        log("k4")
        T_cut, T_top = [], []
        for (q, K, V, _) in ins:
            res = ct.ctopk_certify_ex(q, K, V, eps, want_mask=True, want_scores=True)
            torch.cuda.synchronize()
            bits = unpack_bits(res["sel_mask"], n)
            sc = res["scores"].cpu().numpy()
            T_cut.append(np.array([sc[h][bits[h]].min() for h in range(n_q)], dtype=np.float32))
            T_top.append(np.sort(sc, axis=1)[:, -64].astype(np.float32))
        extra["k4_candidates"] = k4_leg(ct, lib, torch, timer, hip, ins, T_cut, T_top,
                                        args.leg_steps)
    stream_gbps = copy_stream_gbps(torch, [K for (_, K, _, _) in ins])
    del ins, ptrs
    torch.cuda.empty_cache()
    if "long" in legs:
        log("long decode")
        wl = workloads.long_decode(batch=4)
        lins = [tuple(to_dev(torch, wl[k]) for k in ("q", "K", "V", "head_scale"))]
        del wl
        ld = {"workload": "long_decode batch 4: 128 query / 32 KV heads, n=131072, d=128, bf16"}
        for e in (0.01, 0.1):
            ld[f"eps_{e}"] = decode_leg(ct, lib, torch, timer, lins, e, 40, 5)
        extra["long_decode"] = ld
        del lins
        torch.cuda.empty_cache()
    if "logits" in legs:
        log("logits")
        extra["logits_select"] = logits_leg(ct, lib, torch, timer, 20, eps)
        torch.cuda.empty_cache()
    if "encoder" in legs:
        log("encoder")
        extra["encoder"] = encoder_leg(ct, lib, torch, timer, args.leg_steps, eps)
        torch.cuda.empty_cache()
    if "rule" in legs:
        log("design rule table")
        extra["design_rule"] = design_rule_leg(ct, torch)

    e2e_gbps = (k_bytes + v_bytes) / (ms_per_step * 1e-3) / 1e9
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
        "roofline": head.get("roofline"),
        "rooflines": head.get("rooflines"),
        "cpu_baseline": cpu,
        "hbm_gbps_end_to_end": round(e2e_gbps, 1),
        "hbm_frac_end_to_end": round(e2e_gbps / PEAK_HBM_GBPS, 4),
        "copy_stream_gbps": round(stream_gbps, 1),
        "bytes_per_step": head["bytes_per_call"],
        "v_union_fraction": head["v_union_fraction"],
        "mean_k_over_n": head["mean_k_over_n"],
        "plan": head["plan"],
        "kernel_us": head.get("kernel_us"),
        "overhead_kernels_us": head.get("overhead_kernels_us"),
        "us_per_call_events": head["us_per_call"],
    }
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
