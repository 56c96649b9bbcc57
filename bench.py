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
the dominant kernel (the score scan): algorithmic bytes = the K bytes of one
call divided by its average duration, timed live with HIP events recorded by
the library at its stage boundaries inside the timed region.
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
STAGES = ("score_scan", "histogram", "select", "value_stream")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "score_scan_gqa_decode_n32768_pmc.md")
SCAN_SOURCE = os.path.join(ROOT, "certified_top_sparse_amd", "csrc", "score_scan.hip")


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


def source_digest(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic():
    """HBM bytes per score-scan dispatch from the committed rocprofv3 --pmc
    summary, if it was taken on the current score-scan source."""
    try:
        with open(PMC_SUMMARY) as f:
            text = f.read()
    except OSError:
        return None
    m = re.search(r"```json\s*(\{.*?\})\s*```", text, re.S)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("score_scan_source_sha256_16") != source_digest(SCAN_SOURCE):
        return None
    return d.get("traffic_bytes_per_dispatch")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--eps", type=float, default=0.01)
    ap.add_argument("--sets", type=int, default=6, help="rotating input sets (128 MiB each)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline leg")
    ap.add_argument("--no-stage-events", action="store_true")
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
    kmean = []
    for r in range(args.sets):
        res = ct.ctopk_certify_ex(Q[r], Kd[r], Vd[r], args.eps, want_mask=True)
        torch.cuda.synchronize()
        words = res["sel_mask"].cpu().numpy().astype(np.int32).view(np.uint8)
        bits = np.unpackbits(words.reshape(n_q, -1), axis=1, bitorder="little")[:, :n].astype(bool)
        union_rows.append(int(bits.reshape(n_kv, G, n).any(axis=1).sum()))
        kmean.append(float(res["k_eps"].double().mean().item()))
    k_bytes = n_kv * n * d * 2
    v_bytes = float(np.mean(union_rows)) * d * 2

    # A plain copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters.
    src = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst

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

    # Instrumented pass over the same steps: the library records HIP events on
    # the call's stream at its stage boundaries (each record costs a few
    # microseconds, so this pass is not the headline figure).
    n_ev = len(STAGES) + 1
    stage_us = {}
    scan_us = None
    ms_events = None
    if not args.no_stage_events:
        evs = [[hip.event() for _ in range(n_ev)] for _ in range(args.steps)]
        arm = lib.ctopk_record_stage_events
        ev_arrays = [(ctypes.c_void_p * n_ev)(*[ctypes.c_void_p(e) for e in row]) for row in evs]
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(args.steps):
            arm(ev_arrays[i], n_ev)
            step(i)
        torch.cuda.synchronize()
        ms_events = (time.perf_counter() - t1) * 1e3 / args.steps
        per = np.array([[hip.elapsed_ms(row[j], row[j + 1]) for j in range(n_ev - 1)]
                        for row in evs])
        for j, name in enumerate(STAGES):
            stage_us[name] = round(float(per[:, j].mean()) * 1e3, 3)
        scan_us = float(per[:, 0].mean()) * 1e3
        for row in evs:
            for e in row:
                hip.destroy(e)

    roofline = None
    if scan_us:
        achieved = k_bytes / (scan_us * 1e-6) / 1e9
        traffic = read_traffic()
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                    "traffic": traffic, "kernel": "score_scan_kernel<bf16,128,4>",
                    "algorithmic_bytes_per_launch": k_bytes,
                    "avg_launch_us": round(scan_us, 3)}

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
        "roofline": roofline,
        "cpu_baseline": cpu,
        "hbm_gbps_end_to_end": round(e2e_gbps, 1),
        "hbm_frac_end_to_end": round(e2e_gbps / PEAK_HBM_GBPS, 4),
        "bytes_per_step": {"K": k_bytes, "V_union": round(v_bytes)},
        "v_union_fraction": round(v_bytes / k_bytes, 4),
        "mean_k_eps": round(float(np.mean(kmean)), 1),
        "stage_us": stage_us,
        "ms_per_step_with_stage_events": None if ms_events is None else round(ms_events, 5),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
