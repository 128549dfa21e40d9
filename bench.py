#!/usr/bin/env python3
"""Benchmark of the polynomial-sketch hot path on one MI355X.

One step = the whole hot path over one batch of synthetic input of the workload:
reset, ingest every key through sketch_update in the workload's chunks (and the
sub-stream merges), answer all m queries with sketch_query, and run exact_attend
for the same queries (the exact path that measures the sketch's error).

Printed: one JSON line.  ``value`` = (keys ingested + queries answered) per
second of the whole step; the line also carries the per-phase rates, the
roofline of the dominant kernel (the moment update, fp32 MFMA) and the float64
oracle timed on a bounded sample on the host cores.
"""

import argparse
import json
import math
import os
import sys
import time

METRIC = "sketch keys/s + queries/s (MFMA % of peak); exact-path HBM GB/s"
PEAK_FP32_MFMA = 157.3e12
PEAK_HBM = 8.0e12


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", type=int, default=4,
                    help="workload id 1..5 (default 4: 32 heads, d=64, p=2, 128K keys each)")
    ap.add_argument("--quick", action="store_true",
                    help="only the chosen workload (no workload-3 sub-object, no "
                         "per-configuration errors)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the oracle CPU baseline (0 disables it)")
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--layout", choices=["full", "sym"], default="full",
                    help="storage layout of the sketches in the --counters sequence")
    ap.add_argument("--counters", action="store_true",
                    help="short fixed sequence for rocprofv3 --pmc passes: a 1 GiB "
                         "device copy, one pass of the update calls, 3 decode passes")
    return ap.parse_args()


# The sources a kernel's committed traffic counters depend on: the kernel itself
# and the host file that picks its launch shape (split counts, slices).
KERNEL_SOURCES = {
    "sk_update_kernel": ["sk_update.h", "sk_common.h", "sk_elementwise.h", "sk_reduce.h",
                         "expsketch.hip"],
    "sk_update_kr_kernel": ["sk_update_kr.h", "sk_update_kr.hip", "sk_common.h", "sk_reduce.h",
                            "expsketch.hip"],
    "sk_exact_decode": ["sk_exact.h", "sk_common.h", "expsketch.hip"],
}


def exact_batched_kernel(w):
    """The library's choice of batched exact kernel for this shape (m > 8)."""
    if max(w.d, w.dv) < 16:
        return "sk_exact_tiled (VALU)"
    if w.dv == 16 and 16 <= w.d <= 64 and os.environ.get("EXPSKETCH_EXACT_MFMA16", "1") != "0":
        return "sk_exact_mfma16"
    return "sk_exact_mfma"


def source_hash(kernel):
    import hashlib
    root = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "exp_density_sketching_amd", "csrc")
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(root, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source (else None)."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        f"traffic__{kernel}__{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != source_hash(kernel):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, K, V, Q, budget):
    """The float64 oracle as it stands, on a bounded sample of the workload."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    K0, V0, Q0 = K[0], V[0], Q[0]
    # keys: the moment route on a prefix, grown until a third of the budget is used
    nk, t_u = 256, 0.0
    while True:
        t0 = time.perf_counter()
        oracle.MomentSketch(w.d, w.dv, w.p).update(K0[:nk], V0[:nk], chunk=64)
        t_u = time.perf_counter() - t0
        if t_u > budget / 3 or nk >= w.n:
            break
        nk = min(w.n, nk * 2)
    sk = oracle.MomentSketch(w.d, w.dv, w.p).update(K0[:256], V0[:256], chunk=64)
    mq = min(w.m, 64)
    t0 = time.perf_counter()
    sk.query(Q0[:mq])
    t_q = time.perf_counter() - t0
    me = min(w.m, 32)
    t0 = time.perf_counter()
    oracle.exact_attention(K0, V0, Q0[:me])
    t_e = time.perf_counter() - t0
    per_key, per_q, per_eq = t_u / nk, t_q / mq, t_e / me
    t_full = w.h * (w.n * per_key + w.m * (per_q + per_eq))
    return {
        "value": w.h * (w.n + w.m) / t_full,
        "unit": "keys+queries/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"head 0: moment-route update of {nk} keys ({t_u:.1f} s), "
                   f"moment-route query of {mq} queries ({t_q:.2f} s), exact path for "
                   f"{me} queries over all {w.n} keys ({t_e:.2f} s); projected to the "
                   f"whole step of {w.h} head(s)"),
        "keys_per_s": 1.0 / per_key,
        "queries_per_s": 1.0 / per_q,
    }


def state_floats(w, layout):
    """Floats of one head's stored moments (the layout's blocks)."""
    if layout == "full":
        return (w.D - 1) + w.D * w.dv
    top = math.comb(w.d + w.p - 1, w.p)
    lower = math.comb(w.d + w.p, w.p) - top
    return lower * (w.d + w.dv) + top * w.dv


def exact_decode_hbm(w4, E, torch, steps):
    """The exact path in decode mode (one query per head over the whole KV) on the
    32-head workload, whose 2 GiB of keys and values exceed the 256 MB Infinity
    Cache, so the figure is HBM bandwidth.  Inputs are drawn on the GPU (seeded
    torch generator) from that workload's distributions: keys and queries
    Gaussian clipped to norm key_r, values standard normal."""
    g = torch.Generator(device="cuda")
    g.manual_seed(4)

    def clipped(shape):
        x = torch.randn(shape, device="cuda", generator=g)
        return x * torch.clamp(w4.key_r / x.norm(dim=-1, keepdim=True), max=1.0)

    K = clipped((w4.h, w4.n, w4.d))
    V = torch.randn((w4.h, w4.n, w4.dv), device="cuda", generator=g)
    q1 = clipped((w4.h, 1, w4.d))
    out = torch.empty((w4.h, 1, w4.dv), device="cuda")
    Z = torch.empty((w4.h, 1), device="cuda")
    for _ in range(2):
        E.exact_attend(K, V, q1, out, Z)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        E.exact_attend(K, V, q1, out, Z)
    b.record()
    torch.cuda.synchronize()
    t = a.elapsed_time(b) / 1e3 / steps
    kv = 4.0 * w4.h * w4.n * (w4.d + w4.dv)
    del K, V
    torch.cuda.empty_cache()
    return {"workload": w4.name, "us_per_step": t * 1e6, "kv_bytes": kv,
            "GBps": kv / t / 1e9, "frac_of_hbm_peak": kv / t / PEAK_HBM,
            "data": "synthetic, drawn on the GPU"}


def decode_steps(w, E, torch, Kg, Vg, Qg, steps, exact_us):
    """sketch_step on a sketch holding the whole stream: one key/value appended
    and one query answered per head and step.  Algorithmic traffic: one read and
    one write of the stored moments per step."""
    import numpy as np
    res = {}
    for layout in ("full", "sym"):
        sk = E.sketch_create(w.d, w.dv, w.p, w.h, layout)
        step_n = w.chunk or w.n                  # the workload's own update calls
        for c0 in range(0, w.n, step_n):
            E.sketch_update(sk, Kg[:, c0:c0 + step_n], Vg[:, c0:c0 + step_n])
        cnt = max(steps, 3)                      # 3 warm-up steps
        ks = [Kg[:, i].contiguous() for i in range(cnt)]
        vs = [Vg[:, i].contiguous() for i in range(cnt)]
        qs = [Qg[:, i % w.m].contiguous() for i in range(cnt)]
        out = torch.empty((w.h, w.dv), device="cuda")
        z = torch.empty((w.h,), device="cuda")
        for i in range(3):
            E.sketch_step(sk, ks[i], vs[i], qs[i], out, z)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(steps):
            E.sketch_step(sk, ks[i], vs[i], qs[i], out, z)
        b.record()
        torch.cuda.synchronize()
        # the step kernel's own time, in a second pass (its events add to the step)
        E.sketch_timing(sk, True)
        for i in range(steps):
            E.sketch_step(sk, ks[i], vs[i], qs[i], out, z)
        torch.cuda.synchronize()
        kern = E.sketch_kernel_times(sk, "step")
        E.sketch_timing(sk, False)
        sk.destroy()
        t = a.elapsed_time(b) / 1e3 / steps
        tk = float(np.mean(kern)) / 1e3
        nbytes = 2.0 * 4 * w.h * state_floats(w, layout)
        res[layout] = {"us_per_step": t * 1e6, "kernel_us": tk * 1e6,
                       "state_bytes": nbytes / 2, "kernel_GBps": nbytes / tk / 1e9,
                       "speedup_vs_exact_decode": exact_us / (t * 1e6)}
    res["steps"] = steps
    res["resident"] = "cache (state <= 256 MB)"
    return res


def counters_pass(w, E, torch, generate, layout="full"):
    """Fixed sequence for counter passes: copy of known size, update, query, decode."""
    from exp_density_sketching_amd.workload import ingest
    nbytes = 1 << 30
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    K, V, Q = generate(w)
    Kg = torch.from_numpy(K).cuda()
    Vg = torch.from_numpy(V).cuda()
    S = max(1, w.substreams)
    sketches = [E.sketch_create(w.d, w.dv, w.p, w.h, layout) for _ in range(S)]
    ingest(w, Kg, Vg, sketches)
    ukern = E.UPDATE_KERNELS[E.sketch_update_path(sketches[0])]
    Qg = torch.from_numpy(Q).cuda()
    for _ in range(3):
        E.sketch_query(sketches[0], Qg)
    q1 = torch.from_numpy(Q[:, :1].copy()).cuda()
    for _ in range(3):
        E.exact_attend(Kg, Vg, q1)
    torch.cuda.synchronize()
    for sk in sketches:
        sk.destroy()
    print(json.dumps({"counters_pass": w.name, "layout": layout, "copy_bytes": nbytes,
                      "copies": 3,
                      "update_kernel": ukern,
                      "update_sources": source_hash(ukern) if ukern in KERNEL_SOURCES else None,
                      "decode_sources": source_hash("sk_exact_decode"),
                      "kv_bytes": 4 * w.h * w.n * (w.d + w.dv)}), flush=True)
    return 0


def measure_workload(w, E, torch, K, V, Q, args, full_line=True):
    """Warm-up and timed steps of workload w (full layout), the per-call update
    time, the exact path in decode mode and the sketch-vs-exact error.  With
    full_line, also the multiset layout and the decode step."""
    import numpy as np
    from exp_density_sketching_amd.workload import ingest
    Kg = torch.from_numpy(K).cuda()
    Vg = torch.from_numpy(V).cuda()
    Qg = torch.from_numpy(Q).cuda()
    out_s = torch.empty((w.h, w.m, w.dv), device="cuda")
    z_s = torch.empty((w.h, w.m), device="cuda")
    out_e = torch.empty_like(out_s)
    z_e = torch.empty_like(z_s)
    S = max(1, w.substreams)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    n_calls = sum(-(-(w.n * (i + 1) // S - w.n * i // S) // (w.chunk or w.n))
                  for i in range(S))
    chunk = w.chunk or -(-w.n // S)
    keys_per_call = float(np.mean([min(chunk, w.n // S - c0)
                                   for c0 in range(0, w.n // S, chunk)]))

    def measure(layout):
        """Warm-up and timed steps with sketches of the given storage layout."""
        sketches = [E.sketch_create(w.d, w.dv, w.p, w.h, layout) for _ in range(S)]

        def step(rec):
            for sk in sketches:
                E.sketch_reset(sk)
            e0, e1, e2, e3 = ev(), ev(), ev(), ev()
            e0.record()
            ingest(w, Kg, Vg, sketches)
            e1.record()
            E.sketch_query(sketches[0], Qg, out_s, z_s)
            e2.record()
            E.exact_attend(Kg, Vg, Qg, out_e, z_e)
            e3.record()
            rec.append((e0, e1, e2, e3))

        warm = []
        for _ in range(args.warmup):
            step(warm)
        torch.cuda.synchronize()
        for sk in sketches:          # library events around the update/query kernels
            E.sketch_timing(sk, True)
        rec = []
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step(rec)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        r = {"sketches": sketches, "t_step": wall / args.steps,
             "t_upd": np.mean([a.elapsed_time(b) for a, b, _, _ in rec]) / 1e3,
             "t_qry": np.mean([b.elapsed_time(c) for _, b, c, _ in rec]) / 1e3,
             "t_ex": np.mean([c.elapsed_time(d) for _, _, c, d in rec]) / 1e3}
        # the update and query kernels' launches in the timed steps, bracketed by
        # HIP events on the library's stream (sketch_timing)
        upd_ms = [t for sk in sketches for t in E.sketch_kernel_times(sk, "update")]
        qry_ms = E.sketch_kernel_times(sketches[0], "query")
        for sk in sketches:
            E.sketch_timing(sk, False)
        r["dur"] = float(np.mean(upd_ms)) / 1e3
        r["ktime"] = float(np.sum(upd_ms)) / 1e3     # all update launches of the steps
        r["launches"] = len(upd_ms)
        r["t_qk"] = float(np.mean(qry_ms)) / 1e3
        return r

    full = measure("full")
    sketches = full["sketches"]
    ukern = E.UPDATE_KERNELS[E.sketch_update_path(sketches[0])]
    sketch_error = sketch_vs_exact(w, K, Q, z_s, out_s, z_e, out_e)
    tail = coreset_leg(w, E, torch, Kg, Vg, Qg, out_s, z_s, out_e, z_e, max(1, args.steps // 2))
    t_upd, t_qry, t_ex, t_step = full["t_upd"], full["t_qry"], full["t_ex"], full["t_step"]
    dur, t_qk = full["dur"], full["t_qk"]
    flop_per_key = 2.0 * w.D * (1 + w.dv)
    # every key of every timed step went through the update launches (small calls
    # are staged, so a launch may hold several calls' keys): algorithmic flops of
    # all keys / the launches' total time
    keys_timed = float(w.n) * w.h * args.steps
    achieved = flop_per_key * keys_timed / full["ktime"]

    # whole sketch_update calls of one sub-stream, per call: every launch, copy
    # and partial reduction they cause, up to a state that is complete (export)
    sk = sketches[0]
    E.sketch_reset(sk)
    calls = list(range(0, w.n // S, chunk))
    view = E.sketch_export(sk)
    torch.cuda.synchronize()
    a, b = ev(), ev()
    a.record()
    for c0 in calls:
        E.sketch_update(sk, Kg[:, c0:c0 + chunk], Vg[:, c0:c0 + chunk])
    E.sketch_export(sk, view)
    b.record()
    torch.cuda.synchronize()
    call_dur = a.elapsed_time(b) / 1e3 / len(calls)
    del view

    res = {
        "value": w.h * (w.n + w.m) / t_step,
        "unit": "keys+queries/s",
        "ms_per_step": t_step * 1e3,
        "config": {"workload": w.name, "d": w.d, "dv": w.dv, "p": w.p, "D": w.D,
                   "n": w.n, "m": w.m, "heads": w.h, "chunk": w.chunk,
                   "substreams": w.substreams, "update_calls": n_calls},
        "keys_per_s": w.h * w.n / t_upd,
        "queries_per_s": w.h * w.m / t_qry,
        "update_ms": t_upd * 1e3,
        "query_ms": t_qry * 1e3,
        "exact_ms": t_ex * 1e3,
        "query_mfma_frac": flop_per_key * w.h * w.m / t_qry / PEAK_FP32_MFMA,
        "query_kernel_mfma_frac": flop_per_key * w.h * w.m / t_qk / PEAK_FP32_MFMA,
        "query_kernel_us": t_qk * 1e6,
        "update_call_us": call_dur * 1e6,
        "update_call_mfma_frac": flop_per_key * keys_per_call * w.h / call_dur / PEAK_FP32_MFMA,
        "exact_batched": {"ms": t_ex * 1e3, "flop": 2.0 * w.h * w.m * w.n * (w.d + w.dv),
                          "TFLOPs": 2.0 * w.h * w.m * w.n * (w.d + w.dv) / t_ex / 1e12,
                          "mfma_frac": 2.0 * w.h * w.m * w.n * (w.d + w.dv) / t_ex /
                          PEAK_FP32_MFMA,
                          "kernel": exact_batched_kernel(w)},
        "exact_decode": exact_decode(w, E, torch, Kg, Vg, Qg, args.decode_steps),
        "sketch_error": sketch_error,
        "tail_coreset": tail,
        "roofline": {"kernel": ukern, "bound": "mfma",
                     "achieved": achieved / 1e12, "peak": PEAK_FP32_MFMA / 1e12,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_MFMA,
                     "traffic": committed_traffic(ukern, w.name),
                     "flop_per_launch": flop_per_key * keys_timed / full["launches"],
                     "launch_us": dur * 1e6, "launches": full["launches"]},
    }
    for s_ in sketches:
        s_.destroy()
    if not full_line:
        return res
    # the same step with multiset storage of the moments (identical answers,
    # C(d + p, p) rows instead of D); priced at its own algorithmic work
    sym = measure("sym")
    for s_ in sym["sketches"]:
        s_.destroy()
    rows = math.comb(w.d + w.p, w.p)
    sflop = 2.0 * rows * (1 + w.dv)
    s_ach = sflop * keys_timed / sym["ktime"]
    res["sym_layout"] = {
        "value": w.h * (w.n + w.m) / sym["t_step"],
        "ms_per_step": sym["t_step"] * 1e3,
        "rows": rows,
        "keys_per_s": w.h * w.n / sym["t_upd"],
        "queries_per_s": w.h * w.m / sym["t_qry"],
        "update_ms": sym["t_upd"] * 1e3,
        "query_ms": sym["t_qry"] * 1e3,
        "exact_ms": sym["t_ex"] * 1e3,
        "query_kernel_mfma_frac": sflop * w.h * w.m / sym["t_qk"] / PEAK_FP32_MFMA,
        "roofline": {"kernel": "sk_sym_update_kernel", "bound": "mfma",
                     "achieved": s_ach / 1e12, "peak": PEAK_FP32_MFMA / 1e12,
                     "unit": "TFLOP/s", "frac": s_ach / PEAK_FP32_MFMA,
                     "flop_per_launch": sflop * keys_timed / sym["launches"],
                     "launch_us": sym["dur"] * 1e6, "launches": sym["launches"]},
    }
    res["decode_step"] = decode_steps(w, E, torch, Kg, Vg, Qg, args.decode_steps,
                                      res["exact_decode"]["us_per_step"])
    return res


def coreset_leg(w, E, torch, Kg, Vg, Qg, out_s, z_s, out_e, z_e, steps, block=512, c0=0.25):
    """The tail coreset beside the sketch: Merge-and-Reduce ingest of the same
    stream (the workload's calls and sub-stream merges), the tail added to the
    sketch's answers, and the error of head + tail against the exact path."""
    import numpy as np
    S = max(1, w.substreams)
    cs = [E.coreset_create(w.d, w.dv, w.p, w.h, block=block, c0=c0, seed=1) for _ in range(S)]
    bounds = [w.n * i // S for i in range(S + 1)]
    pieces = []
    for i in range(S):
        step = w.chunk if w.chunk > 0 else bounds[i + 1] - bounds[i]
        for c0_ in range(bounds[i], bounds[i + 1], step):
            c1 = min(bounds[i + 1], c0_ + step)
            pieces.append((i, Kg[:, c0_:c1].contiguous(), Vg[:, c0_:c1].contiguous()))
    torch.cuda.synchronize()

    def ingest():
        for c in cs:
            E.coreset_reset(c)
        for i, k, v in pieces:
            E.coreset_update(cs[i], k, v)
        for i in range(1, S):
            E.coreset_merge(cs[0], cs[i])
        # blocks of small calls wait to share launches; info() takes them in, so
        # every reduce of the stream is inside the timed ingest
        cs[0].info()

    ingest()
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    a, b = ev(), ev()
    a.record()
    for _ in range(steps):
        ingest()
    b.record()
    torch.cuda.synchronize()
    t_ing = a.elapsed_time(b) / 1e3 / steps
    pts, cnt, red = cs[0].info()
    out = out_s.clone()
    Z = z_s.clone()
    E.coreset_query(cs[0], Qg, out, Z)
    o2, z2 = out_s.clone(), z_s.clone()
    torch.cuda.synchronize()
    a.record()
    for _ in range(steps):
        E.coreset_query(cs[0], Qg, o2, z2)
    b.record()
    torch.cuda.synchronize()
    t_q = a.elapsed_time(b) / 1e3 / steps
    zc, zex = Z.cpu().double().numpy(), z_e.cpu().double().numpy()
    oc, oex = out.cpu().double().numpy(), out_e.cpu().double().numpy()
    for c in cs:
        c.destroy()
    return {"block": block, "c0": c0, "points_per_head": pts, "reduces": red,
            "ingest_ms": t_ing * 1e3, "keys_per_s": w.h * w.n / t_ing,
            "tail_query_ms": t_q * 1e3, "queries_per_s": w.h * w.m / t_q,
            "error_with_tail": {"z_rel_max": float(np.max(np.abs(zc - zex) / zex)),
                                "o_abs_max": float(np.max(np.abs(oc - oex)))}}


def sketch_vs_exact(w, K, Q, z_s, out_s, z_e, out_e):
    """The sketch's answers against the exact path's on the same queries, and
    the truncation bound rho^(p+1)/(p+1)! e^(2 rho), rho = max|q| max|k| per head."""
    import numpy as np
    zs, ze = z_s.cpu().double().numpy(), z_e.cpu().double().numpy()
    os_, oe = out_s.cpu().double().numpy(), out_e.cpu().double().numpy()
    rho = max(float(np.linalg.norm(K[hd].astype(np.float64), axis=1).max() *
                    np.linalg.norm(Q[hd].astype(np.float64), axis=1).max())
              for hd in range(w.h))
    return {"z_rel_max": float(np.max(np.abs(zs - ze) / ze)),
            "o_abs_max": float(np.max(np.abs(os_ - oe))),
            "z_rel_bound": rho ** (w.p + 1) / math.factorial(w.p + 1) * math.exp(2 * rho),
            "rho": rho}


def exact_decode(w, E, torch, Kg, Vg, Qg, steps):
    """The exact path in decode mode (one query per head), streaming the whole KV:
    algorithmic bytes (d + dv) * 4 per key / time per call, and / the decode
    kernel's own time (median of HIP event pairs around it)."""
    import numpy as np
    dec_out = torch.empty((w.h, 1, w.dv), device="cuda")
    dec_z = torch.empty((w.h, 1), device="cuda")
    q1 = Qg[:, :1].contiguous()
    for _ in range(2):
        E.exact_attend(Kg, Vg, q1, dec_out, dec_z)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        E.exact_attend(Kg, Vg, q1, dec_out, dec_z)
    b.record()
    torch.cuda.synchronize()
    t_dec = a.elapsed_time(b) / 1e3 / steps
    # the decode kernel alone (HIP events around it on the call's stream)
    E.exact_timing(True)
    for _ in range(steps):
        E.exact_attend(Kg, Vg, q1, dec_out, dec_z)
    kern = E.exact_kernel_times()
    E.exact_timing(False)
    t_k = float(np.median(kern)) / 1e3
    kv_bytes = 4.0 * w.h * w.n * (w.d + w.dv)
    hbm = kv_bytes > 256e6
    return {"us_per_step": t_dec * 1e6, "GBps": kv_bytes / t_dec / 1e9,
            "kv_bytes": kv_bytes,
            "frac_of_hbm_peak": kv_bytes / t_dec / PEAK_HBM if hbm else None,
            "kernel_us": t_k * 1e6, "kernel_GBps": kv_bytes / t_k / 1e9,
            "kernel_frac_of_hbm_peak": kv_bytes / t_k / PEAK_HBM if hbm else None,
            "resident": "HBM" if hbm else "cache (<= 256 MB): effective GB/s"}


def error_of_config(w, E, torch, generate, decode_steps_n):
    """One pass of workload w as the bench runs it (ingest, query, exact path):
    the sketch-vs-exact error and the exact decode rate."""
    from exp_density_sketching_amd.workload import run_sketch
    K, V, Q = generate(w)
    Kg, Vg, Qg = (torch.from_numpy(a).cuda() for a in (K, V, Q))
    out_s, z_s, sk = run_sketch(w, Kg, Vg, Qg)
    out_e, z_e = E.exact_attend(Kg, Vg, Qg)
    torch.cuda.synchronize()
    sk.destroy()
    tail = coreset_leg(w, E, torch, Kg, Vg, Qg, out_s, z_s, out_e, z_e, 1)
    r = {"sketch_error": sketch_vs_exact(w, K, Q, z_s, out_s, z_e, out_e),
         "error_with_tail": tail["error_with_tail"],
         "tail_points_per_head": tail["points_per_head"],
         "exact_decode": exact_decode(w, E, torch, Kg, Vg, Qg, decode_steps_n)}
    del Kg, Vg, Qg
    torch.cuda.empty_cache()
    return r


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the sketch shards by sub-stream with one sum all-reduce; see the design "
              "notes)", file=sys.stderr)
        return 2
    import torch
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import exp_density_sketching_amd as E
    from synthetic import WORKLOADS, generate

    w = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    if args.counters:
        return counters_pass(w, E, torch, generate, args.layout)
    print(f"bench: workload {w.name}: generating inputs", file=sys.stderr, flush=True)
    K, V, Q = generate(w)
    res = measure_workload(w, E, torch, K, V, Q, args, full_line=True)
    line = {"metric": METRIC, "value": res.pop("value"), "unit": res.pop("unit"),
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": res.pop("ms_per_step"), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": res.pop("config")}
    line.update(res)
    print(f"bench: workload {w.name} measured", file=sys.stderr, flush=True)
    if line["exact_decode"]["resident"] != "HBM":
        # this workload's KV stays in the Infinity Cache: the exact path's HBM
        # figure comes from the 32-head workload's decode
        line["exact_decode_hbm"] = exact_decode_hbm(WORKLOADS[4], E, torch, args.decode_steps)
    if args.cpu_seconds > 0:
        line["cpu_baseline"] = cpu_baseline(w, K, V, Q, args.cpu_seconds)
    del K, V, Q
    if not args.quick:
        # the largest update (workload 3: 1M keys, 2.34 TFLOP, four sub-streams
        # merged) with its own roofline and CPU baseline
        w3 = WORKLOADS[3]
        if w3.ident != w.ident:
            print(f"bench: workload {w3.name}", file=sys.stderr, flush=True)
            K3, V3, Q3 = generate(w3)
            sub = measure_workload(w3, E, torch, K3, V3, Q3, args, full_line=False)
            if args.cpu_seconds > 0:
                sub["cpu_baseline"] = cpu_baseline(w3, K3, V3, Q3, args.cpu_seconds)
            line["workload3"] = sub
            del K3, V3, Q3
            torch.cuda.empty_cache()
        # the sketch-vs-exact error and the exact decode rate of every configuration
        errs = {}
        for i in sorted(WORKLOADS):
            wi = WORKLOADS[i]
            if wi.ident == w.ident or ("workload3" in line and wi.ident == 3):
                src = line if wi.ident == w.ident else line["workload3"]
                r = {"sketch_error": src["sketch_error"],
                     "error_with_tail": src["tail_coreset"]["error_with_tail"],
                     "tail_points_per_head": src["tail_coreset"]["points_per_head"],
                     "exact_decode": src["exact_decode"]}
            else:
                print(f"bench: error of {wi.name}", file=sys.stderr, flush=True)
                r = error_of_config(wi, E, torch, generate, args.decode_steps)
            errs[wi.name] = r
        line["by_config"] = errs
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
