#!/usr/bin/env python3
"""Benchmark of the deterministic attention backward on one MI355X.

One step = one call of the deterministic backward (pre-pass, main tile
kernel with the ordered dQ reduction, whose last contributor of each dQ
sub-tile writes bf16 dq, and the post-pass that checks the call's failure
flag), on synthetic bf16 inputs already resident
in HBM. The headline workload is the causal B=4, H=32, S=4096, D=128 case;
the same shape with a full mask is measured in the same run and carried as
a sub-record of the line. Every deterministic schedule valid for the mask is
timed, then the atomic-dQ variant; `value` is the fastest deterministic
schedule's throughput under the FLOP convention 2.5 * 4 * B * H * S^2 * D
(halved for a causal mask).

Printed (one JSON line on stdout): the metric, value (TFLOP/s), % of the bf16
dense MFMA peak, the deterministic/non-deterministic ratio, per-schedule
numbers, the roofline of the main tile kernel (its duration taken with HIP
events recorded around its launch on its own stream) and the CPU oracle's
throughput on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C3] [--also C3F]
"""

from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
METRIC = "deterministic attn-bwd TFLOPS (bf16) + % MFMA peak + ratio vs non-det kernel"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent pairs through the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev

    def record(self, ev, stream):
        if self.hip.hipEventRecord(ev, ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(ev)


def time_variant(fn, steps, warmup, torch, events, lib):
    """Wall time of `steps` calls (synchronised both sides), the per-call API times
    (HIP events around each whole call: pre-pass + main kernel + post-pass) and
    the mean main-kernel time (events the library records around that launch)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    pairs = [(events.create(), events.create()) for _ in range(steps)]
    api = [(events.create(), events.create()) for _ in range(steps)]
    t0 = time.perf_counter()
    for (a, b), (c, d) in zip(pairs, api):
        lib.attn_set_timing_events(a, b)
        events.record(c, stream)
        fn()
        events.record(d, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    lib.attn_set_timing_events(None, None)
    kern = [events.elapsed_ms(a, b) for a, b in pairs]
    api_ms = sorted(events.elapsed_ms(c, d) for c, d in api)
    for a, b in pairs + api:
        events.destroy(a)
        events.destroy(b)
    q = lambda f: api_ms[min(len(api_ms) - 1, int(round(f * (len(api_ms) - 1))))]
    return wall / steps * 1e3, sum(kern) / len(kern), {"median": q(0.5), "p10": q(0.1), "p90": q(0.9)}


KERNEL_SOURCES = ("bwd.hip", "common.hpp", "lds.hpp", "schedule.hpp", "launch.hpp")


def code_only(text: str) -> str:
    """C++ source without comments and with whitespace runs collapsed, so that
    edits of comments or layout do not invalidate measurements of the code."""
    import re
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"':  # string literal (asm templates): copied as is
            j = i + 1
            while j < n and text[j] != '"':
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return re.sub(r"\s+", " ", "".join(out)).strip()


def kernel_source_hash(read=None) -> str:
    """Hash of the main kernel's sources (code only). `read(name)` returns a
    file's text (default: the working tree)."""
    import hashlib
    if read is None:
        read = lambda f: open(os.path.join(ROOT, "deterministic_attention_backward_amd", "csrc", f)).read()
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(code_only(read(f)).encode())
    return h.hexdigest()


def traffic_path(workload: str, schedule: str) -> str:
    return os.path.join(ROOT, "profiles", f"bwd_main_{workload}_{schedule}_traffic.json")


def measured_traffic(workload: str, schedule: str, protocol: str):
    """HBM bytes per launch of the main kernel from the committed counter record.

    profiles/bwd_main_<workload>_<schedule>_traffic.json holds FETCH_SIZE +
    WRITE_SIZE (scaled by a 1 GiB copy) for one workload and schedule, with a
    hash of the kernel sources it was taken on. Returns None unless it matches
    this run and the sources are unchanged since.
    """
    path = traffic_path(workload, schedule)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if (rec.get("kernel_source_sha256") != kernel_source_hash() or not rec.get("workload", "").startswith(workload + ":")
            or rec.get("schedule") != schedule or rec.get("dq_protocol") != protocol):
        return None
    return float(rec["traffic_bytes"])


def make_traffic_record(args):
    """Write the traffic record of one workload/schedule from two rocprofv3 --pmc
    runs of this script (FETCH_SIZE, then WRITE_SIZE, both with --copy-calibration):
    per-dispatch means of the main kernel, each scaled by what the same counter
    reads on the three 1 GiB device copies of the same run."""
    import csv
    import attn_inputs

    def read(d, counter):
        rows = []
        for name in os.listdir(d):
            if name.endswith("counter_collection.csv"):
                rows += [r for r in csv.DictReader(open(os.path.join(d, name))) if r["Counter_Name"] == counter]
        main = [r for r in rows if "bwd_main_kernel" in r["Kernel_Name"]]
        kinds = sorted({r["Kernel_Name"] for r in main})
        if len(kinds) != 1:
            raise SystemExit(f"{d}: expected one main-kernel instantiation, found {kinds}")
        # the copies run last, after every timed call: the last three dispatches of a non-library kernel
        other = sorted((int(r["Dispatch_Id"]), float(r["Counter_Value"])) for r in rows
                       if "attn::" not in r["Kernel_Name"])
        copies = [v for _, v in other[-3:]]
        vals = [float(r["Counter_Value"]) for r in main]
        return kinds[0], len(vals), sum(vals) / len(vals), sum(copies) / len(copies)

    fetch_dir, write_dir = args.make_traffic_record
    w = attn_inputs.WORKLOADS[args.workload]
    sched = args.schedules
    kernel, n_f, fetch_kib, fetch_cal = read(fetch_dir, "FETCH_SIZE")
    kernel_w, n_w, write_kib, write_cal = read(write_dir, "WRITE_SIZE")
    if kernel != kernel_w:
        raise SystemExit("the two runs timed different kernels")
    gib = 1 << 30
    fscale = gib / (fetch_cal * 1024)
    wscale = gib / (write_cal * 1024)
    fetch_b = fetch_kib * 1024 * fscale
    write_b = write_kib * 1024 * wscale
    rec = {"workload": f"{w.name}: {w.describe()}", "schedule": sched, "dq_protocol": args.dq_protocol,
           "kernel": kernel, "dispatches": min(n_f, n_w),
           "fetch_size_kib_per_dispatch": round(fetch_kib, 1), "write_size_kib_per_dispatch": round(write_kib, 1),
           "copy_calibration": {"bytes": gib, "fetch_size_kib": round(fetch_cal, 1), "write_size_kib": round(write_cal, 1),
                                "fetch_scale": round(fscale, 4), "write_scale": round(wscale, 4)},
           "fetch_bytes": int(fetch_b), "write_bytes": int(write_b), "traffic_bytes": int(fetch_b + write_b),
           "kernel_source_sha256": kernel_source_hash(),
           "command": f"cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch_dir> -o f -- python3 "
                      f"<repo>/bench.py --workload {w.name} --also '' --schedules {sched} --steps 3 --warmup 1 "
                      f"--cpu-seconds 0 --no-mfma-probe --no-nondet --copy-calibration; the same with --pmc "
                      f"WRITE_SIZE into <write_dir>; then python3 <repo>/bench.py --workload {w.name} --schedules "
                      f"{sched} --make-traffic-record <fetch_dir> <write_dir>"}
    with open(traffic_path(w.name, sched), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def cpu_baseline(w, inputs, o_cpu, lse_cpu, budget_s: float):
    """The float64 oracle backward on whole heads of the same workload, time-bounded."""
    import numpy as np
    from oracle import attention as A
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    B, H = w.B, w.H
    heads = 0
    t0 = time.perf_counter()
    while heads < B * H:
        b, h = divmod(heads, H)
        f = lambda t, hh=h: t[b, hh].to(dtype=__import__("torch").float64).numpy()
        hk = h // (H // w.kv_heads)  # the query head's K/V head (grouped-query workloads)
        q, do = f(inputs["q"]), f(inputs["do"])
        k, v = f(inputs["k"], hk), f(inputs["v"], hk)
        A.backward_head(q, k, v, f(o_cpu), do, lse_cpu[b, h].double().numpy(), w.causal, w.scale)
        heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = w.flops / (B * H) * heads
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{heads} of {B * H} heads of the same workload (float64 backward from the HIP forward's O/LSE), "
                  f"{dt:.1f} s",
    }


def host_info(torch):
    """CPU model, host threads and the ROCm/HIP build the run used."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    gpu = torch.cuda.get_device_name(0) if torch.cuda.is_available() else None
    return {"cpu_model": model, "cpu_threads": os.cpu_count(), "hip": getattr(torch.version, "hip", None),
            "torch": torch.__version__, "gpu": gpu}


def repeat_check(fn, runs, torch):
    """Untimed: run a deterministic call `runs` times and count the runs whose
    dQ, dK and dV carry the first run's bits."""
    ref = [t.clone() for t in fn()]
    same = 1
    for _ in range(runs - 1):
        got = fn()
        if torch.cuda.is_available():
            torch.cuda.synchronize()
        same += all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(ref, got))
    return same


def rnd(x):
    if isinstance(x, dict):
        return {k: rnd(v) for k, v in x.items()}
    return round(x, 4) if isinstance(x, float) else x


def wait_profile(w, sched, args, torch, dab, _lib, tensors):
    """Fractions of wave time spent waiting, from one call of the profiling build (not timed)."""
    q, k, v, o, do, lse = tensors
    prof = _lib.load_profile()
    saved = _lib._lib
    try:
        _lib._lib = prof
        dab.set_dq_protocol(args.dq_protocol)
        ws = dab.alloc_workspace(w.B, w.H, w.S, w.D, w.causal, sched, w.tile, Hkv=w.kv_heads)
        prof.attn_debug_order_violations(1)
        for _ in range(2):
            dab.bwd(q, k, v, o, do, lse, w.causal, sched, w.scale, w.tile, ws)
        torch.cuda.synchronize()
        K = _lib.WAIT_PROFILE_VALUES
        buf = (ctypes.c_uint64 * (K * 1024))()
        n = prof.attn_debug_wait_profile(buf, 1024)
        _lib.check(min(n, 0), "attn_debug_wait_profile")
        bad = prof.attn_debug_order_violations(1)
        _lib.check(min(bad, 0), "attn_debug_order_violations")
    finally:
        _lib._lib = saved
    rows = [[buf[K * g + j] for j in range(K)] for g in range(n)]
    tot = [sum(r[j] for r in rows) for j in range(K)]
    return {"schedule": sched, "workgroups": n,
            "tile_waves_barrier_frac": round(tot[0] / max(tot[1], 1), 4),
            "tile_waves_kv_switch_frac": round(tot[6] / max(tot[1], 1), 4),
            "tile_waves_claim_frac": round(tot[8] / max(tot[1], 1), 4),
            "dq_waves_turn_wait_frac": round(tot[2] / max(tot[4], 1), 4),
            "dq_waves_barrier_frac": round(tot[3] / max(tot[4], 1), 4),
            "turn_wait_cycles_per_subtile": round(tot[2] / max(tot[5], 1), 1),
            "tile_wave_cycles_per_subtile": round(tot[1] / max(tot[5], 1), 1),
            "cycles_per_kv_switch": round(tot[6] / max(tot[7], 1), 1),
            "segments": tot[7], "subtiles": tot[5],
            # the kernel lasts as long as its longest workgroup: mean / max of the
            # workgroups' spans is the fraction of the grid kept busy to the end
            "wg_span_mean_over_max": round(sum(r[1] for r in rows) / max(n * max(r[1] for r in rows), 1), 4),
            "dq_order_violations": bad,
            "note": "s_memtime cycles of one tile wave and one dQ wave per workgroup, profiling build"}


def block_bench(args):
    """One forward + backward step of an 8B-class attention block (random weights), deterministic
    attention backward (the fastest schedule on the block's shapes) against the atomic-dQ one;
    prints its own JSON line."""
    import torch
    import deterministic_attention_backward_amd as dab
    from deterministic_attention_backward_amd.autograd import AttentionBlock

    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible: the benchmark needs an MI355X")
    B, S, hidden, heads, kv_heads, D = 1, 8192, 4096, 32, 8, 128
    log(f"attention block: B={B} S={S} hidden={hidden} heads={heads} kv_heads={kv_heads} head_dim={D} causal")
    g = torch.Generator(device="cpu").manual_seed(9)
    x0 = torch.randn(B, S, hidden, generator=g).to(torch.bfloat16).cuda()
    dy = torch.randn(B, S, hidden, generator=g).to(torch.bfloat16).cuda()
    # the attention backward alone on the block's shapes, every deterministic
    # schedule; the block step then runs the fastest of them
    x = {n: torch.randn(*shape, generator=g).to(torch.bfloat16).cuda()
         for n, shape in (("q", (B, heads, S, D)), ("k", (B, kv_heads, S, D)), ("v", (B, kv_heads, S, D)),
                          ("do", (B, heads, S, D)))}
    o, lse = dab.fwd(x["q"], x["k"], x["v"], True)
    alone = {}
    for sched in ("naive", "descending", "shift", "symmetric_shift"):
        ws = dab.alloc_workspace(B, heads, S, D, True, sched, 0, Hkv=kv_heads)
        fn = lambda sched=sched, ws=ws: dab.bwd(x["q"], x["k"], x["v"], o, x["do"], lse, True, sched, workspace=ws)
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        alone[sched] = (time.perf_counter() - t0) / args.steps * 1e3
        log(f"  attention backward alone ({sched}): {alone[sched]:.3f} ms")
        del ws
    best = min(alone, key=alone.get)
    attn_ms = alone[best]
    res = {}
    for name, sched in (("deterministic", best), ("atomic", None)):
        block = AttentionBlock(hidden, heads, kv_heads, D, causal=True, schedule=sched, seed=1)

        def step():
            block.zero_grad(set_to_none=True)
            xx = x0.detach().requires_grad_()
            block(xx).backward(dy)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        res[name] = (time.perf_counter() - t0) / args.steps * 1e3
        log(f"  {name:14s} {res[name]:8.3f} ms per block step ({B * S / res[name] * 1e3:,.0f} tokens/s)"
            + (f", backward: {best}" if sched else ""))
    line = {"metric": "attention block step (forward + backward), 8B-class shape", "value": round(B * S / res["deterministic"] * 1e3, 1),
            "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(res["deterministic"], 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic (random weights and inputs)",
            "config": {"workload": f"attention block: B={B},S={S},hidden={hidden},heads={heads},kv_heads={kv_heads},"
                                   f"D={D},causal", "schedule": best},
            "atomic_ms_per_step": round(res["atomic"], 4),
            "deterministic_over_atomic_step_time": round(res["deterministic"] / res["atomic"], 4),
            "attention_backward_ms": round(attn_ms, 4),
            "attention_backward_ms_by_schedule": {k: round(v, 4) for k, v in alone.items()},
            "attention_backward_share": round(attn_ms / res["deterministic"], 4)}
    print(json.dumps(line), flush=True)


def measure(w, args, torch, dab, _lib, lib, events):
    """Time every deterministic schedule valid for the workload's mask and the
    atomic-dQ variant on one synthetic draw; returns a record of the results
    plus the inputs (for the CPU baseline and the profiles)."""
    import attn_inputs
    log(f"workload {w.name}: {w.describe()} seed={w.seed}")
    x = attn_inputs.draw_workload(w)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse = dab.fwd(q, k, v, w.causal, w.scale)
    torch.cuda.synchronize()
    T = dab.tile(w.S, w.D, w.tile)
    N = -(-w.S // T)
    if args.schedules:
        scheds = args.schedules.split(",")
    else:
        scheds = ["naive", "descending", "shift"] + (["symmetric_shift"] if w.causal and N % 2 == 0 else [])
    out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    results = {}
    dab.wait_timeouts(reset=True)
    for s in scheds:
        ws = dab.alloc_workspace(w.B, w.H, w.S, w.D, w.causal, s, w.tile, Hkv=w.kv_heads)
        fn = lambda s=s, ws=ws: dab.bwd(q, k, v, o, do, lse, w.causal, s, w.scale, w.tile, ws, out)
        ms, kms, api = time_variant(fn, args.steps, args.warmup, torch, events, lib)
        dab.check_workspace(ws)
        results[s] = {"ms": ms, "kernel_ms": kms, "tflops": w.flops / (ms * 1e-3) / 1e12, "api_ms": api,
                      "wait_timeouts": dab.wait_timeouts(reset=True)}
        log(f"  {s:16s} {ms:8.3f} ms/call  main kernel {kms:8.3f} ms  {results[s]['tflops']:7.1f} TFLOP/s")
        if results[s]["wait_timeouts"]:
            log(f"  WARNING: {results[s]['wait_timeouts']} bounded dQ waits ran out during the {s} calls")
        del ws
    nondet = None
    if not args.no_nondet:
        ws = dab.alloc_workspace(w.B, w.H, w.S, w.D, w.causal, "naive", w.tile, Hkv=w.kv_heads)
        fn = lambda: dab.bwd_nondeterministic(q, k, v, o, do, lse, w.causal, w.scale, w.tile, ws, out)
        ms, kms, api = time_variant(fn, args.steps, args.warmup, torch, events, lib)
        # one fp32 atomic add per element of every task's dQ partial (T rows x D per task)
        tasks = N * (N + 1) // 2 if w.causal else N * N
        adds = w.B * w.H * tasks * T * w.D
        nondet = {"ms": ms, "kernel_ms": kms, "tflops": w.flops / (ms * 1e-3) / 1e12, "api_ms": api,
                  "walk": "shift", "placement": "per-XCD head queue",
                  "atomic_adds_per_launch": adds, "atomic_gops": adds / (kms * 1e-3) / 1e9}
        log(f"  {'atomic (non-det)':16s} {ms:8.3f} ms/call  main kernel {kms:8.3f} ms  {nondet['tflops']:7.1f} TFLOP/s")
        del ws
    best = min(results, key=lambda s: results[s]["ms"])
    ws = dab.alloc_workspace(w.B, w.H, w.S, w.D, w.causal, best, w.tile, Hkv=w.kv_heads)
    same = repeat_check(lambda: dab.bwd(q, k, v, o, do, lse, w.causal, best, w.scale, w.tile, ws, out), 20, torch)
    del ws
    log(f"repeatability ({best}, untimed): {same} of 20 runs give the first run's bits")
    r = results[best]
    achieved = w.flops / (r["kernel_ms"] * 1e-3) / 1e12
    rec = {
        "workload": f"{w.name}: {w.describe()}", "schedule": best, "tile": T, "n_tiles": N, "seed": w.seed,
        "flops_per_step": w.flops,
        "value": round(r["tflops"], 2), "ms_per_step": round(r["ms"], 4),
        "pct_mfma_peak": round(100.0 * r["tflops"] / PEAK_BF16_TFLOPS, 2),
        "ratio_vs_nondet": round(nondet["ms"] / r["ms"], 4) if nondet else None,
        "schedules": {s: {"ms": round(v["ms"], 4), "kernel_ms": round(v["kernel_ms"], 4),
                          "tflops": round(v["tflops"], 2), "api_ms": rnd(v["api_ms"]),
                          "wait_timeouts": v["wait_timeouts"]} for s, v in results.items()},
        "dq_wait_timeouts": sum(v["wait_timeouts"] for v in results.values()),
        "bitwise_identical_runs": {"schedule": best, "runs": 20, "identical": same},
        "nondet": {k2: rnd(v2) for k2, v2 in nondet.items()} if nondet else None,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(w.name, best, args.dq_protocol),
                     "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE)",
                     "kernel": "bwd_main_kernel", "kernel_ms": round(r["kernel_ms"], 4)},
    }
    return rec, (x, q, k, v, o, do, lse)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="C3", help="headline workload (default: causal 4k, D 128)")
    ap.add_argument("--also", default="C3F",
                    help="comma list of workloads measured in the same run as sub-records ('' = none)")
    ap.add_argument("--schedules", default="", help="comma list; default: every schedule valid for the mask")
    ap.add_argument("--no-nondet", action="store_true")
    ap.add_argument("--dq-protocol", default="auto", choices=["auto", "device", "xcd_local"],
                    help="dQ hand-off of the deterministic calls (auto picks XCD-local where it applies)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle leg (0 = skip)")
    ap.add_argument("--no-mfma-probe", action="store_true", help="skip the measured-MFMA-peak probe")
    ap.add_argument("--block", action="store_true",
                    help="time an 8B-class attention block (forward + backward) instead; prints its own JSON line")
    ap.add_argument("--wait-profile", action="store_true",
                    help="one extra, untimed call of the best schedule with the profiling build: wait-cycle fractions")
    ap.add_argument("--make-traffic-record", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/bwd_main_<workload>_<schedule>_traffic.json from two rocprofv3 --pmc runs "
                         "(no GPU needed)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (for HBM counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    if args.block:
        block_bench(args)
        return
    if args.make_traffic_record:
        if not args.schedules or "," in args.schedules:
            raise SystemExit("--make-traffic-record needs one --schedules name")
        make_traffic_record(args)
        return

    import torch
    import attn_inputs
    import deterministic_attention_backward_amd as dab
    from deterministic_attention_backward_amd import _lib

    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible: the benchmark needs an MI355X")
    lib = _lib.load()
    dab.set_dq_protocol(args.dq_protocol)
    events = HipEvents()
    w = attn_inputs.WORKLOADS[args.workload]
    head, (x, q, k, v, o, do, lse) = measure(w, args, torch, dab, _lib, lib, events)
    subs = {}
    for name in [n for n in args.also.split(",") if n and n != args.workload]:
        subs[name], _ = measure(attn_inputs.WORKLOADS[name], args, torch, dab, _lib, lib, events)

    if args.copy_calibration:
        nbytes = 1 << 30
        src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {nbytes} bytes read + {nbytes} bytes written per copy, 3 copies")

    atomic_probe = None
    if not args.no_nondet and not args.no_mfma_probe:
        buf = torch.zeros(64 << 20, dtype=torch.float32, device="cuda")  # 256 MiB, about C3F's dQ accumulator
        g = ctypes.c_double()
        _lib.check(lib.attn_probe_atomic(ctypes.c_void_p(buf.data_ptr()), buf.numel() * 4, 200,
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), ctypes.byref(g)),
                   "attn_probe_atomic")
        del buf
        atomic_probe = {"gops": round(g.value, 1),
                        "probe": "fp32 atomic adds, 64 consecutive floats per instruction, 4 KB blocks, one block "
                                 "per wave at a time, 256 MiB buffer"}
        log(f"measured fp32 atomic-add rate {g.value:.1f} Gop/s")
        for rec in [head] + list(subs.values()):
            if rec.get("nondet"):
                rec["nondet"]["atomic_bound_frac"] = round(rec["nondet"]["atomic_gops"] / g.value, 4)

    mfma = None
    if not args.no_mfma_probe:
        tf, ghz = ctypes.c_double(), ctypes.c_double()
        _lib.check(lib.attn_probe_mfma(200000, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream),
                                       ctypes.byref(tf), ctypes.byref(ghz)), "attn_probe_mfma")
        mfma = {"tflops": round(tf.value, 1), "sclk_ghz": round(ghz.value, 3),
                "probe": "one workgroup per CU, 4 waves, 4 independent bf16 32x32x16 MFMA chains per wave"}
        log(f"measured dense bf16 MFMA peak {tf.value:.1f} TFLOP/s at {ghz.value:.3f} GHz (s_memtime rate)")
    wait = None
    if args.wait_profile:
        wait = wait_profile(w, head["schedule"], args, torch, dab, _lib, (q, k, v, o, do, lse))
        log(f"wait profile ({head['schedule']}): {wait}")
    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": head["workload"], "schedule": head["schedule"], "tile": head["tile"],
                   "n_tiles": head["n_tiles"], "dq_protocol": args.dq_protocol, "seed": head["seed"],
                   "flops_per_step": head["flops_per_step"]},
        "pct_mfma_peak": head["pct_mfma_peak"],
        "ratio_vs_nondet": head["ratio_vs_nondet"],
    }
    for key in ("schedules", "dq_wait_timeouts", "bitwise_identical_runs", "nondet"):
        line[key] = head[key]
    line["mfma_measured"] = mfma
    line["atomic_measured"] = atomic_probe
    line["pct_measured_mfma_peak"] = round(100.0 * head["value"] / mfma["tflops"], 2) if mfma else None
    line["roofline"] = head["roofline"]
    line["sub_records"] = subs
    if wait is not None:
        line["wait_profile"] = wait
    line["host"] = host_info(torch)
    if args.cpu_seconds > 0:
        x_cpu = {n: x[n] for n in ("q", "k", "v", "do")}
        line["cpu_baseline"] = cpu_baseline(w, x_cpu, o.cpu(), lse.cpu(), args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
