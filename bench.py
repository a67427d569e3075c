#!/usr/bin/env python3
"""Benchmark of split-KV decode attention (libfd) on one MI355X.

One step = one fd_decode_attention call (split kernel + LSE combine) over one
batch of the workload, with every input already resident in HBM. The
default workload is the largest single-GPU configuration: Llama-3.1-8B-shaped
decode attention at batch 16, 131,072 cached keys per sequence, 32 query /
8 KV heads, head dim 128, bf16, packed [total_kv, kv_heads, dim] K/V
(8.59 GB per call), split count from the planner. Smaller workloads are
reached with --workload (e.g. mha_b4_h32_l4096_d128_f16) or --all. When one
step's K/V is smaller than three times the 256 MB last-level cache, several
copies are rotated so that the cache never holds the next step's K/V: every
step streams its K/V from HBM.

Prints ONE JSON line: metric/value (achieved GB/s on the KV bytes of one
step), ms_per_step, the roofline of the dominant kernel (the split kernel,
timed by HIP events on the stream it runs on, over a run of split-only
launches right after the timed steps) and the CPU oracle's rate on the same
workload.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--all]
    python bench.py --workload NAME[,NAME...] --sweep-splits 1,2,4,8 [--kernel-path P]
    python bench.py --all --graph     # timed calls replayed from one captured HIP graph

Eager timing (the default) issues every call from Python; through the binding
that costs the host ~12 us per call, which bounds the smallest shapes
(<= ~12 us of GPU work per call). --graph captures the timed calls once and
replays them, so those shapes show their GPU time.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attention µs/call + achieved HBM GB/s (fraction of ~8 TB/s) on 1 MI355X"
DEFAULT_WORKLOAD = "llama8b_b16_l131072_h32kv8_d128_bf16"
PEAK_GBS = 8000.0
LLC_BYTES = 256 * 2 ** 20       # MI355X Infinity Cache (MALL)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# Workloads measured briefly beside the headline in a default run: the other
# long-context and GQA points (flash-decoding 16/2-head shapes, Llama-8B at
# batch 1 and 16, the varlen Qwen batch) and the MHA D = 128 shape.
CONTEXT_WORKLOADS = [
    "fd_ubench_b8_l8192_h16kv2_d128_f16",
    "fd_ubench_b1_l65536_h16kv2_d128_f16",
    "llama8b_b1_l131072_h32kv8_d128_bf16",
    "llama8b_b16_l32768_h32kv8_d128_bf16",
    "varlen_qwen7b_b32_h28kv4_d128_f16",
    "mha_b4_h32_l4096_d128_f16",
]
KERNEL_SOURCES = ["fd_split.h", "fd_internal.h", "fd_steal.h"]


def _code_only(text: str) -> str:
    """C++ source without comments and whitespace (string literals in these
    kernel sources hold no comment markers), so edits to comments alone do
    not count as a kernel change."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return re.sub(r"\s+", "", text)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for n in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "decode_attention_09_amd", "csrc", n)) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def workload_by_name(name: str):
    import workloads as W
    for w in W.all_workloads():
        if w.name == name:
            return w
    raise SystemExit(f"unknown workload {name!r}; known: "
                     + ", ".join(w.name for w in W.all_workloads()))


def choose_schedule(fd, w, requested, lengths, ns_override=0):
    """Set the calling thread's schedule for workload w before its split
    count is planned: the requested one, else fd_plan_schedule's
    recommendation for these lengths -- taken with its split count where
    the planner sets the count, and where the workload fixes the count only
    if the recommendation's count is the same. Returns (schedule name,
    split count or 0 for the planner's)."""
    code = {"auto": fd.FD_SCHED_AUTO, "static": fd.FD_SCHED_STATIC,
            "queue": fd.FD_SCHED_QUEUE, "steal": fd.FD_SCHED_STEAL}
    names = {v: k for k, v in code.items()}
    name, planned = requested or "auto", 0
    if requested is None and min(lengths) > 0:
        dt = {"f32": fd.FD_F32, "f16": fd.FD_F16, "bf16": fd.FD_BF16}[w.dtype]
        rec, ns_rec = fd.fd_plan_schedule(w.batch, w.heads, w.kv_heads, w.dim, dt, lengths)
        fixed = pick_splits(w, lengths, ns_override) if (ns_override or w.num_splits) else 0
        if not fixed:
            name, planned = names[rec], ns_rec
        elif fixed == ns_rec:
            name = names[rec]
    fd.fd_set_schedule(code[name])
    return name, planned


def pick_splits(w, lengths, override=0):
    import workloads as W
    import decode_attention_09_amd as fd
    if override:
        return override
    if w.num_splits is not None:
        return W.varlen_splits(w, lengths) if w.varlen_range else w.num_splits
    code = {"f32": fd.FD_F32, "f16": fd.FD_F16, "bf16": fd.FD_BF16}[w.dtype]
    return fd.fd_plan_splits(w.batch, w.heads, w.kv_heads, w.dim, code, lengths)


def traffic_for(workload_name: str):
    """HBM bytes per split-kernel launch from committed rocprofv3 counter
    runs, or None if absent, for another workload, or the kernel changed."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload_name)
    if not e or e.get("kernel_hash") != kernel_hash():
        return None
    return e.get("hbm_bytes_per_launch")


def cpu_baseline(inp, ns, budget_s: float, fmt: str = "lse", threads: int = 1):
    """The fp64 numpy oracle (split + merge) on the same workload, one
    (sequence, KV head) unit at a time in order, repeated until its own
    compute time reaches ~budget_s seconds; BLAS limited to `threads`
    threads. Host copies of the inputs are made outside the clock."""
    from threadpoolctl import threadpool_limits
    import oracle
    w = inp.workload
    q = inp.q.float().cpu().numpy()
    cu = inp.cu_seqlens_k.cpu().tolist()
    units = [(b, j) for b in range(w.batch) for j in range(w.kv_heads)]
    G = w.group
    bytes_per_key = w.dim * 2 * w.elem_bytes     # one K row + one V row
    done_bytes = 0
    n_units = 0
    oracle_s = 0.0
    with threadpool_limits(limits=threads):
        while oracle_s < budget_s:
            b, j = units[n_units % len(units)]
            L = cu[b + 1] - cu[b]
            if w.layout == "packed":
                kr = inp.k[cu[b]:cu[b + 1], j].float().cpu().numpy()
                vr = inp.v[cu[b]:cu[b + 1], j].float().cpu().numpy()
            else:
                kr = inp.k[b, j, :L].float().cpu().numpy()
                vr = inp.v[b, j, :L].float().cpu().numpy()
            t1 = time.perf_counter()
            if L > 0 and fmt == "unnorm":
                m, l, acc = oracle.split_states_rows(q[b, j * G:(j + 1) * G], kr, vr, ns,
                                                     w.sm_scale)
                oracle.merge_states(m, l, acc)
            elif L > 0:
                op, lse = oracle.split_partials_rows(q[b, j * G:(j + 1) * G], kr, vr,
                                                     min(ns, L), w.sm_scale)
                oracle.merge_partials(op, lse)
            oracle_s += time.perf_counter() - t1
            done_bytes += L * bytes_per_key
            n_units += 1
    rate = done_bytes / oracle_s
    res = {
        "value": round(rate / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{n_units} (sequence, KV head) units of this workload "
                  f"({n_units / len(units):.2f} passes), fp64 split+merge, "
                  f"{oracle_s:.1f} s of oracle time",
    }
    if n_units < len(units):
        # the sample covers part of one call: the whole call's oracle time is
        # an extrapolation at the sampled rate
        res["whole_call_s_extrapolated"] = round(inp.kv_bytes / rate, 2)
        res["sample"] += (f"; extrapolated to the whole call ({len(units)} units): "
                          f"{inp.kv_bytes / rate:.1f} s")
    return res


def split_workgroups(w, ns: int, rows_per_workgroup: int, schedule: str = "auto",
                     cus: int = 256) -> int:
    """Workgroups of the split launch: one per (sequence, KV head, block of
    up to rows_per_workgroup query heads of the group, split); under the
    steal schedule, one per share (the library's layout rule: the largest
    divisor d <= ns/2 of ns with units*d <= cus and ns/d - 1 in 1..15)."""
    units = w.batch * w.kv_heads * math.ceil(w.group / rows_per_workgroup)
    if schedule == "steal" and w.dim == 128 and rows_per_workgroup == 8 and w.group >= 2:
        for d in range(ns // 2, 0, -1):
            if ns % d == 0 and 1 <= ns // d - 1 <= 15 and units * d <= min(cus, 4096):
                return units * d
    return units * ns


def run(w, steps: int, warmup: int, cpu_s: float, copies_min_bytes: int = 3 * LLC_BYTES,
        ns_override: int = 0, rows_per_workgroup: int = 8, fmt: str = "lse", graph: bool = False,
        schedule: str | None = None):
    import torch
    import workloads as W
    import decode_attention_09_amd as fd

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = W.make_inputs(w, dev, seed=0)
    schedule, planned = choose_schedule(fd, w, schedule, inp.lengths, ns_override)
    ns = planned or pick_splits(w, inp.lengths, ns_override)
    kv_bytes = inp.kv_bytes
    copies = max(1, min(16, math.ceil(copies_min_bytes / max(1, kv_bytes))))
    ks = [inp.k] + [inp.k.clone() for _ in range(copies - 1)]
    vs = [inp.v] + [inp.v.clone() for _ in range(copies - 1)]
    out = torch.empty_like(inp.q)
    B, Hq, D = w.batch, w.heads, w.dim
    unnorm = fmt == "unnorm"
    ws_bytes = (fd.fd_workspace_bytes_unnorm if unnorm else fd.fd_workspace_bytes)(B, Hq, ns, D)
    # zero-filled once: the arrival counters of fused calls start at zero
    ws = torch.zeros(max(1, ws_bytes), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    mode = fd.fd_set_combine(fd.FD_COMBINE_SEPARATE)
    fd.fd_set_combine(mode)
    # one launch per call: a single split, or the fused combine (normalised format)
    single_launch = ns == 1 or (mode == fd.FD_COMBINE_FUSED and not unnorm)
    attention = fd.fd_decode_attention_unnorm if unnorm else fd.fd_decode_attention
    split = fd.fd_decode_split_unnorm if unnorm else fd.fd_decode_split

    def step(i, s=None):
        k, v = ks[i % copies], vs[i % copies]
        attention(inp.q, k, v, inp.cu_seqlens_k, ns, out=out, workspace=ws, layout=w.layout,
                  stream=stream if s is None else s)

    def split_only(i, s=None):
        k, v = ks[i % copies], vs[i % copies]
        split(inp.q, k, v, inp.cu_seqlens_k, ns, workspace=ws, layout=w.layout,
              stream=stream if s is None else s)

    def timed(fn, n, offset):
        """Mean ms per call of n back-to-back calls: issued one by one from
        Python (eager), or captured once in a HIP graph and replayed (graph),
        which takes the host's issue cost (~12 us per call through the
        binding) out of the measurement."""
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        g = None
        if graph:
            side = torch.cuda.Stream(dev)
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                fn(offset, side)
            stream.wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                cs = torch.cuda.current_stream()
                for i in range(n):
                    fn(offset + i, cs)
            g.replay()                  # first replay untimed
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        if g is not None:
            g.replay()
        else:
            for i in range(n):
                fn(offset + i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n, time.perf_counter() - t0

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # the timed steps: whole calls, back to back on one stream
    ms_per_step, wall = timed(step, steps, warmup)
    # the dominant kernel: with one split the whole step is that one launch;
    # otherwise the split kernel alone, same inputs and launch configuration
    split_avg = ms_per_step if single_launch else timed(split_only, steps, warmup + steps)[0]
    # per-call spread: an event pair around each call (the events add a
    # little to each call, so the mean above is the headline)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[2 * i].record(stream)
        step(warmup + 2 * steps + i)
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    per_call = sorted(ev[2 * i].elapsed_time(ev[2 * i + 1]) * 1e3 for i in range(steps))

    def pct(p):
        return round(per_call[min(len(per_call) - 1, int(p * len(per_call)))], 3)
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = kv_bytes / (split_avg * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_call": round(ms_per_step * 1e3, 3),
        "per_call_us": {"p10": pct(0.10), "p50": pct(0.50), "p90": pct(0.90), "calls": steps,
                        "how": "HIP events around each call"},
        "higher_is_better": True,
        "schedule": schedule,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) q/K/V, no model weights)",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads,
                   "kv_heads": w.kv_heads, "head_dim": w.dim, "kv_len_total": sum(inp.lengths),
                   "layout": w.layout, "num_splits": ns,
                   "partials": "(m, l, acc), ceil-equal bounds" if unnorm
                   else "(o_s, lse_s), runs of chunks within proportional shares"
                   if schedule == "steal" and not single_launch
                   else "(o_s, lse_s), proportional bounds",
                   "schedule": schedule,
                   "split_workgroups": split_workgroups(
                       w, ns, rows_per_workgroup,
                       schedule if fmt == "lse" and ns > 1 and not single_launch else "static",
                       torch.cuda.get_device_properties(dev).multi_processor_count),
                   "kv_bytes": kv_bytes,
                   "kv_copies_rotated": copies, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBS, 4),
                     "traffic": traffic_for(w.name),
                     "kernel": "split kernel",
                     "kernel_us": round(split_avg * 1e3, 3),
                     "algorithmic_bytes_per_launch": kv_bytes},
        "wall_s_timed": round(wall, 4),
        "timing": "graph replay" if graph else "eager calls",
    }
    if cpu_s > 0:
        res["cpu_baseline"] = cpu_baseline(inp, ns, cpu_s, fmt)
        threads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
        if threads > 1:
            res["cpu_baseline_all_cores"] = cpu_baseline(inp, ns, cpu_s, fmt, threads)
    return res


# The split-count sweeps the planner's time model is fitted to: the three
# settings of 04_flash_decoding.py demo 4 (16/2 heads) and four Llama-8B
# shapes, whole calls replayed from a HIP graph (no host issue cost).
FIT_SWEEPS = [
    ("fd_ubench_b1_l65536_h16kv2_d128_f16", [1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64, 96, 128]),
    ("fd_ubench_b8_l8192_h16kv2_d128_f16", [1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64, 96, 128]),
    ("fd_ubench_b64_l2048_h16kv2_d128_f16", [1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64, 96, 128]),
    ("llama8b_b1_l65536_h32kv8_d128_bf16_ns1", [1, 2, 4, 8, 16, 32, 64, 128]),
    ("llama8b_b16_l8192_h32kv8_d128_bf16", [1, 2, 4, 8, 16, 32, 64, 128]),
    ("llama8b_b1_l8192_h32kv8_d128_bf16", [1, 2, 4, 8, 16, 32, 64, 128]),
    ("llama8b_b16_l1024_h32kv8_d128_bf16", [1, 2, 4, 8, 16, 32, 64, 128]),
    ("llama8b_b1_l131072_h32kv8_d128_bf16", [8, 16, 24, 32, 48, 64, 96, 128, 192, 256]),
    ("llama8b_b1_l32768_h32kv8_d128_bf16", [8, 16, 24, 32, 48, 64, 96, 128, 192]),
    ("fd_ubench_b1_l131072_h16kv2_d128_f16", [16, 32, 48, 64, 96, 128, 192, 256]),
    ("llama8b_b16_l32768_h32kv8_d128_bf16", [1, 2, 3, 4, 6, 8]),
]


def model_call_us(p, units, ns, cus, key_bytes, max_len, partial_bytes):
    """The planner's time model for uniform lengths (fd_api.hip, model_call_us),
    with parameters p = (launch, workgroup, rate, contention, combine,
    combine per MB) in us and bytes/us."""
    launch, wg_us, rate, contention, comb, comb_mb = p
    wg_bytes = math.ceil(max_len / ns) * key_bytes
    t, rem = launch, units * ns
    while rem > 0:
        n = min(rem, cus)
        t += wg_us + wg_bytes * (1.0 / rate + n / contention)
        rem -= n
    if ns > 1:
        t += comb + comb_mb * partial_bytes * 1e-6
    return t


def fit_planner(steps: int, warmup: int):
    """Measure FIT_SWEEPS, fit the time model's six constants (least squares
    on relative error), and print one JSON line: the fitted constants, the
    fit's error, and per point the measured time, the library's modelled
    time (fd_plan_time_us, its compiled-in constants) and the refit's."""
    import torch
    from scipy.optimize import least_squares
    import decode_attention_09_amd as fd
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    pts = []
    for name, splits in FIT_SWEEPS:
        w = workload_by_name(name)
        for ns in splits:
            r = run(w, steps, warmup, 0.0, ns_override=ns, graph=True, schedule="static")
            G = w.group
            pts.append(dict(workload=name, ns=ns, batch=w.batch, heads=w.heads,
                            kv_heads=w.kv_heads, dim=w.dim, kv_len=w.kv_len,
                            units=w.batch * w.kv_heads * math.ceil(G / 8),
                            key_bytes=2 * w.dim * w.elem_bytes,
                            partial_bytes=w.batch * w.heads * ns * (w.dim + 1) * 4,
                            measured_us=r["us_per_call"]))
            print(f"[fit] {name} ns={ns} {r['us_per_call']:.2f} us", file=sys.stderr, flush=True)
            torch.cuda.empty_cache()

    def resid(p):
        return [model_call_us(p, x["units"], x["ns"], cus, x["key_bytes"], x["kv_len"],
                              x["partial_bytes"]) / x["measured_us"] - 1.0 for x in pts]
    fit = least_squares(resid, [3.0, 1.0, 5e4, 1.5e7, 2.5, 0.7],
                        bounds=([0, 0, 1e3, 1e5, 0, 0], [50, 50, 1e7, 1e9, 50, 100]))
    code = {"f32": fd.FD_F32, "f16": fd.FD_F16, "bf16": fd.FD_BF16}
    for x in pts:
        w = workload_by_name(x["workload"])
        x["library_model_us"] = round(fd.fd_plan_time_us(
            w.batch, w.heads, w.kv_heads, w.dim, code[w.dtype], [w.kv_len] * w.batch, x["ns"],
            num_cus=cus), 2)
        x["refit_model_us"] = round(model_call_us(fit.x, x["units"], x["ns"], cus,
                                                  x["key_bytes"], x["kv_len"],
                                                  x["partial_bytes"]), 2)
    rel = [abs(v) for v in fit.fun]
    names = ["launch_us", "workgroup_us", "rate_bytes_per_us", "contention_bytes_per_us",
             "combine_us", "combine_us_per_mb"]
    print(json.dumps({"fit": dict(zip(names, [round(v, 4) for v in fit.x])),
                      "rms_rel": round(math.sqrt(sum(v * v for v in rel) / len(rel)), 4),
                      "max_rel": round(max(rel), 4), "cus": cus, "points": pts}), flush=True)


def context_points(names, steps: int = 100, warmup: int = 100):
    """Short runs of other workloads after the headline, each replayed from
    a captured HIP graph (so the host's per-call issue cost, which bounds
    the smallest shapes when calls are issued one by one, stays out): whole
    call and split kernel, each as a fraction of 8 TB/s on its K/V bytes."""
    import torch
    pts = []
    for n in names:
        torch.cuda.empty_cache()
        try:
            r = run(workload_by_name(n), steps, warmup, 0.0, graph=True)
        except Exception as e:  # a context point never costs the headline its line
            pts.append({"workload": n, "error": f"{type(e).__name__}: {e}"})
            continue
        pts.append({"workload": n, "schedule": r["schedule"],
                    "num_splits": r["config"]["num_splits"],
                    "kv_bytes": r["config"]["kv_bytes"],
                    "us_per_call": r["us_per_call"],
                    "call_frac": round(r["value"] / PEAK_GBS, 4),
                    "split_kernel_us": r["roofline"]["kernel_us"],
                    "split_frac": r["roofline"]["frac"],
                    "traffic": r["roofline"]["traffic"]})
    return {"timing": f"graph replay, {steps} calls after {warmup}", "points": pts}


def copy_calibration(mib: int):
    """Ten device-to-device copies of a mib-MiB buffer: a kernel that reads
    and writes exactly mib MiB per launch, to scale the HBM byte counters."""
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": mib << 20, "launches": 10}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # Untimed calls before the timed ones. On MI355X the first tens of
    # milliseconds of back-to-back calls run slower (the bench line: first 25
    # calls ~1470 us on average, then 1233-1238 us; on another device ~80
    # calls at ~1285 us before ~1236 us), so the default warm-up spans
    # ~0.12 s of the bench line.
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=None,
                    help=f"workload name (default {DEFAULT_WORKLOAD}; without this flag the "
                         "line also carries short graph-replayed runs of the other long-context "
                         "and GQA workloads under 'context')")
    ap.add_argument("--no-context", action="store_true",
                    help="leave out the 'context' runs of a default invocation")
    ap.add_argument("--all", action="store_true",
                    help="one line per workload (no CPU leg unless --cpu-seconds is given)")
    ap.add_argument("--cpu-seconds", type=float, default=None,
                    help="oracle time budget per CPU leg (default 10 for one workload, "
                         "0 = no CPU leg for --all and --sweep-splits)")
    ap.add_argument("--num-splits", type=int, default=0,
                    help="override the workload's split count (sweeps)")
    ap.add_argument("--kernel-path", choices=["auto", "valu", "mfma", "unpacked"],
                    default="auto",
                    help="split kernel variant (default: the library's own choice; "
                         "unpacked = one query head per workgroup, the comparison path)")
    ap.add_argument("--schedule", choices=["auto", "static", "queue", "steal"], default=None,
                    help="how split launches hand segments to workgroups (default: "
                         "fd_plan_schedule's recommendation for the workload's lengths; "
                         "queue = a device-sized grid claiming segments from a "
                         "counter; steal = one workgroup per share of each unit, chunks "
                         "claimed ahead, idle workgroups taking the back half of another "
                         "share's unclaimed chunks)")
    ap.add_argument("--combine", choices=["separate", "fused"], default="separate",
                    help="merge the partials in the combine kernel (default) or in the split "
                         "kernel's last workgroup per (sequence, KV head): one launch")
    ap.add_argument("--format", choices=["lse", "unnorm"], default="lse",
                    help="split format: normalised partials + LSE with proportional bounds "
                         "(default), or (m, l, acc) with ceil-equal bounds")
    ap.add_argument("--sweep-splits", default="",
                    help="comma-separated split counts: one line (no CPU leg) per "
                         "workload in --workload (comma-separated) and split count")
    ap.add_argument("--graph", action="store_true",
                    help="time the calls as one captured HIP graph replay instead of eager "
                         "calls (takes the host's per-call issue cost out; for small shapes)")
    ap.add_argument("--fit-planner", action="store_true",
                    help="measure the split-count sweeps and fit the planner's time model")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-sized device buffer 10 times (reference for the "
                         "FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.fit_planner:
        fit_planner(args.steps, args.warmup)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(this implementation runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    import decode_attention_09_amd as fd
    fd.fd_set_kernel_path({"auto": fd.FD_PATH_AUTO, "valu": fd.FD_PATH_VALU,
                           "mfma": fd.FD_PATH_MFMA,
                           "unpacked": fd.FD_PATH_UNPACKED}[args.kernel_path])
    fd.fd_set_combine(fd.FD_COMBINE_FUSED if args.combine == "fused" else fd.FD_COMBINE_SEPARATE)
    rows = 1 if args.kernel_path == "unpacked" else 8
    if args.all or args.sweep_splits:
        import torch
        import workloads as W
        if args.all:
            todo = [(w, args.num_splits) for w in W.all_workloads()]
        else:
            splits = [int(x) for x in args.sweep_splits.split(",") if x]
            todo = [(workload_by_name(n), ns)
                    for n in (args.workload or DEFAULT_WORKLOAD).split(",")
                    for ns in splits]
        cpu_s = args.cpu_seconds or 0.0
        for w, ns in todo:
            r = run(w, args.steps, args.warmup, cpu_s, ns_override=ns, rows_per_workgroup=rows,
                    fmt=args.format, graph=args.graph, schedule=args.schedule)
            r["kernel_path"] = args.kernel_path
            r["combine"] = args.combine
            print(json.dumps(r), flush=True)
            torch.cuda.empty_cache()
        return
    cpu_s = 10.0 if args.cpu_seconds is None else args.cpu_seconds
    w = workload_by_name(args.workload or DEFAULT_WORKLOAD)
    r = run(w, args.steps, args.warmup, cpu_s, ns_override=args.num_splits,
            rows_per_workgroup=rows, fmt=args.format, graph=args.graph, schedule=args.schedule)
    r["kernel_path"] = args.kernel_path
    r["combine"] = args.combine
    if args.workload is None and not args.no_context and not args.num_splits \
            and args.schedule is None and args.format == "lse":
        r["context"] = context_points(CONTEXT_WORKLOADS)
    print(json.dumps(r), flush=True)


if __name__ == "__main__":
    main()
