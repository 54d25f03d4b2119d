#!/usr/bin/env python3
"""Throughput of split-KV target-verify attention on one MI355X.

One step = one full pass of the hot path over one batch: the prefix kernel
(gather + QK^T + online softmax + PV over every prefix range) and the combine
kernel (range merge + causal draft block + final merge), launched through the
C ABI on one stream.  Inputs are resident in HBM before timing starts.

Cold cache: the K/V working set of the headline workload (134 MB) fits in the
256 MB Infinity Cache, so the timed loop rotates over independent input
replicas (separate pools and kv_indices); each replica was last touched
several hundred MB of traffic earlier, so its K/V comes from HBM.  Warm-cache
and graph-replay figures are reported beside it.

Output: one JSON line on stdout (rank 0, N = 1).  ``value`` is the headline
metric: algorithmic K/V bytes of the batch / time per step, in GB/s.
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "speculative_decoding_attention_amd", "csrc", "va_kernels.hip")
PROFILES = os.path.join(ROOT, "profiles")


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed iterations of each timed loop's body right before it")
    ap.add_argument("--replicas", type=int, default=8,
                    help="independent input sets rotated through the timed loop")
    ap.add_argument("--workload", default="b8_8k")
    ap.add_argument("--quick", action="store_true",
                    help="headline only: no secondary workloads, no CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def kernel_source_hash():
    """Hash of what decides the prefix kernel's traffic: its source, its
    parameter header and the split planner (argument marshalling excluded)."""
    h = hashlib.sha256()
    for name in ("va_kernels.hip", "va_internal.h", "va_plan.cpp"):
        with open(os.path.join(ROOT, "speculative_decoding_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload):
    """HBM bytes per prefix launch from the committed counter summary of this
    workload, or None if it is missing or was taken on a different kernel
    source."""
    try:
        fields = {}
        with open(os.path.join(PROFILES, "prefix_kernel_%s_traffic.txt" % workload)) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("kernel_sources_sha256") != kernel_source_hash():
            return None
        return float(fields["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


class Runner:
    """Pre-marshalled arguments for the two C entry points of one replica.
    ``kv_indices`` may be given to pass a longer buffer whose first
    ``sum n_b`` entries are the replica's (a capacity-sized buffer, as under
    graph capture)."""

    def __init__(self, va, p, workspace, out, kv_indices=None):
        import ctypes
        idx = p.kv_indices if kv_indices is None else kv_indices
        self.va, self.p, self.ws, self.out, self.idx = va, p, workspace, out, idx
        self.desc = va.make_desc(p.q, p.k_ext, p.v_ext, p.k_buf, p.v_buf, idx, out, p.bs)
        self.lib = va.lib()
        F = ctypes.c_float
        self.pre_args = (p.q.data_ptr(), p.k_buf.data_ptr(), p.v_buf.data_ptr(), p.qo_indptr.data_ptr(),
                         p.kv_indptr.data_ptr(), idx.data_ptr(), p.l_ext, F(p.sm_scale),
                         F(p.k_scale), F(p.v_scale), ctypes.byref(self.desc), workspace.data_ptr(),
                         workspace.numel())
        self.com_args = (p.q.data_ptr(), p.k_ext.data_ptr(), p.v_ext.data_ptr(), p.qo_indptr.data_ptr(),
                         p.kv_indptr.data_ptr(), p.l_ext, F(p.sm_scale), out.data_ptr(),
                         ctypes.byref(self.desc), workspace.data_ptr(), workspace.numel())

    def prefix(self, stream):
        rc = self.lib.verify_attn_prefix(*self.pre_args, stream)
        if rc:
            raise RuntimeError("verify_attn_prefix: %d %s" % (rc, self.lib.verify_attn_last_error()))

    def combine(self, stream):
        rc = self.lib.verify_attn_combine(*self.com_args, stream)
        if rc:
            raise RuntimeError("verify_attn_combine: %d %s" % (rc, self.lib.verify_attn_last_error()))


def timed_loop(torch, body, steps, warmup):
    """ms per iteration of body(i) over `steps` iterations on the current
    stream, right after `warmup` untimed iterations of the same body.  The
    warm-up keeps the GPU under the same load until the timed region starts:
    after an idle or lightly loaded gap its clocks come back over several
    milliseconds, and the first few hundred steps would time the ramp.  The
    host enqueues each step faster than the GPU runs it, so the stream never
    starves inside the timed region."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        body(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        body(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_workload(torch, va, W, name, steps, warmup, replicas, seed0=1000, capacity_factor=0):
    dev = torch.device("cuda", 0)
    make = W.CONFIGS[name]
    probs = [make(device=dev, seed=seed0 + r) for r in range(replicas)]
    p0 = probs[0]
    out = torch.empty(p0.q.shape[0], p0.h_q, p0.v_head_dim, dtype=torch.bfloat16, device=dev)
    desc = va.make_desc(p0.q, p0.k_ext, p0.v_ext, p0.k_buf, p0.v_buf, p0.kv_indices, out, p0.bs)
    plan = va.verify_attn_plan(desc, p0.l_ext)
    # replicas of a ragged workload differ in length: size for the largest plan
    ws_bytes = max(va.verify_attn_workspace_bytes(
        va.make_desc(p.q, p.k_ext, p.v_ext, p.k_buf, p.v_buf, p.kv_indices, out, p.bs), p.l_ext)
        for p in probs)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    runners = [Runner(va, p, ws, out) for p in probs]
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    # the timed loops rotate over the replicas: their mean size (ragged replicas differ)
    kv_bytes = sum(p.kv_bytes() for p in probs) / len(probs)

    def step(i):
        r = runners[i % replicas]
        r.prefix(sh)
        r.combine(sh)

    # ---- timed region: whole steps, rotating replicas (cold K/V) ----
    ms_step = timed_loop(torch, step, steps, warmup)

    # ---- prefix kernel alone, back to back ----
    ms_prefix_b2b = timed_loop(torch, lambda i: runners[i % replicas].prefix(sh), steps, warmup)

    # ---- per-kernel durations with events on the launch stream (the roofline's kernel time) ----
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    for i in range(steps):
        r = runners[i % replicas]
        ev[i][0].record(stream)
        r.prefix(sh)
        ev[i][1].record(stream)
        r.combine(sh)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    pre = [ev[i][0].elapsed_time(ev[i][1]) for i in range(steps)]
    com = [ev[i][1].elapsed_time(ev[i][2]) for i in range(steps)]
    call = sorted(ev[i][0].elapsed_time(ev[i][2]) for i in range(steps))

    # ---- warm cache: one replica over and over ----
    def warm_step(i):
        runners[0].prefix(sh)
        runners[0].combine(sh)
    ms_warm = timed_loop(torch, warm_step, steps, warmup)

    # ---- graph replay: one captured step per replica ----
    def capture(runner_list, steps_per_graph):
        """One graph per runner list entry, each holding `steps_per_graph`
        steps (rotating through the replicas from that entry on)."""
        out_graphs = []
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            for j in range(len(runner_list)):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    cs = torch.cuda.current_stream().cuda_stream
                    for k in range(steps_per_graph):
                        r = runner_list[(j + k) % len(runner_list)]
                        r.prefix(cs)
                        r.combine(cs)
                out_graphs.append(g)
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        return out_graphs

    def graph_loop(graphs, steps_per_graph):
        launches = max(1, steps // steps_per_graph)
        for i in range(max(1, warmup // steps_per_graph)):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(launches):
            graphs[i % len(graphs)].replay()
        e1.record(stream)
        host_us = (time.perf_counter() - t0) * 1e6 / launches
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (launches * steps_per_graph), host_us

    ms_graph = ms_graph20 = ms_graph_cap = ms_graph_cap20 = None
    host_graph_us = host_graph20_us = None
    try:
        ms_graph, host_graph_us = graph_loop(capture(runners, 1), 1)
        # 20 steps in one graph: the host launches once per 20 steps
        ms_graph20, host_graph20_us = graph_loop(capture(runners, 20), 20)
        if capacity_factor:
            # kv_indices a buffer of capacity_factor x the batch's tokens (the
            # graph mode of the pages' backend); the plan is made for its length
            caps = []
            for r in runners:
                buf = torch.zeros(capacity_factor * r.p.kv_indices.numel(), dtype=torch.int64, device=dev)
                buf[:r.p.kv_indices.numel()].copy_(r.p.kv_indices)
                caps.append(Runner(va, r.p, ws, out, kv_indices=buf))
            need = max(va.verify_attn_workspace_bytes(r.desc, r.p.l_ext) for r in caps)
            assert need <= ws.numel(), "capacity plan needs a larger workspace"
            ms_graph_cap, _ = graph_loop(capture(caps, 1), 1)
            ms_graph_cap20, _ = graph_loop(capture(caps, 20), 20)
    except Exception as exc:  # report, never hide
        print("graph replay timing failed: %r" % (exc,), file=sys.stderr)

    us = lambda ms: round(ms * 1e3, 3)
    pre_ms = statistics.mean(pre)
    return dict(
        name=name, problem=p0, plan=plan.as_dict(), kv_bytes=kv_bytes,
        ms_step=ms_step, us_step=us(ms_step), gbs=kv_bytes / (ms_step * 1e-3) / 1e9,
        prefix_us_mean=us(pre_ms), prefix_us_median=us(statistics.median(pre)),
        prefix_us_p10=us(sorted(pre)[len(pre) // 10]), prefix_us_p90=us(sorted(pre)[(9 * len(pre)) // 10]),
        combine_us_mean=us(statistics.mean(com)),
        call_us_median=us(statistics.median(call)), call_us_p10=us(call[len(call) // 10]),
        call_us_p90=us(call[(9 * len(call)) // 10]),
        prefix_gbs=kv_bytes / (pre_ms * 1e-3) / 1e9,
        prefix_us_b2b=us(ms_prefix_b2b), prefix_gbs_b2b=kv_bytes / (ms_prefix_b2b * 1e-3) / 1e9,
        us_step_warm=us(ms_warm), gbs_warm=kv_bytes / (ms_warm * 1e-3) / 1e9,
        us_step_graph=us(ms_graph) if ms_graph else None,
        gbs_graph=(kv_bytes / (ms_graph * 1e-3) / 1e9) if ms_graph else None,
        host_us_per_graph_launch=round(host_graph_us, 2) if host_graph_us else None,
        us_step_graph20=us(ms_graph20) if ms_graph20 else None,
        host_us_per_graph20_launch=round(host_graph20_us, 2) if host_graph20_us else None,
        us_step_graph_capacity=us(ms_graph_cap) if ms_graph_cap else None,
        us_step_graph_capacity20=us(ms_graph_cap20) if ms_graph_cap20 else None,
        capacity_factor=capacity_factor or None,
    )


def calibration_copy(torch):
    """A plain device copy of exactly 1 GiB; its FETCH_SIZE / WRITE_SIZE in a
    counter run give the scale factor for the prefix kernel's counters."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def _time_calls(torch, fn, steps, warmup):
    """Mean µs of fn(i) over `steps` calls through the Python binding, right
    after `warmup` untimed calls.  These calls marshal their arguments on the
    host each time, which takes about as long as a small kernel runs, so a
    short spin kernel (sized to the host's enqueue time for the timed calls)
    lets the host get ahead before the timed region starts."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    try:
        torch.cuda._sleep(int(max(1.0, 0.06 * steps) * 1e-3 * 2.4e9))  # ~60 us of host time per call
    except Exception:
        pass
    e0.record(stream)
    for i in range(steps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / steps


def time_extensions(torch, va, W, steps, warmup, replicas):
    """The paths around verify: tree-masked verify and page-table verify on
    the headline shape (cold, rotating replicas), the draft K/V append and the
    kv_indices build.  Returns a dict of µs and GB/s."""
    import numpy as np
    dev = torch.device("cuda", 0)
    res = {}
    probs = [W.config_b8_8k(device=dev, seed=3000 + r) for r in range(replicas)]
    p0 = probs[0]
    out = torch.empty(p0.q.shape[0], p0.h_q, p0.v_head_dim, dtype=torch.bfloat16, device=dev)
    desc = va.make_desc(p0.q, p0.k_ext, p0.v_ext, p0.k_buf, p0.v_buf, p0.kv_indices, out, p0.bs)
    ws = va.alloc_workspace(desc, p0.l_ext, dev)
    kvb = p0.kv_bytes()

    # tree verify: random draft trees (each node sees its ancestors)
    g = torch.Generator().manual_seed(1)
    L, n = p0.l_ext, p0.prefix_lens[0]
    parts, indptr = [], [0]
    for b in range(p0.bs):
        parent = [-1] + [int(torch.randint(-1, i, (1,), generator=g)) for i in range(1, L)]
        m = np.ones((L, n + L), np.uint8)
        m[:, n:] = 0
        for i in range(L):
            j = i
            while j >= 0:
                m[i, n + j] = 1
                j = parent[j]
        parts.append(m.reshape(-1))
        indptr.append(indptr[-1] + m.size)
    mask = torch.from_numpy(np.concatenate(parts)).to(dev)
    mi = torch.tensor(indptr, dtype=torch.int64, device=dev)
    us = _time_calls(torch, lambda i: va.verify_attn_run_tree(
        *(lambda p: (p.q, p.k_ext, p.v_ext, p.k_buf, p.v_buf, p.qo_indptr, p.kv_indptr, p.kv_indices,
                     p.l_ext, mask, mi, p.sm_scale, p.k_scale, p.v_scale))(probs[i % replicas]),
        out=out, workspace=ws, desc=desc), steps, warmup)
    res["tree_verify_b8_8k"] = {"us_per_call": round(us, 3), "gbs": round(kvb / us / 1e3, 2)}

    # page-table verify, 16-token pages over the same pool rows count
    P = 16
    pages = 2 * p0.bs * n // P
    tables = [W.make_paged_block_table(p.prefix_lens, P, pages, seed=10 + r, device=dev)
              for r, p in enumerate(probs)]
    us = _time_calls(torch, lambda i: va.verify_attn_run_paged(
        *(lambda p, t: (p.q, p.k_ext, p.v_ext, p.k_buf, p.v_buf, p.qo_indptr, p.kv_indptr, t, P, p.l_ext,
                        sum(p.prefix_lens), p.sm_scale, p.k_scale, p.v_scale))(probs[i % replicas],
                                                                              tables[i % replicas]),
        out=out, workspace=ws, desc=desc), steps, warmup)
    res["paged16_verify_b8_8k"] = {"us_per_call": round(us, 3), "gbs": round(kvb / us / 1e3, 2)}
    del probs, tables
    torch.cuda.empty_cache()

    # draft K/V append: the headline's draft rows, and a bulk append
    for tag, ntok, kv_dtype in (("append_fp8_32tok", 32, torch.float8_e4m3fn),
                                ("append_fp8_64k", 65536, torch.float8_e4m3fn),
                                ("append_bf16_64k", 65536, torch.bfloat16)):
        pool = 2 * ntok
        k = torch.randn(ntok, 2, 256, device=dev).to(torch.bfloat16)
        v = torch.randn(ntok, 2, 256, device=dev).to(torch.bfloat16)
        loc = torch.randperm(pool, device=dev)[:ntok]
        kb = torch.zeros(pool, 2, 256, device=dev).to(kv_dtype)
        vb = torch.zeros(pool, 2, 256, device=dev).to(kv_dtype)
        us = _time_calls(torch, lambda i: va.verify_attn_append_kv(k, v, loc, kb, vb, 0.05, 0.05), steps, warmup)
        eb = 1 if kv_dtype == torch.float8_e4m3fn else 2
        moved = ntok * 2 * 512 * (2 + eb) + ntok * 8
        res[tag] = {"us_per_call": round(us, 3), "gbs": round(moved / us / 1e3, 2), "bytes": moved}
        del k, v, loc, kb, vb

    # kv_indices build for the headline batch (8 x 8192 tokens)
    bs, n = 8, 8192
    rt = torch.randint(0, 1 << 30, (64, 16384), dtype=torch.int32, device=dev)
    rp = torch.randperm(64, device=dev)[:bs]
    sl = torch.full((bs,), n, dtype=torch.int32, device=dev)
    kvp = torch.empty(bs + 1, dtype=torch.int32, device=dev)
    kvi = torch.empty(bs * n, dtype=torch.int64, device=dev)
    us = _time_calls(torch, lambda i: va.verify_attn_build_kv_indices(rt, rp, sl, kvp, kvi), steps, warmup)
    moved = bs * n * (4 + 8)
    res["build_kv_indices_b8_8k"] = {"us_per_call": round(us, 3), "gbs": round(moved / us / 1e3, 2),
                                     "bytes": moved}
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(torch, W, p_dev, min_seconds=10.0, max_passes=8):
    """The fp64 oracle on the host cores over the whole headline batch, and on
    one thread over a bounded sample of it (sequence 0, every head)."""
    import oracle
    p = p_dev.to("cpu")
    args = (p.q, p.k_ext, p.v_ext, p.k_buf, p.v_buf, p.qo_indptr, p.kv_indptr, p.kv_indices,
            p.sm_scale, p.k_scale, p.v_scale)

    def median_time(select, budget):
        times = []
        t_start = time.perf_counter()
        while len(times) < max_passes and (time.perf_counter() - t_start) < budget:
            t0 = time.perf_counter()
            oracle.verify_attn(*args, select=select)
            times.append(time.perf_counter() - t0)
        return statistics.median(times), len(times)

    t, passes = median_time(None, min_seconds)
    cores = oracle.max_threads()
    # one thread, sequence 0 with all its heads: 1/bs of the batch
    sample = [(0, h) for h in range(p.h_q)]
    oracle.set_threads(1)
    try:
        t1, passes1 = median_time(sample, min_seconds / 2)
    finally:
        oracle.set_threads(cores)
    sample_bytes = p.kv_bytes() * p.prefix_lens[0] / max(1, sum(p.prefix_lens))
    return {
        "value": round(p.kv_bytes() / t / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "whole headline batch (all %d sequences x %d heads), median of %d passes; %.3f s/pass"
                  % (p.bs, p.h_q, passes, t),
        "us_per_call": round(t * 1e6, 1),
        "cpu_model": cpu_model(),
        "single_thread": {
            "value": round(sample_bytes / t1 / 1e9, 4),
            "unit": "GB/s",
            "sample": "sequence 0 x %d heads (1/%d of the batch) on one thread, median of %d passes; "
                      "%.3f s/pass" % (p.h_q, p.bs, passes1, t1),
        },
    }


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)
    import torch
    from speculative_decoding_attention_amd import verify_attn as va
    from speculative_decoding_attention_amd import workloads as W

    torch.cuda.set_device(0)
    calibration_copy(torch)
    torch.cuda.synchronize()
    head = time_workload(torch, va, W, args.workload, args.steps, args.warmup, args.replicas, capacity_factor=4)
    print("[bench] %s: %.2f us/step (%.1f GB/s), prefix kernel %.2f us with per-launch events "
          "(%.1f GB/s), %.2f us back to back; combine %.2f us"
          % (head["name"], head["us_step"], head["gbs"], head["prefix_us_mean"], head["prefix_gbs"],
             head["prefix_us_b2b"], head["combine_us_mean"]), file=sys.stderr, flush=True)

    secondary = {}
    if not args.quick:
        for name, reps in (("b4_64k", 1), ("fp8_ragged", 8), ("decode_b64", 2), ("decode_b512", 1),
                           ("draft_extend_b16", 8)):
            r = time_workload(torch, va, W, name, max(20, args.steps // 4), max(5, args.warmup // 4), reps,
                              seed0=2000)
            secondary[name] = {k: (round(v, 3) if isinstance(v, float) else v) for k, v in r.items()
                               if k not in ("problem", "name")}
            print("[bench] %s: %.2f us/step (%.1f GB/s), prefix %.2f us back to back (%.1f GB/s)"
                  % (name, r["us_step"], r["gbs"], r["prefix_us_b2b"], r["prefix_gbs_b2b"]),
                  file=sys.stderr, flush=True)
            del r
            torch.cuda.empty_cache()

    extensions = {}
    if not args.quick:
        extensions = time_extensions(torch, va, W, max(20, args.steps // 4), args.warmup, args.replicas)
        print("[bench] around verify: %s" % json.dumps(extensions), file=sys.stderr, flush=True)
        torch.cuda.empty_cache()

    cpu = None
    if not (args.quick or args.no_cpu_baseline):
        cpu = cpu_baseline(torch, W, head["problem"])
        print("[bench] cpu oracle: %s" % json.dumps(cpu), file=sys.stderr, flush=True)

    p = head["problem"]
    traffic = recorded_traffic(args.workload)
    lens = sorted(set(p.prefix_lens))
    prefix_desc = ("prefix %d each" % lens[0]) if len(lens) == 1 else (
        "prefix lengths %d..%d (seeded)" % (lens[0], lens[-1]))
    pool_desc = "%s pool (%s kv_indices)" % ("fp8 e4m3" if p.kv_fp8 else "bf16",
                                               "scattered" if p.k_buf.shape[0] > p.total_prefix else "contiguous")
    workload_desc = "%s: B=%d, %s, l_ext=%d, h_q=%d, h_kv=%d, D=Dv=%d, %s, k_scale=%g, v_scale=%g" % (
        args.workload, p.bs, prefix_desc, p.l_ext, p.h_q, p.h_kv, p.head_dim, pool_desc, p.k_scale, p.v_scale)
    qblocks = 1 if head["plan"]["rows"] <= 32 else 2
    kernel_desc = "prefix_kernel<%s, D=%d, %s>" % ("fp8" if p.kv_fp8 else "bf16", p.head_dim,
                                                    "one 32-row query block" if qblocks == 1 else
                                                    "two 32-row query blocks")
    achieved = head["prefix_gbs_b2b"]
    line = {
        "metric": "verify-attn achieved HBM GB/s and us/call (B=8, 8k prefix, l_ext=4, D=256)",
        "value": round(head["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_step"], 6),
        "us_per_call": head["us_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": workload_desc,
            "batch": p.bs, "prefix": p.prefix_lens[0], "l_ext": p.l_ext, "h_q": p.h_q,
            "h_kv": p.h_kv, "head_dim": p.head_dim, "kv_bytes": head["kv_bytes"],
            "cache": "cold (rotating %d replicas)" % args.replicas,
            "plan": head["plan"],
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": kernel_desc,
            "kernel_us": head["prefix_us_b2b"],
            "kernel_timing": "HIP events on the launch stream around %d back-to-back prefix launches "
                             "(cold, rotating replicas) after %d warm-up launches, per launch"
                             % (args.steps, args.warmup),
            "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
        },
        "cpu_baseline": cpu,
        "detail": {
            "prefix_us_back_to_back": head["prefix_us_b2b"],
            "prefix_us_per_launch_events": {"mean": head["prefix_us_mean"], "median": head["prefix_us_median"],
                                            "p10": head["prefix_us_p10"], "p90": head["prefix_us_p90"]},
            "combine_us_mean": head["combine_us_mean"],
            # one event pair around each whole call (both passes), cold
            "call_us_per_call_events": {"median": head["call_us_median"], "p10": head["call_us_p10"],
                                        "p90": head["call_us_p90"]},
            "warm_cache": {"us_per_call": head["us_step_warm"], "gbs": round(head["gbs_warm"], 2)},
            "graph_replay": {"us_per_call": head["us_step_graph"],
                             "gbs": round(head["gbs_graph"], 2) if head["gbs_graph"] else None,
                             "host_us_per_launch": head["host_us_per_graph_launch"],
                             "twenty_steps_per_graph_us_per_call": head["us_step_graph20"],
                             "host_us_per_twenty_step_launch": head["host_us_per_graph20_launch"],
                             "kv_indices_capacity_4x_us_per_call": head["us_step_graph_capacity"],
                             "kv_indices_capacity_4x_twenty_steps_per_graph_us_per_call":
                                 head["us_step_graph_capacity20"]},
            "secondary": secondary,
            "around_verify": extensions,
        },
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
