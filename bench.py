#!/usr/bin/env python3
"""Benchmark of the gfx950 fused attention forward (one GPU).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gqa|mla|mqa512|sparse|tiny]
                    [--primary-only] [--no-cpu-baseline] [--no-ceilings]

A step is one call of the library on one batch of synthetic, already
device-resident inputs: validation + plan + one kernel launch that runs the
whole forward (fold, Q/K/V staging, QK^T, mask, online softmax, PV,
epilogue). The primary line is the dense causal GQA prefill workload
(B=2 H=32 Hkv=8 T=4096 d=128 bf16); the other workloads are measured in the
same run and reported under "workloads" unless --primary-only is given.
Rows beyond the five ("next_rows", skipped with --no-next-rows): split-KV
decode (d512, beside the plain path), the dense backward on gqa / mla / mqa512 /
swa1024 (algorithmic flops = five products per visible pair), decode over a
q8_0 and a q4_0 cache (beside a bf16 cache), the packed variable-length
forward (beside the padded batch), MLA two-part rows (beside the concatenated
call), the sparse backward, the forward's extra returns (p, row_max), attention
dropout (forward and backward) and the sliding-window forward; and two
diagnostics of where the sparse forward's bytes come from (the Infinity
Cache cleared before each launch; a 1 GiB pool). Every workload line also
carries the sha256 of its generated inputs and, unless --no-cpu-baseline,
the fp64 oracle timed on the host over a bounded sample of it (the tiny
workload single-threaded over 100 repeats of its full output).

Warmup: at least W untimed steps and at least 0.2 s of them (the clocks
ramp over the first ~30 ms of load). Prints ONE JSON line on stdout. Kernel
durations come from HIP events
recorded around each launch on the stream the kernel runs on; ms_per_step is
wall time over the K timed steps, bracketed by device synchronisation.
Algorithmic work (what the method must do, not what the kernel happens to do):
  dense : flops = 2 * visible_pairs * (d_qk + d_v); bytes = q + k + v + out + lse (+ sinks)
  sparse: flops = 2 * Sq*Hq*topk * (d_qk + d_v); bytes = Sq*topk*d_qk*2 (each gathered
          pool row once, V == K) + q + out + indices + lse
Peaks (MI355X published): bf16 dense MFMA 2.5 PFLOP/s, HBM3E 8 TB/s.
Measured ceilings (context, not the metric): an MFMA-only 32x32x16 bf16 loop
and a 2 GiB streaming copy from libattn_ceiling.so, plus the peak computed from
the device's CU count and maximum clock; each roofline also reports its
fraction of the measured ceiling.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (% bf16 MFMA peak); sparse top-k GB/s (% HBM peak)"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
WORKLOAD_IDS = {"tiny": 1, "gqa": 2, "mla": 3, "mqa512": 4, "sparse": 5, "decode512": 6, "swa1024": 7}
RIDGE_FLOP_PER_BYTE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
# the forward kernels and the planner that orders their workgroups (which
# decides what shares an L2); recorded traffic counts only while these match
KERNEL_SOURCES = ("attention_forward_attn_amd/csrc/attn_kernels.hip",
                  "attention_forward_attn_amd/csrc/attn_params.h",
                  "attention_forward_attn_amd/csrc/api.cpp")


def log(msg):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def visible_pairs(B, H, Tq, Tk, causal, window=(-1, -1)) -> int:
    """(row, key) pairs the mask keeps: causal bottom-right, and a sliding window
    of (left, right) keys around the diagonal (-1: unbounded)."""
    if not causal and window == (-1, -1):
        return B * H * Tq * Tk
    off = Tk - Tq
    up = 0 if causal else window[1]
    tot = 0
    for t in range(Tq):
        hi = Tk - 1 if up < 0 else min(Tk - 1, t + off + up)
        lo = 0 if window[0] < 0 else max(0, t + off - window[0])
        tot += max(0, hi - lo + 1)
    return B * H * tot


def describe(n: int) -> str:
    import synth

    s = synth.spec(n)
    if s.kind == "dense":
        t = f"T={s.Tq}" if s.Tq == s.Tk else f"Tq={s.Tq} Tk={s.Tk}"
        w = "" if s.window == (-1, -1) else f" window=({s.window[0]},{s.window[1]})"
        return (f"{s.name}: dense causal B={s.B} H={s.H} Hkv={s.Hkv} {t} d_qk={s.d_qk} d_v={s.d_v} "
                f"{s.dtype}" + (" sinks" if s.sinks else "") + w)
    return f"{s.name}: sparse top-k Sq={s.Sq} Hq={s.Hq} N={s.N} d_qk={s.d_qk} d_v={s.d_v} topk={s.topk} bf16"


def work(n: int) -> dict:
    import synth

    s = synth.spec(n)
    if s.kind == "dense":
        elt = 2 if s.dtype == "bf16" else 4
        pairs = visible_pairs(s.B, s.H, s.Tq, s.Tk, s.causal, s.window)
        flops = 2 * pairs * (s.d_qk + s.d_v)
        nbytes = elt * (s.B * s.H * s.Tq * s.d_qk + s.B * s.Hkv * s.Tk * (s.d_qk + s.d_v)
                        + s.B * s.H * s.Tq * s.d_v) + 4 * s.B * s.H * s.Tq + (4 * s.H if s.sinks else 0)
    else:
        pairs = s.Sq * s.Hq * s.topk
        flops = 2 * pairs * (s.d_qk + s.d_v)
        nbytes = (2 * s.Sq * s.topk * s.d_qk + 2 * s.Sq * s.Hq * (s.d_qk + s.d_v) + 4 * s.Sq * s.topk
                  + 4 * s.Sq * s.Hq)
    return {"pairs": pairs, "flops": flops, "bytes": nbytes, "kind": s.kind}


def make_call(n: int, split: bool = False):
    """Device-resident inputs and outputs for workload n and a closure that runs one step
    (split: the split-KV call with a preallocated workspace)."""
    import torch

    import attention_forward_attn_amd as A
    import synth

    s = synth.spec(n)
    inp = synth.make(n)
    if s.kind == "dense":
        q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
        sk = inp["sinks"].cuda() if inp["sinks"] is not None else None
        out = torch.empty((s.B, s.H, s.Tq, s.d_v), dtype=q.dtype, device="cuda")
        lse = torch.empty((s.B, s.H, s.Tq), dtype=torch.float32, device="cuda")

        ws = None
        if split:
            nb = A.splitkv_workspace_bytes(s.B, s.H, s.Hkv, s.Tq, s.Tk, s.d_qk, s.d_v, dtype=s.dtype,
                                           causal=s.causal, sinks=s.sinks)
            ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")

        def step():
            if split:
                A.dense_splitkv(q, k, v, causal=s.causal, scale=s.scale, sinks=sk, out=out, lse=lse, workspace=ws,
                                window=s.window)
            else:
                A.dense(q, k, v, causal=s.causal, scale=s.scale, sinks=sk, out=out, lse=lse, window=s.window)

        path = A.plan_dense(s.B, s.H, s.Hkv, s.Tq, s.Tk, s.d_qk, s.d_v, dtype=s.dtype, sinks=s.sinks)["path"]
    else:
        q, kv, idx = inp["q"].cuda(), inp["kv"].cuda(), inp["idx"].cuda()
        out = torch.empty((s.Sq, s.Hq, s.d_v), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((s.Sq, s.Hq), dtype=torch.float32, device="cuda")

        def step():
            A.sparse_topk(q, kv, idx, d_v=s.d_v, scale=s.scale, out=out, lse=lse)

        path = A.plan_sparse_topk(s.Sq, s.Hq, s.N, s.d_qk, s.d_v, s.topk)["path"]
    return step, path, inp


# The GPU's clocks ramp up over the first ~30 ms of sustained load (measured:
# the first 40 launches of the gqa kernel averaged 301 us, the following ones
# 263 us), so the untimed warmup runs at least `warmup` steps and at least this
# long; the K timed steps then see the steady state a continuously loaded GPU runs at.
MIN_WARMUP_S = 0.2


def time_steps(step, steps: int, warmup: int) -> dict:
    import torch

    calls = 0
    for _ in range(warmup):
        step()
    calls += warmup
    torch.cuda.synchronize()
    t_end = time.perf_counter() + MIN_WARMUP_S
    while time.perf_counter() < t_end:
        for _ in range(max(1, warmup)):
            step()
        calls += max(1, warmup)
        torch.cuda.synchronize()
    calls += steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ks = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    return {"calls": calls, "ms_per_step": (t1 - t0) * 1e3 / steps, "kernel_ms_mean": sum(ks) / len(ks),
            "kernel_ms_median": ks[len(ks) // 2], "kernel_ms_min": ks[0]}


def roofline(n: int, kernel_ms: float) -> dict:
    w = work(n)
    # bound by whichever resource the algorithmic work saturates first
    # (ridge = peak flops / peak bytes = 312.5 flop/B): the prefill layers are
    # MFMA bound, decode and the sparse gather HBM bound
    if w["flops"] / w["bytes"] >= RIDGE_FLOP_PER_BYTE:
        ach = w["flops"] / (kernel_ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": traffic_for(n)}
    ach = w["bytes"] / (kernel_ms * 1e-3) / 1e9
    r = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
         "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic_for(n)}
    if w["kind"] == "sparse":
        r["rate"] = ("effective: algorithmic bytes / kernel time; the 64 MiB pool is served partly from the "
                     "Infinity Cache (1 GiB-pool diagnostic in next_rows)")
    return r


def traffic_for(n: int):
    """HBM bytes per launch from committed rocprofv3 counter summaries, when they were
    taken on the current kernel source (else null)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
    except Exception:
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    ent = rec.get("workloads", {}).get(str(n))
    return None if ent is None else ent.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(n: int, inp: dict, budget_s: float = 12.0) -> dict:
    """The fp64 oracle on a bounded sample of the same workload, timed on this host
    (BLAS on every core it is given; the tiny workload single-threaded over 100
    repeats of its full output)."""
    import numpy as np

    import oracle
    import synth

    s = synth.spec(n)
    if n == 1:
        from threadpoolctl import threadpool_limits

        reps = 100
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            for _ in range(reps):
                oracle.dense_attention(inp["q"], inp["k"], inp["v"], scale=s.scale, causal=s.causal)
            dt = time.perf_counter() - t0
        w = work(1)
        return {"value": round(w["flops"] * reps / dt / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
                "sample": f"the full workload (B1 H4 T128), {reps} repeats, single-threaded BLAS",
                "seconds": round(dt, 2), "ms_per_run": round(dt * 1e3 / reps, 3), "cpu_model": cpu_model()}
    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    done_flops = 0
    t0 = time.perf_counter()
    units = 0
    if s.kind == "dense":
        g = s.H // s.Hkv
        for b in range(s.B):
            for h in range(s.H):
                kvh = h // g
                oracle.dense_attention(inp["q"][b:b + 1, h:h + 1], inp["k"][b:b + 1, kvh:kvh + 1],
                                       inp["v"][b:b + 1, kvh:kvh + 1], scale=s.scale, causal=s.causal,
                                       sinks=None if inp["sinks"] is None else inp["sinks"][h:h + 1],
                                       window=s.window)
                done_flops += 2 * visible_pairs(1, 1, s.Tq, s.Tk, s.causal, s.window) * (s.d_qk + s.d_v)
                units += 1
                if time.perf_counter() - t0 > budget_s:
                    break
            if time.perf_counter() - t0 > budget_s:
                break
        sample = f"{units} of {s.B * s.H} (batch, head) pairs, full {s.Tq}x{s.Tk} causal rows each"
    else:
        step = 64
        for q0 in range(0, s.Sq, step):
            qs = list(range(q0, min(q0 + step, s.Sq)))
            oracle.sparse_topk_attention(inp["q"], inp["kv"], inp["idx"], d_v=s.d_v, scale=s.scale, queries=qs)
            done_flops += 2 * len(qs) * s.Hq * s.topk * (s.d_qk + s.d_v)
            units += len(qs)
            if time.perf_counter() - t0 > budget_s:
                break
        sample = f"{units} of {s.Sq} queries (all {s.Hq} heads, {s.topk} gathered rows each)"
    dt = time.perf_counter() - t0
    if s.kind == "dense":
        value, unit = done_flops / dt / 1e12, "TFLOP/s"
    else:
        w = work(n)
        value, unit = w["bytes"] * units / s.Sq / dt / 1e9, "GB/s"
    return {"value": round(value, 6), "unit": unit, "cores": cores, "kind": "oracle", "sample": sample,
            "seconds": round(dt, 2), "cpu_model": cpu_model()}


def inputs_sha256(inp: dict) -> dict:
    """sha256 of every generated input tensor (reproducibility record)."""
    import synth

    return {k: synth.sha256(v) for k, v in inp.items() if hasattr(v, "dtype")}


def measure(n: int, steps: int, warmup: int, split: bool = False) -> dict:
    import attention_forward_attn_amd as A

    step, path, inp = make_call(n, split)
    A.reset_dispatch_counts()
    t = time_steps(step, steps, warmup)
    launched = A.dispatch_count(path)
    # engagement census: the expected kernel path ran exactly once per step,
    # otherwise the numbers are not this path's and the run stops
    if launched != t["calls"]:
        raise RuntimeError(f"NotEngaged: expected {t['calls']} launches of {path}, saw {launched}")
    if split and A.dispatch_count("splitkv_merge") != t["calls"]:
        raise RuntimeError("NotEngaged: the split-KV merge did not run once per step")
    w = work(n)
    rl = roofline(n, t["kernel_ms_mean"])
    if rl["bound"] == "mfma":
        value, unit = w["flops"] / (t["ms_per_step"] * 1e-3) / 1e12, "TFLOP/s"
    else:
        value, unit = w["bytes"] / (t["ms_per_step"] * 1e-3) / 1e9, "GB/s"
    log(f"[bench] {describe(n)} | path {path}{' split-KV' if split else ''} | kernel {t['kernel_ms_mean']:.4f} ms (median "
        f"{t['kernel_ms_median']:.4f}) | step {t['ms_per_step']:.4f} ms | {rl['achieved']} {rl['unit']} "
        f"= {100 * rl['frac']:.1f}% of peak")
    return {"n": n, "path": path, "timing": t, "value": value, "unit": unit, "roofline": rl, "inp": inp,
            "verdict": "Measured"}


def _event_ms(fn, before=None, steps: int = 10) -> list:
    """HIP-event durations of `fn` launches on torch's current stream (the stream the
    library launches on); `before` runs untimed ahead of each launch."""
    import torch

    out = []
    for _ in range(steps):
        if before is not None:
            before()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        e1.synchronize()
        out.append(e0.elapsed_time(e1))
    return out


SCRUB_MIB = 512
BIG_POOL_ROWS = 1 << 20


def measure_sparse_diagnostic(kind: str, steps: int, warmup: int) -> dict:
    """Where workload 5's bytes come from. Its 64 MiB pool fits the 256 MB Infinity
    Cache, so its GB/s is an effective gather rate. Two diagnostics with the same
    queries, top-k and algorithmic bytes (31.53 GB per launch):
      scrub  -- 512 MiB written by a device fill before every timed launch, so each
                launch starts with the pool, q and the indices out of the cache;
      pool1g -- a pool of 2^20 rows (1 GiB, four times the cache), indices drawn
                like the workload's from [0, 2^20) (numpy default_rng(5)), pool rows
                N(0,1) from a device generator seeded with 5: most gathers miss."""
    import numpy as np
    import torch

    import attention_forward_attn_amd as A
    import synth

    s = synth.spec(5)
    w = work(5)
    if kind == "scrub":
        step, path, inp = make_call(5)
        junk = torch.empty(SCRUB_MIB << 20, dtype=torch.uint8, device="cuda")
        before = lambda: junk.fill_(1)  # noqa: E731
        desc = describe(5) + f", {SCRUB_MIB} MiB written before each launch"
    elif kind == "pool1g":
        inp = synth.make(5)
        q = inp["q"].cuda()
        del inp
        g = torch.Generator(device="cuda").manual_seed(5)
        kv = torch.randn((BIG_POOL_ROWS, s.d_qk), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        idx = torch.from_numpy(synth.make_indices(s.Sq, BIG_POOL_ROWS, s.topk, 5)).cuda()
        out = torch.empty((s.Sq, s.Hq, s.d_v), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((s.Sq, s.Hq), dtype=torch.float32, device="cuda")

        def step():
            A.sparse_topk(q, kv, idx, d_v=s.d_v, scale=s.scale, out=out, lse=lse)

        path = A.plan_sparse_topk(s.Sq, s.Hq, BIG_POOL_ROWS, s.d_qk, s.d_v, s.topk)["path"]
        before = None
        desc = describe(5).replace(f"N={s.N}", f"N={BIG_POOL_ROWS}") + " (1 GiB pool)"
    else:
        raise ValueError(kind)
    A.reset_dispatch_counts()
    _event_ms(step, before, max(2, warmup))
    t_end = time.perf_counter() + MIN_WARMUP_S
    while time.perf_counter() < t_end:
        _event_ms(step, before, 1)
    ms = sorted(_event_ms(step, before, steps))
    mean = sum(ms) / len(ms)
    gbs = w["bytes"] / (mean * 1e-3) / 1e9
    log(f"[bench] {desc} | kernel {mean:.4f} ms (median {ms[len(ms) // 2]:.4f}) | {gbs:.1f} GB/s = "
        f"{100 * gbs / PEAK_HBM_GBS:.1f}% of 8 TB/s")
    return {"row": f"sparse top-k diagnostic: {kind}", "workload": desc, "path": path, "value": round(gbs, 1),
            "unit": "GB/s", "kernel_ms": round(mean, 5), "kernel_ms_median": round(ms[len(ms) // 2], 5),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None},
            "verdict": "Measured" if A.dispatch_count(path) > 0 else "NotEngaged"}


def bwd_flops(n: int) -> int:
    """Algorithmic flops of the backward: five products per visible pair (S recomputed,
    dP = dO V^T, dV = P^T dO, dK = dS^T Q, dQ = dS K), i.e. 2 * pairs * (3 d_qk + 2 d_v)."""
    import synth

    s = synth.spec(n)
    return 2 * visible_pairs(s.B, s.H, s.Tq, s.Tk, s.causal, s.window) * (3 * s.d_qk + 2 * s.d_v)


def bwd_path_name(d_qk: int, d_v: int) -> str:
    return f"dense_bwd_bf16_d{d_qk}" + ("" if d_qk == d_v else f"_v{d_v}")


def measure_bwd(n: int, steps: int, warmup: int) -> dict:
    """The dense backward (all four launches) on workload n, after one forward that
    supplies out and lse; dL/dO is the seeded synthetic gradient."""
    import torch

    import attention_forward_attn_amd as A
    import synth

    s = synth.spec(n)
    inp = synth.make(n)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    sk = inp["sinks"].cuda() if inp["sinks"] is not None else None
    out, lse = A.dense(q, k, v, causal=s.causal, scale=s.scale, sinks=sk, window=s.window)
    dout = synth.make_dout(s).cuda()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dsk = torch.empty_like(sk) if sk is not None else None
    ws = torch.empty(max(16, A.bwd_workspace_bytes(s.B, s.H, s.Hkv, s.Tq, s.Tk, s.d_qk, s.d_v)), dtype=torch.uint8,
                     device="cuda")
    torch.cuda.synchronize()

    def step():
        A.dense_backward(q, k, v, out, dout, lse, causal=s.causal, scale=s.scale, sinks=sk, dq=dq, dk=dk, dv=dv,
                         dsinks=dsk, workspace=ws, window=s.window)

    path = bwd_path_name(s.d_qk, s.d_v)
    A.reset_dispatch_counts()
    t = time_steps(step, steps, warmup)
    if A.dispatch_count(path) != t["calls"]:
        raise RuntimeError(f"NotEngaged: expected {t['calls']} launches of {path}, saw {A.dispatch_count(path)}")
    fl = bwd_flops(n)
    ach = fl / (t["kernel_ms_mean"] * 1e-3) / 1e12
    rl = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
          "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None}
    value = fl / (t["ms_per_step"] * 1e-3) / 1e12
    log(f"[bench] backward {describe(n)} | path {path} | {t['kernel_ms_mean']:.4f} ms per backward (4 launches) "
        f"| {rl['achieved']} TFLOP/s = {100 * rl['frac']:.1f}% of peak")
    return {"row": "dense backward (attn_bwd_dense)", "workload": describe(n), "path": path,
            "value": round(value, 3), "unit": "TFLOP/s", "kernel_ms": round(t["kernel_ms_mean"], 5),
            "roofline": rl, "verdict": "Measured"}


def sparse_bwd_flops(n: int) -> int:
    """Algorithmic flops of the sparse backward: five products per (query, head, slot)
    (S recomputed, dP, dq, the key-role and value-role pool gradients)."""
    import synth

    s = synth.spec(n)
    return 2 * s.Sq * s.Hq * s.topk * (3 * s.d_qk + 2 * s.d_v)


def measure_sparse_bwd(steps: int, warmup: int) -> dict:
    """The sparse top-k backward on workload 5 (after one forward for out and lse);
    dL/dO is the seeded synthetic gradient. All four launches are timed."""
    import torch

    import attention_forward_attn_amd as A
    import synth

    s = synth.spec(5)
    inp = synth.make(5)
    q, kv, idx = inp["q"].cuda(), inp["kv"].cuda(), inp["idx"].cuda()
    out, lse = A.sparse_topk(q, kv, idx, d_v=s.d_v, scale=s.scale)
    dout = synth.make_sparse_dout(s).cuda()
    dq = torch.empty_like(q)
    dkv = torch.empty((s.N, s.d_qk), dtype=torch.float32, device="cuda")
    ws = torch.empty(s.Sq * s.Hq * 4 + 256, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    def step():
        A.sparse_backward(q, kv, idx, out, dout, lse, d_v=s.d_v, scale=s.scale, dq=dq, dkv=dkv, workspace=ws)

    path = "sparse_bwd_bf16_d512"
    A.reset_dispatch_counts()
    t = time_steps(step, steps, warmup)
    if A.dispatch_count(path) != t["calls"]:
        raise RuntimeError(f"NotEngaged: expected {t['calls']} launches of {path}, saw {A.dispatch_count(path)}")
    fl = sparse_bwd_flops(5)
    ach = fl / (t["kernel_ms_mean"] * 1e-3) / 1e12
    rl = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
          "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None}
    log(f"[bench] sparse backward {describe(5)} | path {path} | {t['kernel_ms_mean']:.4f} ms per backward "
        f"(4 launches) | {rl['achieved']} TFLOP/s = {100 * rl['frac']:.1f}% of peak")
    return {"row": "sparse top-k backward (attn_bwd_sparse_topk)", "workload": describe(5), "path": path,
            "value": round(fl / (t["ms_per_step"] * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
            "kernel_ms": round(t["kernel_ms_mean"], 5), "roofline": rl, "verdict": "Measured"}


def measure_qkv(fmt: str, steps: int, warmup: int) -> dict:
    """Multi-sequence decode over a quantized cache (synth.QUANT_DECODE shape in
    ``fmt``), memory bound: bytes = q + the cache's raw K/V bytes + out + lse. The
    same shape over a bf16 cache (split-KV forward) is timed beside it."""
    import torch

    import attention_forward_attn_amd as A
    import synth

    s = dict(synth.QUANT_DECODE, fmt=fmt)
    inp = synth.make_quant_kv(s["B"], s["H"], s["Hkv"], s["Tq"], s["Tk"], s["d"], fmt, seed=s["seed"])
    q, k, v = inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda()
    B, H, Tq, d = q.shape
    out = torch.empty((B, H, Tq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device="cuda")
    a = A.qkv_args(q, k, v, out, lse, fmt=fmt, causal=True, scale=1 / math.sqrt(d))
    ws = torch.empty(max(16, int(A.load_library().attn_qkv_workspace_bytes(a, 0))), dtype=torch.uint8, device="cuda")

    def step():
        A.dense_qkv(q, k, v, fmt=fmt, causal=True, out=out, lse=lse, workspace=ws)

    path = f"dense_qkv_{fmt}_d{d}"
    A.reset_dispatch_counts()
    t = time_steps(step, steps, warmup)
    if A.dispatch_count(path) != t["calls"]:
        raise RuntimeError(f"NotEngaged: expected {t['calls']} launches of {path}, saw {A.dispatch_count(path)}")
    nbytes = (2 * B * H * Tq * d * 2 + k.numel() + v.numel() + 4 * B * H * Tq)
    ach = nbytes / (t["kernel_ms_mean"] * 1e-3) / 1e9
    rl = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
          "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None}
    # the same decode over a bf16 cache, for context
    g = torch.Generator("cpu").manual_seed(s["seed"])
    kf = torch.randn((B, s["Hkv"], s["Tk"], d), generator=g).to(torch.bfloat16).cuda()
    vf = torch.randn((B, s["Hkv"], s["Tk"], d), generator=g).to(torch.bfloat16).cuda()
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    ws2 = torch.empty(max(16, A.splitkv_workspace_bytes(B, H, s["Hkv"], Tq, s["Tk"], d, d)), dtype=torch.uint8,
                      device="cuda")
    t2 = time_steps(lambda: A.dense_splitkv(q, kf, vf, causal=True, out=out2, lse=lse2, workspace=ws2), steps, warmup)
    log(f"[bench] qdecode {fmt}: B={B} H={H} Hkv={s['Hkv']} Tq={Tq} Tk={s['Tk']} d={d} | path {path} | "
        f"{t['kernel_ms_mean']:.4f} ms | {rl['achieved']} GB/s = {100 * rl['frac']:.1f}% of peak | bf16 cache "
        f"{t2['kernel_ms_mean']:.4f} ms")
    return {"row": f"decode over a {fmt} K/V cache (attn_fwd_dense_qkv), in-kernel dequant",
            "workload": f"qdecode: causal B={B} H={H} Hkv={s['Hkv']} Tq={Tq} Tk={s['Tk']} d={d} {fmt} K/V, bf16 q/out",
            "path": path + " + splitkv_merge", "value": round(nbytes / (t["ms_per_step"] * 1e-3) / 1e9, 1),
            "unit": "GB/s", "kernel_ms": round(t["kernel_ms_mean"], 5), "roofline": rl, "verdict": "Measured",
            "bf16_cache": {"path": "dense_bf16_d128 split-KV", "kernel_ms": round(t2["kernel_ms_mean"], 5)}}


def measure_varlen(steps: int, warmup: int) -> dict:
    """The packed variable-length forward on synth.VARLEN_PREFILL (the gqa layer over
    sequences of mixed lengths); flops = 2 * (visible pairs summed over the sequences)
    * (d_qk + d_v). The padded batch (every sequence at the longest length, one dense
    call) is timed beside it."""
    import torch

    import attention_forward_attn_amd as A
    import synth

    s = synth.VARLEN_PREFILL
    inp = synth.make_varlen(s)
    q, k, v = inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda()
    cu = torch.from_numpy(inp["cu"]).cuda()
    lens = [int(x) for x in inp["lens"]]
    H, Hkv, d = s["H"], s["Hkv"], s["d"]
    scale = 1 / math.sqrt(d)
    out = torch.empty((q.shape[0], H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, q.shape[0]), dtype=torch.float32, device="cuda")
    mx = max(lens)

    def step():
        A.dense_varlen(q, k, v, cu, cu, mx, causal=True, scale=scale, out=out, lse=lse)

    path = f"dense_bf16_d{d}"
    A.reset_dispatch_counts()
    t = time_steps(step, steps, warmup)
    if A.dispatch_count(path) != t["calls"]:
        raise RuntimeError(f"NotEngaged: expected {t['calls']} launches of {path}, saw {A.dispatch_count(path)}")
    fl = sum(2 * visible_pairs(1, H, L, L, True) * 2 * d for L in lens)
    ach = fl / (t["kernel_ms_mean"] * 1e-3) / 1e12
    rl = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
          "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None}
    # the padded batch: [n, H, max, d], each sequence's rows first and N(0,1) padding
    # after them (MFMA timing depends on the data, so no zero padding), one dense call
    n = len(lens)
    gp = torch.Generator("cpu").manual_seed(s["seed"] + 1)
    pq = torch.randn((n, H, mx, d), generator=gp).to(torch.bfloat16)
    pk = torch.randn((n, Hkv, mx, d), generator=gp).to(torch.bfloat16)
    pv = torch.randn((n, Hkv, mx, d), generator=gp).to(torch.bfloat16)
    for i, L in enumerate(lens):
        a, e = int(inp["cu"][i]), int(inp["cu"][i + 1])
        pq[i, :, :L] = inp["q"][a:e].transpose(0, 1)
        pk[i, :, :L] = inp["k"][a:e].transpose(0, 1)
        pv[i, :, :L] = inp["v"][a:e].transpose(0, 1)
    pq, pk, pv = pq.cuda(), pk.cuda(), pv.cuda()
    po = torch.empty_like(pq)
    pl = torch.empty((n, H, mx), dtype=torch.float32, device="cuda")
    t2 = time_steps(lambda: A.dense(pq, pk, pv, causal=True, scale=scale, out=po, lse=pl), steps, warmup)
    del pq, pk, pv, po, pl
    log(f"[bench] varlen: {n} sequences, lengths {lens}, H={H}/{Hkv} d={d} causal | path {path} (packed) | "
        f"{t['kernel_ms_mean']:.4f} ms | {rl['achieved']} TFLOP/s = {100 * rl['frac']:.1f}% of peak | padded batch "
        f"{t2['kernel_ms_mean']:.4f} ms")
    return {"row": "packed variable-length forward (attn_fwd_varlen)",
            "workload": f"varlen: causal packed batch of {n} sequences (lengths {lens}, total {sum(lens)}) "
                        f"H={H} Hkv={Hkv} d={d} bf16",
            "path": path + " (packed)", "value": round(fl / (t["ms_per_step"] * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
            "kernel_ms": round(t["kernel_ms_mean"], 5), "roofline": rl, "verdict": "Measured",
            "padded_batch": {"path": path, "shape": f"B={n} T={mx}", "kernel_ms": round(t2["kernel_ms_mean"], 5)}}


def measure_two_part(steps: int, warmup: int) -> dict:
    """The MLA workload (3) with the query and key rows in two parts read in place:
    q / k no-rope [.., 128] and rope [.., 64] as strided views of the workload's
    tensors, the rope key of kv head 0 shared by all heads (an expanded view).
    Same algorithmic flops as workload 3; the concatenated call on the same values
    is timed beside it."""
    import torch

    import attention_forward_attn_amd as A
    import synth

    s = synth.spec(3)
    inp = synth.make(3)
    q, k, v = inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda()
    dn = 128
    qn, qr, kn = q[..., :dn], q[..., dn:], k[..., :dn]
    kr = k[:, :1, :, dn:].expand(s.B, s.Hkv, s.Tk, s.d_qk - dn)
    out = torch.empty((s.B, s.H, s.Tq, s.d_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((s.B, s.H, s.Tq), dtype=torch.float32, device="cuda")

    def step():
        A.dense(qn, kn, v, causal=True, scale=s.scale, out=out, lse=lse, q_rope=qr, k_rope=kr)

    path = "dense_bf16_d192_v128_rope64"
    A.reset_dispatch_counts()
    t = time_steps(step, steps, warmup)
    if A.dispatch_count(path) != t["calls"]:
        raise RuntimeError(f"NotEngaged: expected {t['calls']} launches of {path}, saw {A.dispatch_count(path)}")
    fl = work(3)["flops"]
    ach = fl / (t["kernel_ms_mean"] * 1e-3) / 1e12
    rl = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
          "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None}
    qc, kc = torch.cat([qn, qr], -1), torch.cat([kn, kr], -1)
    t2 = time_steps(lambda: A.dense(qc, kc, v, causal=True, scale=s.scale, out=out, lse=lse), steps, warmup)
    log(f"[bench] two-part mla: {describe(3)}, rope key shared | path {path} | {t['kernel_ms_mean']:.4f} ms | "
        f"{rl['achieved']} TFLOP/s = {100 * rl['frac']:.1f}% of peak | concatenated rows {t2['kernel_ms_mean']:.4f} ms")
    return {"row": "MLA two-part rows read in place (attn_fwd_dense with q_rope / k_rope)",
            "workload": describe(3) + ", q/k as no-rope 128 + rope 64 views, rope key shared by the heads",
            "path": path, "value": round(fl / (t["ms_per_step"] * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
            "kernel_ms": round(t["kernel_ms_mean"], 5), "roofline": rl, "verdict": "Measured",
            "concatenated": {"path": "dense_bf16_d192_v128", "kernel_ms": round(t2["kernel_ms_mean"], 5)}}


def measure_extras(steps: int, warmup: int) -> dict:
    """The forward's extra returns on the gqa workload (2): probabilities (fp32, every
    (row, key) pair written, masked ones as 0) and row maxima, from q, k and the
    forward's lse. HBM bound: bytes = p + q + k + lse + row_max."""
    import torch

    import attention_forward_attn_amd as A
    import synth

    s = synth.spec(2)
    inp = synth.make(2)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    out, lse = A.dense(q, k, v, causal=True, scale=s.scale)
    p = torch.empty((s.B, s.H, s.Tq, s.Tk), dtype=torch.float32, device="cuda")
    rm = torch.empty((s.B, s.H, s.Tq), dtype=torch.float32, device="cuda")

    def step():
        A.dense_extras(q, k, v, out, lse, causal=True, scale=s.scale, p=p, row_max=rm)

    path = "dense_extras_bf16"
    A.reset_dispatch_counts()
    t = time_steps(step, steps, warmup)
    if A.dispatch_count(path) != t["calls"]:
        raise RuntimeError(f"NotEngaged: expected {t['calls']} launches of {path}, saw {A.dispatch_count(path)}")
    nbytes = p.numel() * 4 + q.numel() * 2 + k.numel() * 2 + 2 * lse.numel() * 4
    ach = nbytes / (t["kernel_ms_mean"] * 1e-3) / 1e9
    rl = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
          "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None}
    t2 = time_steps(lambda: A.dense_extras(q, k, v, out, lse, causal=True, scale=s.scale, want_p=False, row_max=rm),
                    steps, warmup)
    del p
    log(f"[bench] extras: {describe(2)} | path {path} | p + row_max {t['kernel_ms_mean']:.4f} ms | "
        f"{rl['achieved']} GB/s = {100 * rl['frac']:.1f}% of peak | row_max only {t2['kernel_ms_mean']:.4f} ms")
    return {"row": "the forward's extra returns p, row_max (attn_fwd_dense_extras)", "workload": describe(2),
            "path": path, "value": round(nbytes / (t["ms_per_step"] * 1e-3) / 1e9, 1), "unit": "GB/s",
            "kernel_ms": round(t["kernel_ms_mean"], 5), "roofline": rl, "verdict": "Measured",
            "row_max_only": {"kernel_ms": round(t2["kernel_ms_mean"], 5)}}


def measure_dropout(steps: int, warmup: int) -> dict:
    """Attention dropout (p = 0.1, the caller's keep mask) on the gqa workload (2), and
    beside it on the 512-wide MQA workload (4): the forward and the backward with the
    same mask. Flops as the dense paths (the mask adds no products); the fused forward
    without dropout is the comparison."""
    import torch

    import attention_forward_attn_amd as A
    import synth

    s = synth.spec(2)
    inp = synth.make(2)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    kw = synth.pack_keep(synth.make_keep(s.B, s.H, s.Tq, s.Tk, 0.1, seed=2)).cuda()
    out = torch.empty_like(q)
    lse = torch.empty((s.B, s.H, s.Tq), dtype=torch.float32, device="cuda")
    A.reset_dispatch_counts()
    t = time_steps(lambda: A.dense(q, k, v, causal=True, scale=s.scale, out=out, lse=lse, keep=kw, p_drop=0.1),
                   steps, warmup)
    if A.dispatch_count("dense_dropout_bf16") != t["calls"]:
        raise RuntimeError("NotEngaged: the dropout forward did not run once per step")
    dout = synth.make_dout(s).cuda()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(16, A.bwd_workspace_bytes(s.B, s.H, s.Hkv, s.Tq, s.Tk, s.d_qk, s.d_v)), dtype=torch.uint8,
                     device="cuda")
    tb = time_steps(lambda: A.dense_backward(q, k, v, out, dout, lse, causal=True, scale=s.scale, dq=dq, dk=dk,
                                             dv=dv, workspace=ws, keep=kw, p_drop=0.1), steps, warmup)
    fl = work(2)["flops"]
    ach = fl / (t["kernel_ms_mean"] * 1e-3) / 1e12
    rl = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
          "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None}
    bach = bwd_flops(2) / (tb["kernel_ms_mean"] * 1e-3) / 1e12
    log(f"[bench] dropout p=0.1: {describe(2)} | forward {t['kernel_ms_mean']:.4f} ms = {rl['achieved']} TFLOP/s | "
        f"backward {tb['kernel_ms_mean']:.4f} ms = {bach:.1f} TFLOP/s")
    # the same on the 512-wide MQA workload (4, with sinks): the fused 512-wide
    # forward with the mask applied inside, then the 512-wide backward kernels
    s4 = synth.spec(4)
    inp4 = synth.make(4)
    q4, k4, v4 = (inp4[x].cuda() for x in ("q", "k", "v"))
    sk4 = inp4["sinks"].cuda()
    kw4 = synth.pack_keep(synth.make_keep(s4.B, s4.H, s4.Tq, s4.Tk, 0.1, seed=4)).cuda()
    out4 = torch.empty((s4.B, s4.H, s4.Tq, s4.d_v), dtype=torch.bfloat16, device="cuda")
    lse4 = torch.empty((s4.B, s4.H, s4.Tq), dtype=torch.float32, device="cuda")
    A.reset_dispatch_counts()
    t4 = time_steps(lambda: A.dense(q4, k4, v4, causal=True, scale=s4.scale, sinks=sk4, out=out4, lse=lse4, keep=kw4,
                                    p_drop=0.1), steps, warmup)
    if A.dispatch_count("dense_bf16_d512_dropout") != t4["calls"]:
        raise RuntimeError("NotEngaged: the fused 512-wide dropout forward did not run once per step")
    dout4 = synth.make_dout(s4).cuda()
    dq4, dk4, dv4, dsk4 = torch.empty_like(q4), torch.empty_like(k4), torch.empty_like(v4), torch.empty_like(sk4)
    ws4 = torch.empty(max(16, A.bwd_workspace_bytes(s4.B, s4.H, s4.Hkv, s4.Tq, s4.Tk, s4.d_qk, s4.d_v)),
                      dtype=torch.uint8, device="cuda")
    tb4 = time_steps(lambda: A.dense_backward(q4, k4, v4, out4, dout4, lse4, causal=True, scale=s4.scale, sinks=sk4,
                                              dq=dq4, dk=dk4, dv=dv4, dsinks=dsk4, workspace=ws4, keep=kw4,
                                              p_drop=0.1), steps, warmup)
    f4 = work(4)["flops"] / (t4["kernel_ms_mean"] * 1e-3) / 1e12
    b4 = bwd_flops(4) / (tb4["kernel_ms_mean"] * 1e-3) / 1e12
    log(f"[bench] dropout p=0.1: {describe(4)} | forward {t4['kernel_ms_mean']:.4f} ms = {f4:.1f} TFLOP/s"
        f" | backward {tb4['kernel_ms_mean']:.4f} ms = {b4:.1f} TFLOP/s")
    return {"row": "attention dropout, keep mask shared by forward and backward", "workload": describe(2) + ", p=0.1",
            "path": "dense_dropout_bf16", "value": round(fl / (t["ms_per_step"] * 1e-3) / 1e12, 3),
            "unit": "TFLOP/s", "kernel_ms": round(t["kernel_ms_mean"], 5), "roofline": rl, "verdict": "Measured",
            "backward": {"path": "dense_bwd_bf16_d128 (dropout)", "kernel_ms": round(tb["kernel_ms_mean"], 5),
                         "tflops": round(bach, 2)},
            "mqa512": {"workload": describe(4) + ", p=0.1",
                       "forward": {"path": "dense_bf16_d512_dropout", "kernel_ms": round(t4["kernel_ms_mean"], 5),
                                   "tflops": round(f4, 2)},
                       "backward": {"path": "dense_bwd_bf16_d512 (dropout)", "kernel_ms": round(tb4["kernel_ms_mean"], 5),
                                    "tflops": round(b4, 2)}}}


def measure_sparse_fp8(steps: int, warmup: int) -> dict:
    """Sparse top-k decode over an fp8 pool (synth.SPARSE_FP8_DECODE: 128 queries x 64
    heads, top-k 2048 of 65536 rows), HBM bound: bytes = gathered codes (512 B per
    slot) and scales (16 B per slot) + q + out + indices + lse. Beside it: the bf16
    sparse path over the same pool decoded to bf16, and the sparse prefill shape
    (workload 5's sizes) over an fp8 pool against the bf16 path."""
    import torch

    import attention_forward_attn_amd as A
    import synth

    s = synth.SPARSE_FP8_DECODE
    res = {}
    for tag, Sq in (("decode", s["Sq"]), ("prefill", synth.spec(5).Sq)):
        inp = synth.make_sparse_fp8(Sq, s["Hq"], s["N"], s["d"], s["topk"] if tag == "decode" else synth.spec(5).topk,
                                    seed=s["seed"])
        q, codes, scales, idx = inp["q"].cuda(), inp["codes"].cuda(), inp["scales"].cuda(), inp["idx"].cuda()
        topk = idx.shape[1]
        scale = 1 / math.sqrt(s["d"])
        out = torch.empty((Sq, s["Hq"], s["d"]), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((Sq, s["Hq"]), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(16, A.sparse_fp8_workspace_bytes(Sq, s["Hq"], s["N"], s["d"], topk)), dtype=torch.uint8,
                         device="cuda")
        A.reset_dispatch_counts()
        t = time_steps(lambda: A.sparse_fp8(q, codes, scales, idx, scale=scale, out=out, lse=lse, workspace=ws),
                       steps, warmup)
        if A.dispatch_count("sparse_fp8_d512") != t["calls"]:
            raise RuntimeError("NotEngaged: the fp8 sparse decode did not run once per step")
        nbytes = Sq * topk * (s["d"] + 16) + 2 * q.numel() * 2 + idx.numel() * 4 + lse.numel() * 4
        # the same attention over the pool decoded to bf16, on the bf16 sparse path
        pool = (codes.cpu().view(torch.float8_e4m3fn).float()
                * scales.cpu().repeat_interleave(128, dim=1)).to(torch.bfloat16).cuda()
        t2 = time_steps(lambda: A.sparse_topk(q, pool, idx, d_v=s["d"], scale=scale, out=out, lse=lse), steps, warmup)
        res[tag] = (t, nbytes, t2, Sq, topk)
        del q, codes, scales, idx, out, lse, ws, pool
        torch.cuda.empty_cache()
    t, nbytes, t2, Sq, topk = res["decode"]
    ach = nbytes / (t["kernel_ms_mean"] * 1e-3) / 1e9
    rl = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
          "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None}
    tp, nbp, t2p, Sqp, topkp = res["prefill"]
    achp = nbp / (tp["kernel_ms_mean"] * 1e-3) / 1e9
    log(f"[bench] sparse fp8 decode: Sq={Sq} Hq={s['Hq']} N={s['N']} topk={topk} | path sparse_fp8_d512 + merge | "
        f"{t['kernel_ms_mean']:.4f} ms | {rl['achieved']} GB/s = {100 * rl['frac']:.1f}% of peak | bf16 pool "
        f"{t2['kernel_ms_mean']:.4f} ms | prefill shape Sq={Sqp}: fp8 {tp['kernel_ms_mean']:.3f} ms ({achp:.0f} GB/s) "
        f"vs bf16 {t2p['kernel_ms_mean']:.3f} ms")
    return {"row": "sparse top-k decode over an fp8 pool (attn_fwd_sparse_fp8), in-kernel dequant",
            "workload": f"fp8decode: Sq={Sq} Hq={s['Hq']} N={s['N']} d=512 topk={topk}, E4M3 codes + fp32 scale "
                        f"per 128 columns",
            "path": "sparse_fp8_d512 + splitkv_merge", "value": round(nbytes / (t["ms_per_step"] * 1e-3) / 1e9, 1),
            "unit": "GB/s", "kernel_ms": round(t["kernel_ms_mean"], 5), "roofline": rl, "verdict": "Measured",
            "bf16_pool": {"path": "sparse_bf16_d512", "kernel_ms": round(t2["kernel_ms_mean"], 5)},
            "prefill_shape": {"Sq": Sqp, "topk": topkp, "fp8_ms": round(tp["kernel_ms_mean"], 4),
                              "fp8_GBps": round(achp, 1), "bf16_ms": round(t2p["kernel_ms_mean"], 4)}}


def ceilings() -> dict:
    """Achievable MFMA and copy rates on this device (best of a few launches)."""
    import ctypes

    import torch

    from attention_forward_attn_amd import build as B

    if not os.path.exists(B.CEILING_LIB):
        raise RuntimeError(f"{B.CEILING_LIB} is missing: build with `python -m attention_forward_attn_amd.build`")
    lib = ctypes.CDLL(B.CEILING_LIB)
    lib.attn_ceiling_device_info.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
    lib.attn_ceiling_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.attn_ceiling_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    lib.attn_ceiling_spin.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    cus, clk = ctypes.c_int(0), ctypes.c_int(0)
    if lib.attn_ceiling_device_info(ctypes.byref(cus), ctypes.byref(clk)) != 0:
        raise RuntimeError("hipDeviceGetAttribute failed")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def best_ms(launch, reps=5):
        launch()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch()
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        return min(ts)

    blocks, iters = cus.value, 20000
    out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")

    def mfma():
        if lib.attn_ceiling_mfma(ctypes.c_void_p(out.data_ptr()), blocks, iters, sp) != 0:
            raise RuntimeError("MFMA loop launch failed")

    mfma_flops = blocks * 8 * iters * 8 * (2 * 32 * 32 * 16)
    mfma_tflops = mfma_flops / (best_ms(mfma) * 1e-3) / 1e12
    del out
    nbytes = 1 << 30  # 1 GiB read + 1 GiB written
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)

    def copy():
        if lib.attn_ceiling_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                 nbytes, cus.value * 64, sp) != 0:
            raise RuntimeError("copy launch failed")

    copy_gbs = 2 * nbytes / (best_ms(copy) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    # timer self-test: a kernel of known duration (it spins on the device's
    # 100 MHz real-time counter) must time within 5% with the same events
    spin_us = 2000
    ticks = torch.zeros(1, dtype=torch.int64, device="cuda")

    def spin():
        if lib.attn_ceiling_spin(spin_us, ctypes.c_void_p(ticks.data_ptr()), sp) != 0:
            raise RuntimeError("spin launch failed")

    ev_ms = best_ms(spin, reps=3)
    dev_ms = int(ticks.item()) / 1e5
    timer = {"expected_ms": spin_us / 1e3, "device_ms": round(dev_ms, 4), "event_ms": round(ev_ms, 4),
             "ok": abs(ev_ms / (spin_us / 1e3) - 1.0) <= 0.05}
    res = {"mfma_bf16_tflops": round(mfma_tflops, 1), "copy_gbs": round(copy_gbs, 1), "cus": cus.value,
           "max_clock_mhz": round(clk.value / 1e3), "computed_bf16_peak_tflops":
           round(cus.value * 4 * 1024 * clk.value * 1e3 / 1e12, 1), "timer_selftest": timer}
    log(f"[bench] ceilings: {res}")
    return res


def add_ceiling_fraction(roof: dict, ceil: dict) -> None:
    c = ceil["mfma_bf16_tflops"] if roof["bound"] == "mfma" else ceil["copy_gbs"]
    roof["ceiling"] = c
    roof["frac_of_ceiling"] = round(roof["achieved"] / c, 4) if c > 0 else None


def copy_calibration(mib: int, reps: int = 5):
    """A plain device copy of known size, to scale the HBM byte counters."""
    import torch

    src = torch.ones(mib << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copied {mib} MiB x {reps}")


def _counter_means(csv_path: str, counter: str) -> dict:
    """Mean value of one counter per dispatch, keyed by kernel name."""
    import collections
    import csv

    tot, disp = collections.defaultdict(float), collections.defaultdict(set)
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            tot[r["Kernel_Name"]] += float(r["Counter_Value"])
            disp[r["Kernel_Name"]].add(r["Dispatch_Id"])
    return {k: tot[k] / len(disp[k]) for k in tot}


def _workload_of_kernel(name: str):
    """Map a kernel's template arguments to the workload it serves (None if not ours)."""
    if "attn_fwd" not in name or "<" not in name:
        return None
    args = [a.strip() for a in name[name.index("<") + 1:name.index(">")].split(",")]
    dqk, dv = int(args[0]), int(args[1])
    if "attn_fwd_dma_kernel" in name:
        sparse = args[6] == "true"
        if sparse:
            return 5
        return {(128, 128): 2, (192, 128): 3, (512, 512): 4}.get((dqk, dv))
    return 1 if (dqk, dv) == (64, 64) else None


def traffic_from(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_mib, commands):
    """Write profiles/traffic.json: HBM bytes per launch for each workload kernel."""
    cf = _counter_means(copy_fetch_csv, "FETCH_SIZE")
    cw = _counter_means(copy_write_csv, "WRITE_SIZE")
    # the plain copy (the calibration run also has the fill that creates its source)
    ck = [k for k in cf if "copy" in k.lower()]
    if not ck:
        raise SystemExit("no copy kernel in the calibration profile")
    copy_kib = copy_mib * 1024.0
    sf = copy_kib / max(cf[ck[0]], 1.0)
    sw = copy_kib / max(cw[ck[0]], 1.0)
    fetch, write = _counter_means(fetch_csv, "FETCH_SIZE"), _counter_means(write_csv, "WRITE_SIZE")
    out = {"kernel_source_hash": kernel_source_hash(), "copy_calibration_mib": copy_mib,
           "fetch_scale": round(sf, 4), "write_scale": round(sw, 4), "commands": commands, "workloads": {}}
    for k in fetch:
        n = _workload_of_kernel(k)
        if n is None or k not in write:
            continue
        b = (fetch[k] * sf + write[k] * sw) * 1024.0
        out["workloads"][str(n)] = {"kernel": k, "fetch_kib_raw": round(fetch[k], 1),
                                    "write_kib_raw": round(write[k], 1), "hbm_bytes_per_launch": int(b),
                                    "algorithmic_bytes": work(n)["bytes"]}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gqa", choices=sorted(WORKLOAD_IDS))
    ap.add_argument("--primary-only", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured MFMA / copy ceilings")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip the rows beyond the five workloads (split-KV decode, backward, quantized cache, window)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="turn rocprofv3 FETCH_SIZE / WRITE_SIZE counter CSVs into profiles/traffic.json")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--commands", default="", help="the profiling commands, recorded in traffic.json")
    ap.add_argument("--traffic-of", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="HBM bytes per launch of every kernel in a FETCH_SIZE / WRITE_SIZE counter run, scaled "
                         "by the copy calibration recorded in profiles/traffic.json")
    ap.add_argument("--sparse-diagnostic", choices=("scrub", "pool1g"),
                    help="only the sparse forward with the Infinity Cache cleared before each launch, or over a "
                         "1 GiB pool (one JSON line; for counter runs)")
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from(*args.traffic_from, args.copy_mib, args.commands)
        return
    if args.traffic_of:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            cal = json.load(f)
        fetch, write = _counter_means(args.traffic_of[0], "FETCH_SIZE"), _counter_means(args.traffic_of[1], "WRITE_SIZE")
        for k in fetch:
            b = (fetch[k] * cal["fetch_scale"] + write.get(k, 0.0) * cal["write_scale"]) * 1024.0
            print(json.dumps({"kernel": k, "fetch_kib_raw": round(fetch[k], 1), "write_kib_raw": round(write.get(k, 0.0), 1),
                              "hbm_bytes_per_launch": int(b)}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the attention forward "
              "of this library runs on one device. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    import attention_forward_attn_amd as A

    A.load_library()
    if args.sparse_diagnostic:
        print(json.dumps(measure_sparse_diagnostic(args.sparse_diagnostic, args.steps, args.warmup)), flush=True)
        return
    n = WORKLOAD_IDS[args.workload]
    prim = measure(n, args.steps, args.warmup, split=(n == 6))
    others = []
    if not args.primary_only:
        for m in (1, 2, 3, 4, 5):
            if m == n:
                continue
            r = measure(m, max(10, args.steps // 2), max(3, args.warmup // 2))
            ent = {"workload": describe(m), "path": r["path"], "value": round(r["value"], 3),
                   "unit": r["unit"], "kernel_ms": round(r["timing"]["kernel_ms_mean"], 5),
                   "roofline": r["roofline"], "verdict": r["verdict"], "inputs_sha256": inputs_sha256(r["inp"])}
            if m == 1:
                ent["verdict"] = "Measured (launch-latency bound: 8.4 MFLOP per launch)"
            if not args.no_cpu_baseline:
                ent["cpu_baseline"] = cpu_baseline(m, r["inp"], budget_s=6.0)
                log(f"[bench] cpu oracle ({describe(m)}): {ent['cpu_baseline']}")
            others.append(ent)
            del r
            torch.cuda.empty_cache()
    # rows beyond the five: the split-KV forward on a decode step (Tq = 1),
    # with the plain one-launch path on the same inputs for context
    next_rows = []
    if not args.primary_only and not args.no_next_rows and n != 6:
        st, wu = max(10, args.steps // 2), max(3, args.warmup // 2)
        r = measure(6, st, wu, split=True)
        rp = measure(6, st, wu, split=False)
        next_rows.append({"row": "split-KV forward (attn_fwd_dense_splitkv), decode", "workload": describe(6),
                          "path": r["path"] + " + splitkv_merge", "value": round(r["value"], 3), "unit": r["unit"],
                          "kernel_ms": round(r["timing"]["kernel_ms_mean"], 5), "roofline": r["roofline"],
                          "verdict": r["verdict"],
                          "plain_path": {"path": rp["path"], "value": round(rp["value"], 3), "unit": rp["unit"],
                                         "kernel_ms": round(rp["timing"]["kernel_ms_mean"], 5)}})
        del r, rp
        torch.cuda.empty_cache()
        # the dense backward on the prefill workloads it is compiled for
        for m in (2, 3, 4, 7):
            next_rows.append(measure_bwd(m, st, wu))
            torch.cuda.empty_cache()
        # where the sparse forward's bytes come from: cache cleared, 1 GiB pool
        for kind in ("scrub", "pool1g"):
            next_rows.append(measure_sparse_diagnostic(kind, 10, 2))
            torch.cuda.empty_cache()
        # the sparse backward
        next_rows.append(measure_sparse_bwd(max(3, st // 4), 1))
        torch.cuda.empty_cache()
        # the sparse decode over an fp8 pool
        next_rows.append(measure_sparse_fp8(max(5, st // 2), 2))
        torch.cuda.empty_cache()
        # decode over quantized caches
        for fmt in ("q8_0", "q4_0"):
            next_rows.append(measure_qkv(fmt, st, wu))
            torch.cuda.empty_cache()
        # packed variable-length batches
        next_rows.append(measure_varlen(st, wu))
        torch.cuda.empty_cache()
        # MLA rows in two parts
        next_rows.append(measure_two_part(st, wu))
        torch.cuda.empty_cache()
        # the forward's extra returns
        next_rows.append(measure_extras(max(3, st // 4), 1))
        torch.cuda.empty_cache()
        # attention dropout
        next_rows.append(measure_dropout(st, wu))
        torch.cuda.empty_cache()
        # the sliding-window forward
        r = measure(7, st, wu)
        next_rows.append({"row": "sliding-window forward (window_left = 1024)", "workload": describe(7),
                          "path": r["path"], "value": round(r["value"], 3), "unit": r["unit"],
                          "kernel_ms": round(r["timing"]["kernel_ms_mean"], 5), "roofline": r["roofline"],
                          "verdict": r["verdict"]})
        del r
        torch.cuda.empty_cache()
    ceil = None
    if not args.no_ceilings:
        ceil = ceilings()
        add_ceiling_fraction(prim["roofline"], ceil)
        for o in others + next_rows:
            add_ceiling_fraction(o["roofline"], ceil)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(n, prim["inp"])
        log(f"[bench] cpu oracle: {cpu}")
    import synth

    s = synth.spec(n)
    line = {
        "metric": METRIC,
        "value": round(prim["value"], 3),
        "unit": prim["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(prim["timing"]["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if s.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) inputs of the workload's shapes; no dataset)",
        "config": {"workload": describe(n), "path": prim["path"], "kernel_ms": round(prim["timing"]["kernel_ms_mean"], 5),
                   "verdict": prim["verdict"], "inputs_sha256": inputs_sha256(prim["inp"])},
        "roofline": prim["roofline"],
        "cpu_baseline": cpu,
        "ceilings": ceil,
        "workloads": others,
        "next_rows": next_rows,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
