"""Benchmark: valid-token TFLOPS of sigmoid attention (forward + backward) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--precision fast|split|auto]
                    [--quick] [--no-cpu-baseline] [--cpu-seconds S] [--causal]
                    [--bias seqlen|per_head] [--dtype bf16|fp16] [--layout bhld|blhd]
                    [--attn sigmoid|softmax] [--compare-softmax] [--layer] [--settle-ms MS] [--split-bwd]

A step is one pass of the whole path over one batch already resident in HBM:
sigattn_fwd, then sigattn_bwd (the dQ and dK/dV work in one fused launch;
with --split-bwd, sigattn_bwd_dq then sigattn_bwd_dkdv, one launch each).
Untimed steps for --settle-ms of wall time (default 500 ms: from cold the
clocks need about a hundred steps to settle), then W untimed warm-up steps,
then exactly K timed steps bracketed by device syncs; HIP events recorded on
the launch stream around every call (created before the timed region) give
the per-kernel durations and cost about 3 % of the step.  FLOPs are algorithmic and count valid (query, key) pairs only:
forward 4 n^2 d and backward 10 n^2 d per (sequence, head) — the FlashAttention
convention; recomputation inside the backward kernels is not counted.

Prints ONE JSON line.  Besides the headline workload it carries, from the
same run: "padding_sweep" (the three padding-sweep workloads at 0 / 25 / 50 %
padding, forward-only and forward+backward TFLOPS, each time ratio against the
covered-tile and valid-pair ratios, and the TFLOPS drop from 0 % to 25 %),
"workloads" (the dense 8K batch at head dim 128 and the 8K log-normal
batch with x4 inputs in split precision, each with its roofline fraction and
its dominant kernel's time) and "short_sequences" (equal work as 4 sequences
of 4096, 1024 of 256 or 4096 of 128, with launches per pass and the slowdown
of the short cells).  --quick leaves them out.

Only one GPU is used: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
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

METRIC = "valid-token TFLOPS fwd/bwd, sigmoid attn d=64 L≤8K padded; % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published (no sparsity)
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCE = os.path.join(ROOT, "sigmoid_attention_amd", "csrc", "kernels.hip")
# Algorithmic FLOP per valid (query, key) pair and head dim, per kernel:
# forward: S = QK^T and PV (4); dK/dV kernel: S, dP, dV, dK (8); dQ kernel: dQ (2)
# (its S and dP recompute what the dK/dV kernel already counts).  Sum: 14 = 4 + 10.
KERNEL_FLOP_UNITS = {"fwd": 4, "bwd": 10, "bwd_dq": 2, "bwd_dkdv": 8}
# "bwd" is the fused backward launch (the dK/dV and dQ work of sigattn_bwd).
# MFMA work the kernels actually issue, same units, (fast, split precision):
# the backward recomputes S and dP on the dQ side, and split precision doubles
# the products that take P or dX.
EXECUTED_UNITS = {"fwd": (4, 6), "bwd": (14, 20), "bwd_dq": (6, 8), "bwd_dkdv": (8, 12)}
# ... except where sigattn_bwd runs the short-sequence backward (every
# sequence within 256 rows, head dim 64, fast precision, no mask): S and dP
# once, so it issues exactly the algorithmic 10.
ONE_TILE_EXECUTED = 10
# Algorithmic HBM bytes per launch: each input's valid rows read once, each
# output written whole (padded rows as zeros), as (inputs, outputs) counts.
KERNEL_TENSORS = {"fwd": (3, 1), "bwd": (4, 3), "bwd_dq": (4, 1), "bwd_dkdv": (4, 2)}
# The softmax comparison path adds a memory pass (delta = rowsum(dO * O)) that
# counts no FLOPs; its other kernels follow the same convention.


def pair_flops(seqlens, H, d, causal=False):
    """H d times the number of valid (query, key) pairs: n^2 per sequence,
    n (n + 1) / 2 under the causal mask."""
    n = np.asarray(seqlens, dtype=np.float64)
    pairs = n * (n + 1) / 2 if causal else n * n
    return float(H * d * pairs.sum())


def one_tile_bwd(w, precision, causal=False) -> bool:
    """Whether sigattn_bwd runs the short-sequence backward (one workgroup per
    (sequence, head)) for this workload."""
    return w.d == 64 and precision == "fast" and not causal and w.Lmax <= 256


def executed_units(kname, w, precision, causal=False):
    if kname == "bwd" and one_tile_bwd(w, precision, causal):
        return ONE_TILE_EXECUTED
    return EXECUTED_UNITS[kname][precision == "split"]


def kernel_bytes(kname, seqlens, w) -> float:
    """Algorithmic HBM bytes of one launch (16-bit elements)."""
    ins, outs = KERNEL_TENSORS[kname]
    valid = float(np.sum(np.asarray(seqlens, dtype=np.float64))) * w.H * w.d * 2
    return ins * valid + outs * float(w.B) * w.H * w.Lmax * w.d * 2


def roofline_bound(flops, nbytes, ms):
    """The roofline that bounds a launch of `flops` and `nbytes` (the lower of
    the MFMA and HBM times) and the fraction of each peak achieved."""
    tf = flops / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    hbm = flops / nbytes < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    return {"bound": "hbm" if hbm else "mfma",
            "achieved": round(gbs if hbm else tf, 2), "peak": PEAK_HBM_GBS if hbm else PEAK_BF16_TFLOPS,
            "unit": "GB/s" if hbm else "TFLOP/s",
            "frac": round(gbs / PEAK_HBM_GBS if hbm else tf / PEAK_BF16_TFLOPS, 4),
            "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "bytes_per_launch": nbytes, "flop_per_launch": flops}


def kernel_source_hash() -> str:
    """Hash of the code that decides what the kernels move: the kernel file,
    its device header and the planner, with // comments and whitespace
    removed (so a comment edit does not void measured counters)."""
    h = hashlib.sha256()
    for path in (KERNEL_SOURCE, *(os.path.join(ROOT, "sigmoid_attention_amd", "csrc", x)
                                  for x in ("device_common.h", "plan.h", "plan.cpp"))):
        with open(path, encoding="utf-8") as f:
            code = re.sub(r"//[^\n]*", "", f.read())
        h.update("".join(code.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str, precision: str):
    """HBM bytes per launch measured with rocprofv3 counters for this exact
    kernel source, or None if absent or stale."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    entry = rec.get("kernels", {}).get(f"{kernel}/{workload}/{precision}")
    return None if entry is None else entry.get("bytes_per_launch")


SETTLE_MS = 500.0  # default GPU time of untimed steps before the warm-up steps


def settle(step, ms):
    """Run untimed steps for about `ms` milliseconds of wall time (synchronised
    every few steps), so that clocks and caches reach the steady state of a
    long training run before warm-up and timing: from cold, the first hundred
    or so steps of the headline batch run up to 25 % slower.  Returns the
    number of steps run."""
    import torch

    done, t0 = 0, time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            step()
        done += 8
        torch.cuda.synchronize()
    return done


def time_workload(name, precision, steps, warmup, seed=0, layout="bhld", attn="sigmoid", causal=False,
                  bias="seqlen", dtype="bf16", settle_ms=SETTLE_MS, split_bwd=False):
    """Time `steps` passes of forward + backward (HIP events around every
    call, on the launch stream).  attn="softmax" times the softmax comparison
    path on the same inputs and schedule: forward, the delta pass, dQ, dK/dV.
    bias="per_head": a learnable per-head bias (values -ln of the mean
    length), its gradient rows from the dK/dV call and the per-head sum."""
    import torch

    import sigmoid_attention_amd as sa
    import workloads

    case = workloads.make(name, seed=seed, dtype=torch.float16 if dtype == "fp16" else torch.bfloat16)
    w = case["workload"]
    n = case["seqlens"]
    dev = torch.device("cuda:0")
    if layout == "blhd":  # [B, Lmax, H, d] activations, as a model holds them
        q, k, v, do = (case[t].permute(0, 2, 1, 3).contiguous().to(dev) for t in ("q", "k", "v", "do"))
    else:
        q, k, v, do = (case[t].to(dev) for t in ("q", "k", "v", "do"))
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    kw = dict(precision=precision, layout=layout)
    lse2 = delta = None
    if causal:
        kw["causal"] = True
    rows = db = None
    if bias == "per_head":
        (_, H_, _, _), _ = sa._binding.layout_strides(q, layout)
        kw["bias_mode"] = "per_head"
        kw["bias_arg"] = torch.full((H_,), -math.log(max(1.0, float(np.mean(n)))), dtype=torch.float32, device=dev)
        rows = sa._binding._rows_like(q, layout)
        db = torch.empty(H_, dtype=torch.float32, device=dev)
    if attn == "softmax":
        (B, H, L, _), _ = sa._binding.layout_strides(q, layout)
        lse2 = torch.empty((B, H, L), dtype=torch.float32, device=dev)
        delta = torch.empty_like(lse2)
    bwd_names = ("bwd_dq", "bwd_dkdv") if split_bwd else ("bwd",)
    names = ("fwd",) + (("bwd_prep",) if attn == "softmax" else ()) + bwd_names
    if rows is not None:
        names += ("bwd_bias_grad",)

    def step(ev=None):
        m = iter(range(len(names) + 1))

        def mark():
            i = next(m)
            if ev is not None:
                ev[i].record()
        mark()
        if attn == "sigmoid":
            sa.fwd(q, k, v, n, o=o, **kw)
            mark()
            if not split_bwd:
                sa.bwd(q, k, v, do, n, dq=dq, dk=dk, dv=dv, dbias=rows, **kw)
                mark()
            else:
                sa.bwd_dq(q, k, v, do, n, dq=dq, **kw)
                mark()
                if rows is None:
                    sa.bwd_dkdv(q, k, v, do, n, dk=dk, dv=dv, **kw)
                else:
                    sa.bwd_dkdv_dbias(q, k, v, do, n, dk=dk, dv=dv, dbias=rows, **kw)
                mark()
            if rows is not None:
                sa.bias_grad(rows, n, db=db)
                mark()
        else:
            sa.softmax_fwd(q, k, v, n, o=o, lse2=lse2, **kw)
            mark()
            sa.softmax_bwd_prep(o, do, n, delta, precision=precision, layout=layout)
            mark()
            if not split_bwd:
                sa._binding.softmax_bwd_fused(q, k, v, do, lse2, delta, n, dq, dk, dv, **kw)
                mark()
            else:
                sa.softmax_bwd_dq(q, k, v, do, lse2, delta, n, dq, **kw)
                mark()
                sa.softmax_bwd_dkdv(q, k, v, do, lse2, delta, n, dk, dv, **kw)
                mark()

    settled = settle(step, settle_ms)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
    for ev in events:  # create the HIP events now: torch creates them at their first record
        for e in ev:
            e.record()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    host_s = time.perf_counter() - t0
    per = {kname: [ev[i].elapsed_time(ev[i + 1]) for ev in events] for i, kname in enumerate(names)}
    step_ms = events[0][0].elapsed_time(events[-1][-1]) / steps
    base = pair_flops(n, w.H, w.d, causal)
    avg = {kname: float(np.mean(v_)) for kname, v_ in per.items()}
    med = {kname: float(np.median(v_)) for kname, v_ in per.items()}
    res = {
        "workload": w, "seqlens": n, "step_ms": step_ms, "host_step_ms": host_s * 1e3 / steps,
        "kernel_avg_ms": avg, "kernel_median_ms": med, "kernel_min_ms": {k_: float(np.min(v_)) for k_, v_ in per.items()},
        "pair_flops": base, "settle_steps": settled,
        "fwd_flops": 4 * base, "bwd_flops": 10 * base,
        "outputs": tuple(t.permute(0, 2, 1, 3) if layout == "blhd" else t for t in (o, dq, dk, dv)),
        "case": case,
    }
    return res


def time_layer(attn, steps, warmup, d_model=768, heads=12, mlp=3072, seed=0, settle_ms=SETTLE_MS):
    """Forward + backward of one pre-norm bidirectional transformer layer of
    the 160M-parameter class (d_model 768, 12 heads of 64, MLP 3072, bf16,
    random weights) on the headline batch's lengths: LayerNorm, fused QKV
    projection, attention on [B, Lmax, H, d] views of it, output projection,
    residual, LayerNorm, GELU MLP, residual.  attn: "sigmoid", "softmax" (both
    this library's kernels) or "none" (attention replaced by V, to isolate the
    rest of the layer).  Returns the mean ms per step (HIP events)."""
    import torch
    import torch.nn.functional as F

    import sigmoid_attention_amd as sa
    import workloads

    w = workloads.WORKLOADS[workloads.HEADLINE]
    n = workloads.lengths(workloads.HEADLINE)
    B, L, dh = w.B, w.Lmax, d_model // heads
    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(seed)

    def param(*shape, fan_in):
        return (torch.randn(*shape, generator=g) / math.sqrt(fan_in)).to(dev, torch.bfloat16).requires_grad_(True)

    wqkv, wo = param(3 * d_model, d_model, fan_in=d_model), param(d_model, d_model, fan_in=d_model)
    w1, w2 = param(mlp, d_model, fan_in=d_model), param(d_model, mlp, fan_in=mlp)
    ln1 = torch.nn.LayerNorm(d_model).to(dev, torch.bfloat16)
    ln2 = torch.nn.LayerNorm(d_model).to(dev, torch.bfloat16)
    x = torch.randn(B, L, d_model, generator=g).to(dev, torch.bfloat16).requires_grad_(True)
    gy = torch.randn(B, L, d_model, generator=g).to(dev, torch.bfloat16)

    def layer(x):
        qkv = F.linear(ln1(x), wqkv).view(B, L, 3, heads, dh)
        q, k, v = qkv.unbind(2)
        if attn == "sigmoid":
            a = sa.sigmoid_attention(q, k, v, n, layout="blhd")
        elif attn == "softmax":
            a = sa.softmax_attention(q, k, v, n, layout="blhd")
        else:
            a = v.contiguous()
        x = x + F.linear(a.reshape(B, L, d_model), wo)
        return x + F.linear(F.gelu(F.linear(ln2(x), w1)), w2)

    def step():
        layer(x).backward(gy)

    settle(step, settle_ms)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def tflops(flops, ms):
    return flops / (ms * 1e-3) / 1e12


def host_cpu():
    """The host's CPU model (from /proc/cpuinfo), the logical CPUs this
    process may run on, and the threads the BLAS pool uses."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover - not Linux
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        blas = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover - threadpoolctl missing
        blas = 1
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "usable_cpus": usable, "blas_threads": int(blas)}


def cpu_baseline(case, outputs, budget_s):
    """Time the CPU oracle (as it stands) on a bounded sample of the same
    workload: whole heads, cycling through the sequences longest first, until
    about budget_s seconds of work.  Returns the record and the worst parity
    ratio of the GPU outputs on those heads."""
    import oracle
    from workloads import as_f64

    hw = host_cpu()
    cores = hw["blas_threads"]
    w = case["workload"]
    n = case["seqlens"]
    order = [int(b) for b in np.argsort(-np.asarray(n), kind="stable") if n[b] > 0]
    done, flops, secs, worst = [], 0.0, 0.0, 0.0
    i = 0
    while secs < budget_s and order and i < len(order) * w.H:
        b = order[i % len(order)]
        h = (i // len(order)) % w.H
        i += 1
        args = [as_f64(case[t][b, h]) for t in ("q", "k", "v", "do")]
        t0 = time.perf_counter()
        ref = oracle.head(*args, int(n[b]))
        secs += time.perf_counter() - t0
        flops += 14.0 * w.d * float(n[b]) ** 2
        done.append((b, h, int(n[b])))
        for got, r in zip(outputs, ref):
            g = as_f64(got[b, h])
            worst = max(worst, float(np.max(np.abs(g - r) / (2e-2 * (1.0 + np.abs(r))))))
    rec = {
        "value": flops / secs / 1e12 if secs > 0 else None,
        "unit": "TFLOPS",
        "cores": int(cores),
        **hw,
        "kind": "oracle",
        "sample": f"fp64 oracle forward+backward on {len(done)} of {w.B * w.H} heads of {w.name} "
                  f"(longest sequences first; lengths {sorted({x[2] for x in done}, reverse=True)}), "
                  f"{secs:.1f} s, same algorithmic FLOP convention",
        "seconds": secs,
    }
    return rec, worst


def covered_pairs(seqlens, H, outer, inner):
    n = np.asarray(seqlens, dtype=np.int64)
    return int((H * -(-n // outer) * -(-n // inner)).sum())


SWEEP = ("sweep_b16h16d64_l4096_pad00", "sweep_b16h16d64_l4096_pad25", "sweep_b16h16d64_l4096_pad50")
# Workloads timed beside the headline in the default run: head dim 128 at 8K
# (dense), and the 8K log-normal batch whose x4 inputs saturate sigma (split
# precision).
EXTRA = (("dense_b4h16d128_l8192", "fast"), ("cells8k_b8h12d64_l8192_x4", "split"))
# Equal work per head cut into few long or many short sequences: the schedule
# keeps every pass one launch, and the TFLOPS ratio shows what short items cost.
SHORT = ("few_b4h16d64_l4096", "many_b1024h16d64_l256", "many_b4096h16d64_l128")


def measure_copy_gbs(reps=10) -> float:
    """HBM rate of a plain device copy of 1 GiB (bytes read + written per
    second), timed with HIP events: the rate a streaming kernel reaches on
    this chip, beside the published 8 TB/s."""
    import torch

    x = torch.empty(1 << 29, dtype=torch.int16, device="cuda:0").fill_(1)
    y = torch.empty_like(x)
    y.copy_(x)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    gbs = reps * 2 * x.numel() * 2 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del x, y
    torch.cuda.empty_cache()
    return gbs


def workload_record(r, precision, copy_gbs=None):
    """Throughput of one timed workload (forward + fused backward) with the
    roofline fraction of its dominant kernel."""
    n = r["seqlens"]
    w = r["workload"]
    fwd_ms = r["kernel_avg_ms"]["fwd"]
    bwd_ms = sum(v_ for k_, v_ in r["kernel_avg_ms"].items() if k_.startswith("bwd"))
    timed = [k_ for k_ in KERNEL_FLOP_UNITS if k_ in r["kernel_avg_ms"]]
    dom = max(timed, key=r["kernel_avg_ms"].get)
    roof = roofline_bound(KERNEL_FLOP_UNITS[dom] * r["pair_flops"], kernel_bytes(dom, n, w), r["kernel_avg_ms"][dom])
    roof.update({"kernel": dom, "avg_launch_ms": round(r["kernel_avg_ms"][dom], 5),
                 "executed_mfma_frac": round(tflops(executed_units(dom, w, precision) * r["pair_flops"],
                                                    r["kernel_avg_ms"][dom]) / PEAK_BF16_TFLOPS, 4),
                 "traffic": load_traffic(dom, w.name, precision)})
    if copy_gbs and roof["bound"] == "hbm":
        roof["frac_of_measured_copy"] = round(roof["achieved"] / copy_gbs, 4)
    return {
        "B": w.B, "H": w.H, "d": w.d, "Lmax": w.Lmax, "seqlens": [int(x) for x in n], "precision": precision,
        "value": round(tflops(r["fwd_flops"] + r["bwd_flops"], r["step_ms"]), 2),
        "ms_per_step": round(r["step_ms"], 5),
        "fwd_tflops": round(tflops(r["fwd_flops"], fwd_ms), 2),
        "bwd_tflops": round(tflops(r["bwd_flops"], bwd_ms), 2),
        "kernel_avg_ms": {k_: round(v_, 5) for k_, v_ in r["kernel_avg_ms"].items()},
        "roofline": roof,
    }


def padding_sweep(steps, settle_ms, attn="sigmoid", compare_softmax=False):
    """The padding sweep (B16 H16 d64 Lmax 4096 at 0 / 25 / 50 % padding):
    forward-only and forward+backward valid-token TFLOPS, the time ratios
    against 0 % padding beside the covered-tile and valid-pair ratios (the
    work the schedule skips), and the TFLOPS drop from 0 % to 25 %."""
    import torch

    sweep = {}
    base = None
    for sw in SWEEP:
        rs = time_workload(sw, "fast", steps, 2, attn=attn, settle_ms=settle_ms)
        ws = rs["workload"]
        fwd_ms = rs["kernel_avg_ms"]["fwd"]
        step_ms = rs["step_ms"]
        if base is None:
            base = (fwd_ms, step_ms)
        dense_pairs = covered_pairs([ws.Lmax] * ws.B, ws.H, 128, 64)
        cmp_ = {}
        if compare_softmax:
            rc = time_workload(sw, "fast", steps, 2, attn="softmax", settle_ms=settle_ms)
            cmp_ = {"softmax_fwd_tflops": round(tflops(rc["fwd_flops"], rc["kernel_avg_ms"]["fwd"]), 2),
                    "softmax_fwd_bwd_tflops": round(tflops(rc["fwd_flops"] + rc["bwd_flops"], rc["step_ms"]), 2),
                    "sigmoid_fwd_speedup": round(rc["kernel_avg_ms"]["fwd"] / fwd_ms, 4),
                    "sigmoid_step_speedup": round(rc["step_ms"] / step_ms, 4)}
            del rc
        sweep[sw] = {**cmp_,
            "seqlens": [int(x) for x in rs["seqlens"]],
            "padding": round(1 - float(np.sum(rs["seqlens"])) / (ws.B * ws.Lmax), 4),
            "fwd_tflops": round(tflops(rs["fwd_flops"], fwd_ms), 2),
            "fwd_bwd_tflops": round(tflops(rs["fwd_flops"] + rs["bwd_flops"], step_ms), 2),
            "fwd_ms": round(fwd_ms, 5), "step_ms": round(step_ms, 5),
            "fwd_time_ratio": round(fwd_ms / base[0], 4),
            "step_time_ratio": round(step_ms / base[1], 4),
            "covered_tile_ratio": round(covered_pairs(rs["seqlens"], ws.H, 128, 64) / dense_pairs, 4),
            "valid_pair_ratio": round(float(np.sum(np.asarray(rs["seqlens"], np.float64) ** 2))
                                      / (ws.B * ws.Lmax ** 2), 4),
        }
        del rs
        torch.cuda.empty_cache()
    p0, p25 = sweep[SWEEP[0]], sweep[SWEEP[1]]
    sweep["tflops_drop_0_to_25"] = {
        "fwd": round(1 - p25["fwd_tflops"] / p0["fwd_tflops"], 4),
        "fwd_bwd": round(1 - p25["fwd_bwd_tflops"] / p0["fwd_bwd_tflops"], 4),
        "tile_granularity_floor": round(1 - p25["valid_pair_ratio"] / p25["covered_tile_ratio"], 4),
    }
    return sweep


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--precision", default="auto", choices=["auto", "fast", "split"])
    ap.add_argument("--quick", action="store_true",
                    help="time the headline workload only (no padding sweep, no 8K workloads)")
    ap.add_argument("--attn", default="sigmoid", choices=["sigmoid", "softmax"],
                    help="time the softmax comparison path instead of sigmoid attention")
    ap.add_argument("--compare-softmax", action="store_true",
                    help="also time the softmax path on the same workload (and sweep) and report ratios")
    ap.add_argument("--layer", action="store_true",
                    help="instead: time one 160M-class transformer layer (fwd+bwd) with sigmoid vs softmax "
                         "attention and print that as the JSON line")
    ap.add_argument("--layout", default="bhld", choices=["bhld", "blhd"],
                    help="tensor layout handed to the library: [B,H,Lmax,d] or [B,Lmax,H,d] (strided path)")
    ap.add_argument("--causal", action="store_true",
                    help="causal mask (query i sees keys 0..i); FLOPs count the n(n+1)/2 visible pairs")
    ap.add_argument("--bias", default="seqlen", choices=["seqlen", "per_head"],
                    help="per_head: a learnable per-head bias, with its gradient computed in the backward")
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "fp16"],
                    help="element type of the tensors (fp16: the fp16 build of the kernels)")
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="wall time of untimed steps run before the warm-up steps (clocks reach steady state)")
    ap.add_argument("--split-bwd", action="store_true",
                    help="time the backward as two launches (dQ, then dK/dV) instead of the fused sigattn_bwd")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the sustained-MFMA probe reported beside the roofline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 1 GiB, 5 times (HBM counter calibration)")
    a = ap.parse_args()

    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {a.gpus}). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import sigmoid_attention_amd as sa
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    sa.load()  # fail loudly if the library is not built

    if a.copy_calibration:
        x = torch.empty(1 << 29, dtype=torch.int16, device="cuda:0").fill_(1)
        y = torch.empty_like(x)
        for _ in range(5):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read_per_copy": x.numel() * 2,
                          "bytes_written_per_copy": y.numel() * 2, "copies": 5}))
        return

    if a.layer:
        ms = {k_: time_layer(k_, a.steps, a.warmup, settle_ms=a.settle_ms) for k_ in ("sigmoid", "softmax", "none")}
        w = workloads.WORKLOADS[workloads.HEADLINE]
        n = workloads.lengths(workloads.HEADLINE)
        print(json.dumps({
            "metric": "ms per forward+backward of one transformer layer (d_model 768, 12 heads, MLP 3072)",
            "value": round(ms["sigmoid"], 4), "unit": "ms", "higher_is_better": False, "steps": a.steps,
            "warmup": a.warmup, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": workloads.HEADLINE, "B": w.B, "Lmax": w.Lmax, "seqlens": [int(x) for x in n],
                       "d_model": 768, "heads": 12, "head_dim": 64, "mlp": 3072, "layout": "blhd (fused QKV views)"},
            "sigmoid_ms": round(ms["sigmoid"], 4), "softmax_ms": round(ms["softmax"], 4),
            "no_attention_ms": round(ms["none"], 4),
            "sigmoid_layer_speedup": round(ms["softmax"] / ms["sigmoid"], 4),
            "attention_share_sigmoid": round(1 - ms["none"] / ms["sigmoid"], 4),
            "attention_share_softmax": round(1 - ms["none"] / ms["softmax"], 4),
        }))
        return

    name = a.workload or workloads.HEADLINE
    w = workloads.WORKLOADS[name]
    precision = a.precision if a.precision != "auto" else ("split" if w.scale_qkv > 1.0 else "fast")
    r = time_workload(name, precision, a.steps, a.warmup, layout=a.layout, attn=a.attn, causal=a.causal,
                      bias=a.bias, dtype=a.dtype, settle_ms=a.settle_ms, split_bwd=a.split_bwd)
    n = r["seqlens"]
    total = r["fwd_flops"] + r["bwd_flops"]
    value = tflops(total, r["step_ms"])
    fwd_tf = tflops(r["fwd_flops"], r["kernel_avg_ms"]["fwd"])
    bwd_tf = tflops(r["bwd_flops"], sum(v_ for k_, v_ in r["kernel_avg_ms"].items() if k_.startswith("bwd")))

    timed = [k_ for k_ in KERNEL_FLOP_UNITS if k_ in r["kernel_avg_ms"]]
    dominant = max(timed, key=r["kernel_avg_ms"].get)
    dom_flops = KERNEL_FLOP_UNITS[dominant] * r["pair_flops"]
    achieved = tflops(dom_flops, r["kernel_avg_ms"][dominant])
    roofline = roofline_bound(dom_flops, kernel_bytes(dominant, n, w), r["kernel_avg_ms"][dominant])
    roofline.update({
        "traffic": load_traffic(dominant, name, precision),
        "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
        "kernel": dominant,
        "executed_mfma_frac": round(tflops(executed_units(dominant, w, precision, a.causal) * r["pair_flops"],
                                           r["kernel_avg_ms"][dominant]) / PEAK_BF16_TFLOPS, 4),
        "avg_launch_ms": round(r["kernel_avg_ms"][dominant], 5),
        "per_kernel": {
            kname: {"avg_ms": round(r["kernel_avg_ms"][kname], 5), "median_ms": round(r["kernel_median_ms"][kname], 5),
                     "min_ms": round(r["kernel_min_ms"][kname], 5),
                     "algorithmic_tflops": round(tflops(KERNEL_FLOP_UNITS[kname] * r["pair_flops"],
                                                        r["kernel_avg_ms"][kname]), 2)}
            for kname in timed},
    })
    if not a.no_probe:  # the chip's sustained MFMA rate and clock, right after the timed region
        pr = sa.probe_mfma()
        roofline["measured_mfma_peak"] = {"tflops": round(pr["tflops"], 1),
                                          "shader_clock_ghz": round(pr["shader_clock_ghz"], 3),
                                          "kernel": "back-to-back bf16 32x32x16 MFMAs, 4 chains per wave, "
                                                    "4 waves per SIMD (sigattn_probe_mfma)"}
        roofline["frac_of_measured_peak"] = round(achieved / pr["tflops"], 4)
        copy_gbs = measure_copy_gbs()
        roofline["measured_hbm_copy"] = {"gbps": round(copy_gbs, 1),
                                         "kernel": "device copy of 1 GiB, bytes read + written"}
        if roofline["bound"] == "hbm":
            roofline["frac_of_measured_copy"] = round(roofline["achieved"] / copy_gbs, 4)
    else:
        copy_gbs = None
    if roofline["traffic"] is not None:  # achieved HBM rate of the dominant kernel
        roofline["hbm_gbps"] = round(roofline["traffic"] / (r["kernel_avg_ms"][dominant] * 1e-3) / 1e9, 1)
    if "bwd_bias_grad" in r["kernel_avg_ms"]:
        roofline["per_kernel"]["bwd_bias_grad"] = {"avg_ms": round(r["kernel_avg_ms"]["bwd_bias_grad"], 5),
                                               "median_ms": round(r["kernel_median_ms"]["bwd_bias_grad"], 5)}
    if "bwd_prep" in r["kernel_avg_ms"]:
        roofline["per_kernel"]["bwd_prep"] = {"avg_ms": round(r["kernel_avg_ms"]["bwd_prep"], 5),
                                              "median_ms": round(r["kernel_median_ms"]["bwd_prep"], 5)}
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(r["step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": a.dtype,
        "data": "synthetic",
        "config": {
            "workload": name, "B": w.B, "H": w.H, "d": w.d, "Lmax": w.Lmax, "seqlens": [int(x) for x in n],
            "precision": precision,
            "bias": ("none (softmax)" if a.attn != "sigmoid" else
                     "learnable per head, with gradient" if a.bias == "per_head" else "-ln(n_b)"),
            "layout": a.layout, "attention": a.attn, "mask": "causal" if a.causal else "none",
            "valid_token_frac": round(float(np.sum(n)) / (w.B * w.Lmax), 4),
            "valid_pair_frac": round(float(np.sum(np.asarray(n, np.float64) ** 2)) / (w.B * w.Lmax ** 2), 4),
        },
        "fwd_tflops": round(fwd_tf, 2),
        "bwd_tflops": round(bwd_tf, 2),
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_pct_bf16_peak": round(100 * fwd_tf / PEAK_BF16_TFLOPS, 2),
        "bwd_pct_bf16_peak": round(100 * bwd_tf / PEAK_BF16_TFLOPS, 2),
        "host_ms_per_step": round(r["host_step_ms"], 5),
        "settle": {"ms": a.settle_ms, "steps": r["settle_steps"]},
        "roofline": roofline,
    }

    if not a.quick:
        sub_steps, sub_settle = max(5, a.steps // 2), min(a.settle_ms, 200.0)
        out["padding_sweep"] = padding_sweep(sub_steps, sub_settle, attn=a.attn, compare_softmax=a.compare_softmax)
        if a.attn == "sigmoid" and not a.causal and a.bias == "seqlen" and a.layout == "bhld":
            out["workloads"] = {}
            for wn, prec in EXTRA:
                if wn == name:
                    continue
                rx = time_workload(wn, prec, sub_steps, 2, dtype=a.dtype, settle_ms=sub_settle)
                out["workloads"][wn] = workload_record(rx, prec, copy_gbs)
                del rx
                torch.cuda.empty_cache()
            short = {}
            for wn in SHORT:
                rx = time_workload(wn, "fast", sub_steps, 2, dtype=a.dtype, settle_ms=sub_settle)
                rec = workload_record(rx, "fast", copy_gbs)
                ws = rx["workload"]
                rec.pop("seqlens")
                rec["launches_per_pass"] = {p_: int(sa.plan_stats(ws.B, ws.H, ws.Lmax, ws.d, rx["seqlens"], p_)[2])
                                            for p_ in ("fwd", "bwd")}
                short[wn] = rec
                del rx
                torch.cuda.empty_cache()
            for wn in SHORT[1:]:
                short[wn]["slowdown_vs_" + SHORT[0]] = {
                    k_: round(short[SHORT[0]][k_] / short[wn][k_], 4) for k_ in ("value", "fwd_tflops", "bwd_tflops")}
            out["short_sequences"] = short

    if a.compare_softmax and a.attn == "sigmoid":
        rc = time_workload(name, precision, a.steps, a.warmup, layout=a.layout, attn="softmax", causal=a.causal,
                           settle_ms=a.settle_ms, split_bwd=a.split_bwd)
        out["softmax_comparison"] = {
            "value": round(tflops(total, rc["step_ms"]), 2),
            "fwd_tflops": round(tflops(rc["fwd_flops"], rc["kernel_avg_ms"]["fwd"]), 2),
            "bwd_tflops": round(tflops(rc["bwd_flops"], sum(v_ for k_, v_ in rc["kernel_avg_ms"].items()
                                                            if k_.startswith("bwd"))), 2),
            "kernel_avg_ms": {k_: round(v_, 5) for k_, v_ in rc["kernel_avg_ms"].items()},
            "sigmoid_fwd_speedup": round(rc["kernel_avg_ms"]["fwd"] / r["kernel_avg_ms"]["fwd"], 4),
            "sigmoid_step_speedup": round(rc["step_ms"] / r["step_ms"], 4),
        }
        del rc

    if not a.no_cpu_baseline and a.attn == "sigmoid" and not a.causal and a.bias == "seqlen":
        rec, worst = cpu_baseline(r["case"], r["outputs"], a.cpu_seconds)
        out["cpu_baseline"] = {k_: v_ for k_, v_ in rec.items() if k_ != "seconds"}
        out["parity_worst_ratio_on_cpu_sample"] = round(worst, 4)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
