#!/usr/bin/env python3
"""Benchmark of the batched Newton-Schulz / Muon step on one MI355X.

Headline (the metric's own configuration): one `ns_orthogonalize_batched`
call over 32 matrices 768x3072 (bf16, seeded N(0, 0.01^2), resident in HBM),
FAST precision, 5 quintic iterations.  `value` is nominal NS TFLOP/s:
32 * 5 * (4 m^2 n + 2 m^3) flops (m = 768, n = 3072) divided by the
wall-clock time of one call; matrices/s is 32 per call.

Beside it the JSON line carries
  * roofline: the dominant kernel of the call (the NS kernel family with the
    most time; with the automatic schedule the persistent loop k_ns_loop),
    timed with hipEvents the library records around each launch, at three
    flop counts: nominal (the metric's), executed (the 256-wide tiles the
    kernel computes: symmetric products skip lower tiles) and algorithmic
    (the method's symmetric work 5 (3 m^2 n + m^3)); plus the MFMA-busy
    fraction and the HBM traffic from committed rocprofv3 counter runs
    (profiles/, null once the kernel source changed);
  * percentiles of the call time (per-call events) with a warm and a cold
    (1 GiB written between calls) Infinity Cache;
  * extras: the full 124M custom-sizing Muon step (muon_step_multi over 43
    matrices) with its element-wise kernels' HBM rates, one GPU's share of it
    under 8-way sharding by whole matrices, full steps of the GPT-2-medium-like
    96 x 1024x4096 batch and of the large dense ACCURATE batch (nominal and
    executed MFMA rates), the AdamW step of the 124M model;
  * cpu_baseline: the fp64 NumPy oracle on a bounded sample of the same
    workload on the host cores.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Newton-Schulz TFLOP/s and matrices/s at 32x768x3072 bf16; % of MFMA peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
GEMM_SOURCE = os.path.join(ROOT, "newton_schulz_muon_amd", "csrc", "ns_gemm.hip")
EW_SOURCE = os.path.join(ROOT, "newton_schulz_muon_amd", "csrc", "muon_elementwise.hip")
ADAM_SOURCE = os.path.join(ROOT, "newton_schulz_muon_amd", "csrc", "adamw.hip")
NS_FAMILIES = ("ns_loop", "gram", "poly", "bx")
FAMILY_NAMES = {"ns_loop": "k_ns_loop (all NS iterations of a call in one launch: X X^T, aI + bA + cA^2, B' X)",
                "gram": "k_gemm<kGram> (A = X X^T)",
                "poly": "k_gemm<kPoly> (B' = aI + bA + cA^2)",
                "bx": "k_gemm<kBx> (X <- B' X)"}
SETTLE_CALLS = 12              # calls before warm-up that let the automatic NS schedule choose
NS_STEPS = 5
# the quintic's coefficients (the parameter-golf walkthrough, Part 1; the library's defaults)
NS_COEFFS = (3.4445, -4.7750, 2.0315)


def ns_flops(m: int, n: int, steps: int = NS_STEPS) -> float:
    """Nominal NS work of one block (the metric's count): steps (4 m^2 n + 2 m^3), m <= n."""
    m, n = min(m, n), max(m, n)
    return float(steps) * (4.0 * m * m * n + 2.0 * m ** 3)


def ns_flops_symmetric(m: int, n: int, steps: int = NS_STEPS) -> float:
    """The method's own work with A and B' symmetric: steps (3 m^2 n + m^3)."""
    m, n = min(m, n), max(m, n)
    return float(steps) * (3.0 * m * m * n + float(m) ** 3)


def loop_executed_flops(m: int, n: int, steps: int = NS_STEPS) -> float:
    """MFMA flops the persistent loop executes for one block: 256-wide tiles of
    the padded oriented block (mp x np), upper-triangle tiles of the symmetric
    products (T (T + 1) / 2 of them, the T diagonal ones computing 10 of
    their 16 64 x 64 blocks), every tile of B' X."""
    m, n = min(m, n), max(m, n)
    mp, np_ = -(-m // 128) * 128, -(-n // 128) * 128
    t, tn = mp // 256, np_ // 256
    nsym, nbx = t * (t + 1) // 2 - 0.375 * t, t * tn
    return float(steps) * 2.0 * 256 * 256 * (nsym * np_ + nsym * mp + nbx * mp)


def source_digest(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_profile(name: str, source: str, key: str):
    """A figure from a committed rocprofv3 summary (profiles/<name>.json), or
    None when it is missing or the kernel source changed since it was taken."""
    try:
        with open(os.path.join(PROFILES, name + ".json")) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256_16") != source_digest(source):
        return None
    return t.get(key)


def percentiles(xs):
    xs = sorted(xs)

    def q(p):
        k = (len(xs) - 1) * p
        lo, hi = int(k), min(int(k) + 1, len(xs) - 1)
        return xs[lo] + (xs[hi] - xs[lo]) * (k - lo)
    return {"p10": round(q(0.1), 4), "p50": round(q(0.5), 4), "p90": round(q(0.9), 4)}


# ----------------------------------------------------------------------------- host description
def host_info():
    import numpy as np
    info = {"os_cpu_count": os.cpu_count()}
    try:
        info["affinity_cpus"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        info["affinity_cpus"] = None
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    info["cpu_model"] = model or platform.processor() or None
    blas, threads = None, None
    try:
        from threadpoolctl import threadpool_info
        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if pools:
            blas = f"{pools[0].get('internal_api')} {pools[0].get('version')}"
            threads = max(int(p.get("num_threads", 1)) for p in pools)
    except Exception:
        pass
    if blas is None:
        try:
            cfg = np.show_config(mode="dicts")
            blas = cfg.get("Build Dependencies", {}).get("blas", {}).get("name")
        except Exception:
            blas = None
    info["blas"] = blas
    info["blas_threads"] = threads
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS"):
        info[var] = os.environ.get(var)
    return info


def cpu_baseline(seconds: float):
    """The fp64 oracle (as it stands) on 768x3072 blocks of the headline
    workload, one after another, until about `seconds` of work."""
    import numpy as np
    import oracle
    import workloads
    wl = workloads.get_workload("metric32")
    g = wl.groups[0]
    done, t0 = 0, time.perf_counter()
    while True:
        bits = workloads.grad_bits_host(wl, g, 0, [done % g.count])
        oracle.ns_batched(workloads.bf16_bits_to_f32(bits).astype(np.float64), steps=NS_STEPS)
        done += 1
        if time.perf_counter() - t0 > seconds:
            break
    dt = time.perf_counter() - t0
    info = host_info()
    cores = info["blas_threads"] or info["affinity_cpus"] or info["os_cpu_count"] or 1
    return {"value": round(done * ns_flops(768, 3072) / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"fp64 numpy oracle NS (5 iterations) of {done} of the 32 matrices 768x3072, one at a time, "
                      f"in {dt:.1f} s: {done / dt:.3f} matrices/s, nominal flops",
            "host": info}


# ----------------------------------------------------------------------------- GPU parts
class Timer:
    """Library-recorded hipEvent timing of selected kernel families."""

    def __init__(self, nsm, families):
        self.nsm, self.families = nsm, list(families)

    def __enter__(self):
        self.nsm.muon_timing_collect()
        self.nsm.muon_timing_enable(self.families)
        return self

    def __exit__(self, *exc):
        import torch
        torch.cuda.synchronize()
        self.nsm.muon_timing_enable([])
        self.result = self.nsm.muon_timing_collect(with_flops=True)
        return False


def timed_region(fn, steps):
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1000.0 / steps


def per_call_ms(fn, steps, flush=None):
    """Per-call event times on torch's current stream (the library launches
    there); with `flush`, a 1 GiB write runs between calls (outside the events)."""
    import torch
    out = []
    for _ in range(steps):
        if flush is not None:
            flush.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        e1.synchronize()
        out.append(e0.elapsed_time(e1))
    return out


def headline(nsm, args, dev):
    import torch
    import workloads
    wl = workloads.get_workload("metric32")
    g = wl.groups[0]
    x = workloads.grads_device(wl, g, 0, dev)
    out = torch.empty_like(x)
    call = lambda: nsm.ns_orthogonalize_batched(x, out, precision="fast")     # noqa: E731
    # The automatic NS schedule times its first ten calls per set of shapes
    # (alternating the per-product launches and the persistent loop) and keeps
    # the faster once those calls' events have completed: let it settle.
    for _ in range(SETTLE_CALLS):
        call()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ms = timed_region(call, args.steps)                       # uninstrumented: `value`
    m, n, nb = g.rows, g.cols, g.count
    nominal = nb * ns_flops(m, n)
    res = {"ms": ms, "nominal": nominal, "nb": nb}
    # per-call distribution, warm and with the Infinity Cache flushed between calls
    res["warm"] = percentiles(per_call_ms(call, args.steps))
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    res["cold"] = percentiles(per_call_ms(call, args.steps, flush))
    del flush
    # the call's kernels, each launch bracketed by events (a region of its own)
    with Timer(nsm, nsm.KERNEL_KINDS) as t:
        for _ in range(args.steps):
            call()
    res["families"] = t.result
    res["status"] = nsm.last_call_status(dev)
    del x, out
    return res


def roofline_of(res, steps):
    fam = res["families"]
    ns = {k: v for k, v in fam.items() if k in NS_FAMILIES}
    if not ns:
        return None
    k = max(ns, key=lambda f: ns[f][1])
    launches, tot_ms, nominal, executed = ns[k]
    avg_ms = tot_ms / launches
    nom = nominal / launches
    r = {"bound": "mfma", "kernel": FAMILY_NAMES[k], "flops_basis": "nominal 5 (4 m^2 n + 2 m^3) per block",
         "achieved": round(nom / (avg_ms / 1e3) / 1e12, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    r["frac"] = round(r["achieved"] / PEAK_BF16_TFLOPS, 4)
    if k == "ns_loop":
        per_block = nom / res["nb"]
        assert abs(per_block - ns_flops(768, 3072)) < 1e-6 * per_block
        ex = executed / launches          # the library's count of the tiles the launch ran
        assert abs(ex - res["nb"] * loop_executed_flops(768, 3072)) <= 1e-9 * ex
        alg = res["nb"] * ns_flops_symmetric(768, 3072)
        r["achieved_executed"] = round(ex / (avg_ms / 1e3) / 1e12, 2)
        r["frac_executed"] = round(r["achieved_executed"] / PEAK_BF16_TFLOPS, 4)
        r["achieved_algorithmic"] = round(alg / (avg_ms / 1e3) / 1e12, 2)
        r["frac_algorithmic"] = round(r["achieved_algorithmic"] / PEAK_BF16_TFLOPS, 4)
        r["executed_flops_per_launch"] = ex
        r["algorithmic_flops_per_launch"] = alg
        r["mfma_busy_frac"] = load_profile("k_ns_loop_metric32_sq", GEMM_SOURCE, "mfma_busy_frac")
        r["traffic"] = load_profile("k_ns_loop_metric32_traffic", GEMM_SOURCE, "bytes_per_launch")
    else:
        r["traffic"] = None
    r.update({"launches": launches, "avg_launch_ms": round(avg_ms, 5), "flops_per_launch": nom,
              "ns_family_ms_per_call": {f: round(v[1] / steps, 4) for f, v in ns.items()}})
    total_reported = sum(v[2] for v in ns.values()) / steps
    r["flops_accounted"] = abs(total_reported - res["nominal"]) <= 1e-9 * res["nominal"]
    return r


def gpt124m_step(nsm, args, dev):
    """The full Muon step of the 124M custom-sizing set (muon_step_multi)."""
    import torch
    import workloads
    wl = workloads.get_workload("gpt124m")
    state = []
    for g in wl.groups:
        P = workloads.params_device(wl, g, dev)
        state.append((g, P, workloads.grads_device(wl, g, 0, dev), torch.zeros_like(P)))
    mats = [dict(params=P[i], grads=G[i], momentum_buf=M[i], view_blocks=g.view_blocks)
            for g, P, G, M in state for i in range(g.count)]
    step = lambda: nsm.muon_step_multi(mats, lr=wl.lr, weight_decay=wl.weight_decay,   # noqa: E731
                                       momentum=wl.momentum, ns_steps=wl.ns_steps, precision="fast")
    for _ in range(SETTLE_CALLS):
        step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    ms = timed_region(step, args.steps)
    with Timer(nsm, nsm.KERNEL_KINDS) as t:
        for _ in range(args.steps):
            step()
    fam = t.result
    flops = sum(g.n_blocks * ns_flops(*g.block_shape) for g in wl.groups)
    n_blocks = sum(g.n_blocks for g in wl.groups)
    ns = {k: v for k, v in fam.items() if k in NS_FAMILIES}
    ns_ms = sum(v[1] for v in ns.values()) / args.steps
    executed = sum(v[3] for v in ns.values()) / args.steps
    # the element-wise kernels (blocks on the matrix-core path): 12 B per
    # element before NS (g 2, M 8, U 2), 10 B after (P 8, O 2)
    mfma_elems = sum(g.count * g.rows * g.cols for g in wl.groups if min(g.block_shape) > 64)
    out = {"workload": "124M GPT custom sizing: 11 gates 1x12 (fp32 small-block path) + 10 attn 768x3072 viewed "
                       "as 4x768x768 + 22 mlp 768x3072; muon_step_multi, momentum 0.95 Nesterov, 5 NS steps, "
                       "lr 0.05, wd 0, FAST",
           "ms": round(ms, 4), "tflops_nominal": round(flops / (ms / 1e3) / 1e12, 2),
           "mfma_peak_frac_nominal": round(flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "matrices_per_s": round(wl.n_matrices / (ms / 1e3), 1),
           "matrices_per_s_excluding_gates": round(32 / (ms / 1e3), 1),
           "ns_blocks_per_s": round(n_blocks / (ms / 1e3), 1),
           "ns_kernels": {"ms_per_step": round(ns_ms, 4),
                          "tflops_executed": round(executed / (ns_ms / 1e3) / 1e12, 2),
                          "frac_executed": round(executed / (ns_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
           "kernel_ms_per_step": {k: round(v[1] / args.steps, 4) for k, v in fam.items()}}
    for kind, bpe, name in (("prep", 12, "k_prep"), ("finish", 10, "k_finish")):
        if kind in fam:
            n_l, tot = fam[kind][0], fam[kind][1]
            gbs = bpe * mfma_elems / (tot / args.steps / 1e3) / 1e9
            out[kind] = {"kernel": name, "bound": "hbm", "bytes_per_element": bpe, "elements": mfma_elems,
                         "launches_per_step": n_l // args.steps, "ms_per_step": round(tot / args.steps, 4),
                         "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": load_profile(f"{name}_gpt124m_traffic", EW_SOURCE, "bytes_per_step")}
    out["status"] = nsm.last_call_status(dev)
    del state, mats
    return out


def rank_shares(nsm, args, dev):
    """One GPU's share of the 124M set under 8-way sharding by whole matrices:
    2 attn matrices (8 blocks of 768x768) or 2 mlp matrices 768x3072, each a
    muon_step_batched call."""
    import torch
    import workloads
    wl = workloads.get_workload("gpt124m")
    groups = {g.name: g for g in wl.groups}
    out = {}
    for name, gname in (("c3_share_attn", "attn"), ("c3_share_mlp", "mlp")):
        g = groups[gname]
        P = workloads.params_device(wl, g, dev)[:2].contiguous()
        G = workloads.grads_device(wl, g, 0, dev)[:2].contiguous()
        M = torch.zeros_like(P)
        step = lambda: nsm.muon_step_batched(P, G, M, lr=wl.lr, weight_decay=wl.weight_decay,  # noqa: E731
                                             momentum=wl.momentum, view_blocks=g.view_blocks,
                                             ns_steps=wl.ns_steps, precision="fast")
        for _ in range(SETTLE_CALLS):
            step()
            torch.cuda.synchronize()
        for _ in range(args.warmup):
            step()
        ms = timed_region(step, args.steps)
        with Timer(nsm, nsm.KERNEL_KINDS) as t:
            for _ in range(args.steps):
                step()
        # The same step captured once into a HIP graph and replayed (the launch
        # gaps of its ~17 dependent launches are most of what a share waits for).
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        ms_graph = timed_region(graph.replay, args.steps)
        flops = 2 * g.view_blocks * ns_flops(*g.block_shape)
        out[name] = {"blocks": f"{2 * g.view_blocks} x {g.block_shape[0]}x{g.block_shape[1]}",
                     "ms": round(ms, 4), "tflops_nominal": round(flops / (ms / 1e3) / 1e12, 2),
                     "mfma_peak_frac_nominal": round(flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "kernel_ms_per_step": {k: round(v[1] / args.steps, 4) for k, v in t.result.items()},
                     "graph_replay": {"ms": round(ms_graph, 4),
                                      "tflops_nominal": round(flops / (ms_graph / 1e3) / 1e12, 2),
                                      "mfma_peak_frac_nominal": round(flops / (ms_graph / 1e3) / 1e12
                                                                      / PEAK_BF16_TFLOPS, 4)}}
        del P, G, M, graph
    return out


def large_step(nsm, args, dev, name):
    """A full Muon step of a large workload (each shape group one
    muon_step_batched call in the group's precision): the GPT-2-medium-like
    96 x 1024x4096 batch (48 stored tall) or the large dense batch
    8 x 4096^2 + 8 x 4096x14336 (ACCURATE)."""
    import torch
    import workloads
    wl = workloads.get_workload(name)
    state = []
    for g in wl.groups:
        P = workloads.params_device(wl, g, dev)
        state.append((g, P, workloads.grads_device(wl, g, 0, dev), torch.zeros_like(P)))

    def step():
        for g, P, G, M in state:
            nsm.muon_step_batched(P, G, M, lr=wl.lr, weight_decay=wl.weight_decay, momentum=wl.momentum,
                                  view_blocks=g.view_blocks, ns_steps=wl.ns_steps, precision=g.precision)
    steps = max(1, min(args.steps, 10))
    for _ in range(SETTLE_CALLS):
        step()
        torch.cuda.synchronize()
    for _ in range(min(args.warmup, 3)):
        step()
    ms = timed_region(step, steps)
    with Timer(nsm, nsm.KERNEL_KINDS) as t:
        for _ in range(steps):
            step()
    fam = t.result
    nominal = sum(g.n_blocks * ns_flops(*g.block_shape) for g in wl.groups)
    ns = {k: v for k, v in fam.items() if k in NS_FAMILIES}
    ns_ms = sum(v[1] for v in ns.values()) / steps
    executed = sum(v[3] for v in ns.values()) / steps
    out = {"workload": wl.description, "precision": sorted({g.precision for g in wl.groups}),
           "steps": steps, "ms": round(ms, 4), "nominal_ns_gflop_per_step": round(nominal / 1e9, 1),
           "tflops_nominal": round(nominal / (ms / 1e3) / 1e12, 2),
           "mfma_peak_frac_nominal": round(nominal / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "executed_gflop_per_step": round(executed / 1e9, 1),
           "ns_kernels": {"ms_per_step": round(ns_ms, 4),
                          "tflops_executed": round(executed / (ns_ms / 1e3) / 1e12, 2),
                          "frac_executed": round(executed / (ns_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                          "tflops_nominal": round(nominal / (ns_ms / 1e3) / 1e12, 2)},
           "matrices_per_s": round(wl.n_matrices / (ms / 1e3), 1),
           "kernel_ms_per_step": {k: round(v[1] / steps, 4) for k, v in fam.items()},
           "status": list(nsm.last_call_status(dev))}
    del state
    torch.cuda.empty_cache()
    return out


def adamw_gpt124m(nsm, args, dev):
    import torch
    import workloads
    awl = workloads.ADAM_WORKLOADS["gpt124m_adam"]
    tens = []
    for i in range(len(awl.tensors)):
        P = workloads.adam_params_device(awl, i, dev)
        tens.append(dict(params=P, grads=workloads.adam_grads_device(awl, i, 0, dev),
                         exp_avg=torch.zeros_like(P), exp_avg_sq=torch.zeros_like(P), step=1))

    def adam_step():
        nsm.adamw_step_multi(tens, lr=awl.lr, betas=awl.betas, eps=awl.eps, weight_decay=awl.weight_decay)
        for t in tens:
            t["step"] += 1
    for _ in range(3):
        adam_step()
    torch.cuda.synchronize()
    with Timer(nsm, ["adamw"]) as t:
        for _ in range(args.steps):
            adam_step()
    n_l, a_ms = t.result.get("adamw", (0, 0.0, 0.0))[:2]
    del tens
    if not n_l:
        return None
    ms = a_ms / n_l
    gbs = 26.0 * awl.numel / (ms / 1e3) / 1e9
    return {"kernel": "k_adamw", "elements": awl.numel, "launches": n_l, "avg_launch_ms": round(ms, 5),
            "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_element": 26,
            "traffic": load_profile("k_adamw_gpt124m_traffic", ADAM_SOURCE, "bytes_per_launch")}


def library_baseline(nsm, args, dev, headline_ms=None):
    """The same NS call written as plain PyTorch on the GPU (torch.bmm on
    hipBLASLt, bf16 operands, the pages' five quintic iterations with the
    Gram of the short side), and one large square bf16 GEMM as the rate the
    vendor library reaches when nothing but a single product is asked of it.
    A comparison leg only: the library's own path never calls torch."""
    import torch
    import workloads
    wl = workloads.get_workload("metric32")
    g = wl.groups[0]
    x = workloads.grads_device(wl, g, 0, dev)
    a, b, c = NS_COEFFS

    def torch_ns():
        y = (x.float() / (torch.linalg.vector_norm(x.float(), dim=(1, 2), keepdim=True) + 1e-7)).to(x.dtype)
        for _ in range(NS_STEPS):
            gram = torch.bmm(y, y.transpose(1, 2).contiguous())
            poly = b * gram + c * torch.bmm(gram, gram)
            y = a * y + torch.bmm(poly, y)
        return y

    for _ in range(args.warmup):
        torch_ns()
    torch.cuda.synchronize()
    ms = timed_region(torch_ns, args.steps)
    nominal = g.count * ns_flops(g.rows, g.cols)
    res = {"what": "the same 32 x 768x3072 NS in PyTorch eager (torch.bmm / hipBLASLt, bf16), 5 iterations",
           "ms": round(ms, 4), "tflops_nominal": round(nominal / (ms / 1e3) / 1e12, 2)}
    if headline_ms:
        res["speedup_of_this_library"] = round(ms / headline_ms, 2)
    del x
    n = 8192
    p = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    q = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        p @ q
    torch.cuda.synchronize()
    ms = timed_region(lambda: p @ q, args.steps)
    res["gemm_8192_bf16"] = {"ms": round(ms, 4), "tflops": round(2 * n ** 3 / (ms / 1e3) / 1e12, 2),
                             "frac_of_peak": round(2 * n ** 3 / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    del p, q
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="the headline call only")
    ap.add_argument("--extras", default="step,shares,c4,c5,adamw,library",
                    help="comma-separated extras: step (124M Muon step), shares (one GPU's 8-way share), "
                         "c4 (96 x 1024x4096 step), c5 (large dense ACCURATE step), adamw, "
                         "library (the same NS call in PyTorch eager on hipBLASLt)")
    ap.add_argument("--ns-schedule", choices=("auto", "persistent", "per_product"), default="auto",
                    help="auto: the library's per-shape choice (default); persistent: all NS iterations of "
                         "a call in one launch; per_product: three launches per iteration")
    ap.add_argument("--extras-only", action="store_true",
                    help="skip the headline call and print the extras alone (for per-extra kernel profiles)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="run a plain device copy of MIB MiB first (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(see DESIGN.md for how the step would shard).", file=sys.stderr)
        sys.exit(2)

    import torch
    import newton_schulz_muon_amd as nsm

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    nsm.load_library()
    nsm.muon_set_ns_schedule(args.ns_schedule)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.extras_only:
        want = set(x.strip() for x in args.extras.split(",") if x.strip())
        result = {"extras_only": True, "extras": sorted(want)}
        if "step" in want:
            result["gpt124m_step"] = gpt124m_step(nsm, args, dev)
        if "shares" in want:
            result["rank_share_8way"] = rank_shares(nsm, args, dev)
        if "c4" in want:
            result["gpt2_medium_step"] = large_step(nsm, args, dev, "gpt2_medium")
        if "c5" in want:
            result["large_dense_step"] = large_step(nsm, args, dev, "large_dense")
        if "adamw" in want:
            result["adamw_gpt124m"] = adamw_gpt124m(nsm, args, dev)
        if "library" in want:
            result["library_baseline"] = library_baseline(nsm, args, dev)
        print(json.dumps(result), flush=True)
        return

    h = headline(nsm, args, dev)
    value = h["nominal"] / (h["ms"] / 1e3) / 1e12
    fams = h["families"]
    used = "persistent" if "ns_loop" in fams else "per_product"
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(h["ms"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "32 matrices 768x3072 bf16 ~N(0, 0.01^2), one ns_orthogonalize_batched call, "
                               "FAST (bf16 MFMA, fp32 accumulate), 5 quintic NS iterations",
                   "matrices": h["nb"], "ns_steps": NS_STEPS, "precision": "fast",
                   "nominal_ns_gflop_per_call": round(h["nominal"] / 1e9, 2), "ns_schedule": args.ns_schedule,
                   "ns_schedule_used": used},
        "matrices_per_s": round(h["nb"] / (h["ms"] / 1e3), 1),
        "mfma_peak_frac_nominal": round(value / PEAK_BF16_TFLOPS, 4),
        "call_ms_percentiles": {"warm": h["warm"], "cold_infinity_cache": h["cold"]},
        "kernel_ms_per_call": {k: round(v[1] / args.steps, 4) for k, v in fams.items()},
        "status": list(h["status"]),
        "roofline": roofline_of(h, args.steps),
    }
    if not args.no_extras:
        want = set(x.strip() for x in args.extras.split(",") if x.strip())
        if "step" in want:
            result["gpt124m_step"] = gpt124m_step(nsm, args, dev)
        if "shares" in want:
            result["rank_share_8way"] = rank_shares(nsm, args, dev)
        if "c4" in want:
            result["gpt2_medium_step"] = large_step(nsm, args, dev, "gpt2_medium")
        if "c5" in want:
            result["large_dense_step"] = large_step(nsm, args, dev, "large_dense")
        if "adamw" in want:
            result["adamw_gpt124m"] = adamw_gpt124m(nsm, args, dev)
        if "library" in want:
            lib = library_baseline(nsm, args, dev, h["ms"])
            result["library_baseline"] = lib
            # the vendor library's large-GEMM rate on the same box, as a practical ceiling
            rf = result["roofline"]
            ceil = lib["gemm_8192_bf16"]["tflops"]
            if rf.get("achieved_executed") is not None:
                rf["vendor_gemm_ceiling"] = {"tflops": ceil, "frac_of_peak": lib["gemm_8192_bf16"]["frac_of_peak"],
                                             "executed_frac_of_ceiling": round(rf["achieved_executed"] / ceil, 4)}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
