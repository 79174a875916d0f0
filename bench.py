#!/usr/bin/env python3
"""Benchmark of the batched Muon step on one MI355X.

A step is one pass of the whole hot path over one batch: momentum, per-block
Frobenius normalisation, 5 quintic Newton-Schulz iterations, aspect-scaled
decoupled-decay update, for the 124M GPT custom-sizing set: 11 gate matrices
1x12 (first), 10 attention matrices stored 768x3072 and viewed as 4 x 768x768,
and 22 MLP matrices 768x3072 (seeded synthetic bf16 gradients ~N(0, 1e-2),
fp32 parameters and momentum buffers resident in HBM).

Prints one JSON line.  `value` is nominal Newton-Schulz TFLOP/s of the whole
step (5 (4 m^2 n + 2 m^3) flops per NS block, m <= n, divided by the wall-clock
step time); matrices/s and NS blocks/s are reported beside it.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Newton-Schulz TFLOP/s and matrices/s at 32x768x3072 bf16; % of MFMA peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
WORKLOAD = "gpt124m"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_bx_gpt124m_traffic.json")
LOOP_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_ns_loop_gpt124m_traffic.json")
# The NS kernel families (library timing names) and the counter runs of each.
NS_FAMILIES = {"ns_loop": "k_ns_loop (every NS iteration of a wave: X X^T, aI + bA + cA^2, B' X; nominal flops)",
               "gram": "k_gemm<kGram> (A = X X^T; nominal flops)",
               "poly": "k_gemm<kPoly> (B' = aI + bA + cA^2; nominal flops of A A)",
               "bx": "k_gemm<kBx> (X <- B' X; nominal flops)"}
TRAFFIC_FILES = {"ns_loop": LOOP_TRAFFIC_FILE, "bx": TRAFFIC_FILE}
GEMM_SOURCE = os.path.join(ROOT, "newton_schulz_muon_amd", "csrc", "ns_gemm.hip")
ADAM_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_adamw_gpt124m_traffic.json")
ADAM_SOURCE = os.path.join(ROOT, "newton_schulz_muon_amd", "csrc", "adamw.hip")
SETTLE_CALLS = 12              # calls before warm-up that let the automatic NS schedule choose


def ns_flops(m: int, n: int, steps: int) -> float:
    """Nominal NS work of one block: steps * (4 m^2 n + 2 m^3), m <= n."""
    m, n = min(m, n), max(m, n)
    return float(steps) * (4.0 * m * m * n + 2.0 * m ** 3)


def source_digest(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(path: str = TRAFFIC_FILE, source: str = GEMM_SOURCE):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter
    runs, or None when they are missing or the kernel source changed since."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256_16") != source_digest(source):
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(wl, seconds: float):
    """The fp64 oracle on a bounded sample of the workload (host cores)."""
    import numpy as np
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        threads = os.cpu_count() or 1
    groups = {g.name: g for g in wl.groups}
    plan = [("gate", i) for i in range(groups["gate"].count)]
    for i in range(max(groups["mlp"].count, groups["attn"].count)):
        if i < groups["mlp"].count:
            plan.append(("mlp", i))
        if i < groups["attn"].count:
            plan.append(("attn", i))
    done_flops, done_mats, used = 0.0, 0, []
    t0 = time.perf_counter()
    for name, i in plan:
        g = groups[name]
        G = workloads.bf16_bits_to_f32(workloads.grad_bits_host(wl, g, 0, [i])).astype(np.float64)
        P = workloads.param_init_host(wl, g, [i]).astype(np.float64)
        M = np.zeros_like(G)
        oracle.muon_step(P, G, M, lr=wl.lr, weight_decay=wl.weight_decay, momentum=wl.momentum,
                         view_blocks=g.view_blocks, ns_steps=wl.ns_steps)
        r, c = g.block_shape
        done_flops += g.view_blocks * ns_flops(r, c, wl.ns_steps)
        done_mats += 1
        used.append(f"{name}[{i}]")
        if time.perf_counter() - t0 > seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": done_flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 numpy oracle, one full Muon step of {done_mats} matrices "
                      f"({', '.join(used)}) in {dt:.1f} s; {done_mats / dt:.3f} matrices/s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the kernel breakdown and NS-only passes")
    ap.add_argument("--api", choices=("multi", "batched"), default="multi",
                    help="multi: one muon_step_multi call per step over all matrices (default); "
                         "batched: one muon_step_batched call per shape group")
    ap.add_argument("--ns-schedule", choices=("auto", "persistent", "per_product"), default="auto",
                    help="auto: the library's per-shape choice (default); persistent: all NS iterations of "
                         "a wave in one launch; per_product: three launches per iteration")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="run a plain device copy of MIB MiB first (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(see DESIGN.md for how the step would shard).", file=sys.stderr)
        sys.exit(2)

    import torch
    import newton_schulz_muon_amd as nsm
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    nsm.load_library()
    nsm.muon_set_ns_schedule(args.ns_schedule)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workloads.get_workload(WORKLOAD)

    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    state = []
    for g in wl.groups:
        P = workloads.params_device(wl, g, dev)
        G = workloads.grads_device(wl, g, 0, dev)
        M = torch.zeros_like(P)
        state.append((g, P, G, M))
    torch.cuda.synchronize()

    # every matrix of the workload, each a [rows, cols] slice of its group's stack
    matrices = [dict(params=P[i], grads=G[i], momentum_buf=M[i], view_blocks=g.view_blocks)
                for g, P, G, M in state for i in range(g.count)]

    def step():
        if args.api == "multi":
            nsm.muon_step_multi(matrices, lr=wl.lr, weight_decay=wl.weight_decay, momentum=wl.momentum,
                                ns_steps=wl.ns_steps, precision="fast")
            return
        for g, P, G, M in state:
            nsm.muon_step_batched(P, G, M, lr=wl.lr, weight_decay=wl.weight_decay, momentum=wl.momentum,
                                  view_blocks=g.view_blocks, ns_steps=wl.ns_steps, precision=g.precision)

    # The library's automatic NS schedule times its first ten calls per set of
    # shapes (alternating the per-product launches and the persistent loop)
    # and keeps the faster one once those calls' events have completed: let it
    # settle, synchronising after each call, before the warm-up proper.
    for _ in range(SETTLE_CALLS):
        step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: K steps, no instrumentation
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    # ---- roofline region: the same K steps again, each launch of the NS
    # kernel families bracketed by a hipEvent pair on the library's stream;
    # the library reports each launch's nominal flops beside its time (with
    # the automatic schedule one step may run some waves in the persistent
    # loop and others per product).  Every event record costs a short
    # dispatch bubble, which is why `value` comes from the uninstrumented
    # region above.
    nsm.muon_timing_collect()
    nsm.muon_timing_enable(list(NS_FAMILIES))
    torch.cuda.synchronize()
    r0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    r1 = time.perf_counter()
    nsm.muon_timing_enable([])
    kt = nsm.muon_timing_collect(with_flops=True)

    ms_per_step = (t1 - t0) * 1000.0 / args.steps
    flops_step = sum(g.view_blocks * g.count * ns_flops(*g.block_shape, wl.ns_steps) for g in wl.groups)
    n_blocks = sum(g.n_blocks for g in wl.groups)
    value = flops_step / (ms_per_step / 1000.0) / 1e12

    # Blocks with m <= 64 and m n <= 8192 take the one-launch fp32 small-block
    # path and issue no B'X launch.
    mfma_groups = [g for g in wl.groups
                   if not (min(g.block_shape) <= 64 and g.block_shape[0] * g.block_shape[1] <= 8192)]
    # Every MFMA-path NS flop of the step is reported by exactly one family.
    mfma_flops_step = sum(g.n_blocks * ns_flops(*g.block_shape, wl.ns_steps) for g in mfma_groups)
    reported_step = sum(v[2] for v in kt.values()) / args.steps
    roofline = None
    if kt:
        # dominant kernel: the NS family with the most time per step
        fam = max(kt, key=lambda k: kt[k][1])
        launches, fam_ms, fam_flops = kt[fam]
        achieved = fam_flops / (fam_ms / 1000.0) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                    "traffic": load_traffic(TRAFFIC_FILES.get(fam)) if fam in TRAFFIC_FILES else None,
                    "kernel": NS_FAMILIES[fam],
                    "launches": launches, "avg_launch_ms": round(fam_ms / launches, 5),
                    "flops_per_launch_avg": fam_flops / launches,
                    "region_ms_per_step": round((r1 - r0) * 1000.0 / args.steps, 4),
                    "ns_family_ms_per_step": {k: round(v[1] / args.steps, 4) for k, v in kt.items()},
                    "ns_family_tflops": {k: round(v[2] / (v[1] / 1000.0) / 1e12, 2) for k, v in kt.items()},
                    "flops_accounted": abs(reported_step - mfma_flops_step) <= 1e-9 * mfma_flops_step}

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "124M GPT custom sizing: 11 gates 1x12 + 10 attn 768x3072 viewed as "
                               "4x768x768 + 22 mlp 768x3072; full Muon step (momentum 0.95 Nesterov, "
                               "5 NS steps, lr 0.05, wd 0)",
                   "matrices": wl.n_matrices, "ns_blocks": n_blocks, "ns_steps": wl.ns_steps,
                   "precision": "fast (bf16 MFMA, fp32 accumulate); gates on the fp32 small-block path",
                   "nominal_ns_gflop_per_step": round(flops_step / 1e9, 2)},
        "ns_schedule": args.ns_schedule, "settle_calls": SETTLE_CALLS,
        "matrices_per_s": round(wl.n_matrices / (ms_per_step / 1000.0), 1),
        "ns_blocks_per_s": round(n_blocks / (ms_per_step / 1000.0), 1),
        "mfma_peak_frac_nominal": round(value / PEAK_BF16_TFLOPS, 4),
        "roofline": roofline,
    }

    if not args.no_extras:
        # ---- attribution pass (separate from the timed region): every kernel family timed
        nsm.muon_timing_enable(list(nsm.KERNEL_KINDS))
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        nsm.muon_timing_enable([])
        allk = nsm.muon_timing_collect()
        result["kernel_ms_per_step"] = {k: round(v[1] / args.steps, 4) for k, v in allk.items()}
        ew_bytes = sum(g.count * g.rows * g.cols for g in mfma_groups)
        if "prep" in allk:
            prep_ms = allk["prep"][1] / args.steps
            result["prep_hbm_gbs"] = round(12.0 * ew_bytes / (prep_ms / 1000.0) / 1e9, 1)
        if "finish" in allk:
            fin_ms = allk["finish"][1] / args.steps
            result["finish_hbm_gbs"] = round(10.0 * ew_bytes / (fin_ms / 1000.0) / 1e9, 1)
        # ---- NS only on the metric's exact batch: 32 x 768 x 3072, no view
        x = workloads.grads_device(workloads.get_workload("metric32"), workloads.get_workload("metric32").groups[0], 0, dev)
        out = torch.empty_like(x)
        for _ in range(SETTLE_CALLS):
            nsm.ns_orthogonalize_batched(x, out)
            torch.cuda.synchronize()
        for _ in range(3):
            nsm.ns_orthogonalize_batched(x, out)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            nsm.ns_orthogonalize_batched(x, out)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        # a second pass with every kernel family bracketed by hipEvents (its
        # own region: the events add dispatch bubbles)
        nsm.muon_timing_collect()
        nsm.muon_timing_enable(list(nsm.KERNEL_KINDS))
        for _ in range(args.steps):
            nsm.ns_orthogonalize_batched(x, out)
        torch.cuda.synchronize()
        nsm.muon_timing_enable([])
        fam = nsm.muon_timing_collect()
        used = "persistent" if "ns_loop" in fam else "per_product"
        f = 32 * ns_flops(768, 3072, 5)
        ns_kernels = [k for k in ("ns_loop", "gram", "poly", "bx") if k in fam]
        ns_ms = sum(fam[k][1] for k in ns_kernels) / args.steps
        result["ns_only_32x768x3072"] = {"ms": round(ms, 4), "tflops": round(f / (ms / 1000) / 1e12, 2),
                                         "schedule": used,
                                         "kernel_ms_per_call": {k: round(v[1] / args.steps, 4) for k, v in fam.items()},
                                         "ns_kernels_tflops": round(f / (ns_ms / 1000) / 1e12, 2),
                                         "ns_kernels_frac": round(f / (ns_ms / 1000) / 1e12 / PEAK_BF16_TFLOPS, 4),
                                         "matrices_per_s": round(32 / (ms / 1000), 1),
                                         "mfma_peak_frac_nominal": round(f / (ms / 1000) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del x, out
        # ---- AdamW for the same model's embedding, head and scalars (the other
        # optimizer of the step): 26 bytes of HBM traffic per element.
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
        nsm.muon_timing_enable(["adamw"])
        for _ in range(args.steps):
            adam_step()
        torch.cuda.synchronize()
        nsm.muon_timing_enable([])
        n_l, a_ms = nsm.muon_timing_collect().get("adamw", (0, 0.0))
        if n_l:
            ms = a_ms / n_l
            gbs = 26.0 * awl.numel / (ms / 1000.0) / 1e9
            result["adamw_gpt124m"] = {"kernel": "k_adamw", "elements": awl.numel, "launches": n_l,
                                       "avg_launch_ms": round(ms, 5), "bound": "hbm", "achieved": round(gbs, 1),
                                       "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                                       "traffic": load_traffic(ADAM_TRAFFIC_FILE, ADAM_SOURCE),
                                       "bytes_per_element": 26}
        del tens

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
