#!/usr/bin/env python3
"""Throughput of the virtual-noise ES linear layer on one MI355X.

One step = the whole hot path over one batch of synthetic input: the
perturbed-linear forward of every layer of the workload, then the weight and
bias gradient estimators of every parameter block.  Inputs are resident in
HBM before the timed region.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload 2] [--no-cpu-baseline]

The default workload is the MLP hidden layer (pop 256, batch 32 per
individual, 1024 -> 1024, fp32).  Per-kernel durations come from HIP events
recorded on the stream the kernels are launched on, inside the timed steps.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "perturbed-linear TFLOP/s + noise-gradient elements/s, % of roofline, 1 GPU"

# MI355X (gfx950) unit counts and clock used for the ALU roofline.
N_CU = 256
LANES_PER_CU_CLK = 64          # 4 SIMDs x 16 lanes: full-rate 32-bit VALU lane-ops per clock per CU
CLOCK_HZ = 2.4e9
# Lane-cycles per noise element of the shipped kernels (ISA count of one hash,
# quarter-rate 32-bit multiplies counted 4): state add 1, 2 x (64-bit shift 1,
# xor 2, multiply 3 x 4 + add 1), final shift+xor 2, >>8 1, cvt 1, fma 1.
HASH_LANE_CYCLES = {"forward": 39.0, "gradient": 39.0}
HBM_PEAK_GBS = 8000.0


def hash_peak_per_s(kind: str) -> float:
    return N_CU * LANES_PER_CU_CLK * CLOCK_HZ / HASH_LANE_CYCLES[kind]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0,
                    help="approximate CPU seconds for the oracle baseline sample")
    return ap.parse_args()


class Step:
    """The workload's tensors on the device and one pass of the hot path."""

    def __init__(self, wl, torch, vn, device):
        self.wl = wl
        self.vn = vn
        self.torch = torch
        dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        self.x = torch.from_numpy(wl.x).to(dt).to(device)
        self.layers = []
        for L in wl.layers:
            w = torch.from_numpy(L.weight).to(dt).to(device)
            b = None if L.bias is None else torch.from_numpy(L.bias).to(device)
            self.layers.append((L, w, b))
        self.seeds = torch.from_numpy(wl.seeds).to(device)
        self.fit = torch.from_numpy(wl.fitness).to(device)
        # outputs preallocated so the step does no allocation
        self.ys = [torch.empty((wl.pop, wl.batch, L.out_features), dtype=torch.float32, device=device)
                   for L in wl.layers]
        self.gws = [torch.empty(L.out_features * L.in_features, dtype=torch.float32, device=device)
                    for L in wl.layers]
        self.gbs = [None if L.bias is None else torch.empty(L.out_features, dtype=torch.float32, device=device)
                    for L in wl.layers]

    def forward_only(self, math):
        """Forward of every layer in the given math mode (for a side measurement)."""
        wl, vn = self.wl, self.vn
        h = self.x
        n = len(self.layers)
        for li, (L, w, b) in enumerate(self.layers):
            act = "relu" if (wl.relu_between and li < n - 1) else None
            vn.virtual_perturbed_linear(h, w, b, self.seeds, wl.sigma, L.w_offset, activation=act,
                                        out=self.ys[li], math=math)
            h = self.ys[li]

    def run(self, events=None):
        """events: optional list to which (name, start_event, end_event) are appended."""
        wl, vn, torch = self.wl, self.vn, self.torch
        E = torch.cuda.Event

        def timed(name, fn):
            if events is None:
                fn()
                return
            a, b = E(enable_timing=True), E(enable_timing=True)
            a.record()
            fn()
            b.record()
            events.append((name, a, b))

        h = self.x
        n = len(self.layers)
        for li, (L, w, b) in enumerate(self.layers):
            act = "relu" if (wl.relu_between and li < n - 1) else None
            y = self.ys[li]
            timed(f"forward{li}", lambda h=h, w=w, b=b, L=L, y=y, act=act: vn.virtual_perturbed_linear(
                h, w, b, self.seeds, wl.sigma, L.w_offset, activation=act, out=y))
            h = y
        for li, (L, w, b) in enumerate(self.layers):
            timed(f"grad_w{li}", lambda L=L, g=self.gws[li]: vn.virtual_flat_gradient(
                self.fit, self.seeds, L.out_features * L.in_features, wl.sigma, wl.pop, L.w_offset, out=g))
            if b is not None:
                timed(f"grad_b{li}", lambda L=L, g=self.gbs[li]: vn.virtual_flat_gradient(
                    self.fit, self.seeds, L.out_features, wl.sigma, wl.pop, L.b_offset, out=g))


def flops_of(wl) -> float:
    return float(sum(2.0 * wl.pop * wl.batch * L.in_features * L.out_features for L in wl.layers))


def fwd_hashes(wl) -> float:
    return float(sum(wl.pop * (L.out_features * L.in_features + (L.out_features if L.bias is not None else 0))
                     for L in wl.layers))


def grad_elems(wl) -> float:
    return float(sum(wl.pop * (L.out_features * L.in_features + (L.out_features if L.bias is not None else 0))
                     for L in wl.layers))


def cpu_baseline(wl, budget_s: float):
    """Time the CPU oracle (single thread) on a bounded sample of the same
    workload and scale it to one step of the metric's unit."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(1)
    except Exception:  # pragma: no cover
        limiter = None
    sig = float(np.float32(wl.sigma))
    fit = wl.fitness.astype(np.float64)
    # forward: whole individuals through every layer
    t0 = time.perf_counter()
    k = 0
    while k < wl.pop and (time.perf_counter() - t0) < budget_s / 2:
        h = wl.x[k:k + 1].astype(np.float64)
        for li, L in enumerate(wl.layers):
            h = oracle.perturbed_linear(h, L.weight, L.bias, wl.seeds[k:k + 1], sig, L.w_offset)
            if wl.relu_between and li < len(wl.layers) - 1:
                h = np.maximum(h, 0.0)
        k += 1
    t_fwd = time.perf_counter() - t0
    fwd_per_indiv = t_fwd / k
    # gradients: chunks of flat elements of the chained parameter vector (all individuals)
    rng = np.random.default_rng(0)
    total = wl.total_params
    t1 = time.perf_counter()
    m = 0
    chunk = 4096
    while m < total and (time.perf_counter() - t1) < budget_s / 2:
        start = int(rng.integers(0, max(total - chunk, 1)))
        oracle.weight_gradient_at(fit, wl.seeds, sig, wl.pop, 0, np.arange(start, min(start + chunk, total)))
        m += min(chunk, total)
    t_grad = time.perf_counter() - t1
    grad_per_elem = t_grad / m
    if limiter is not None:
        limiter.unregister() if hasattr(limiter, "unregister") else None
    est_step = fwd_per_indiv * wl.pop + grad_per_elem * total
    return {
        "value": flops_of(wl) / est_step / 1e12,
        "unit": "TFLOP/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"numpy oracle, 1 thread: forward of {k} of {wl.pop} individuals through all layers "
                   f"({t_fwd:.1f} s) and gradients of {m} of {total} flat elements over all {wl.pop} "
                   f"individuals ({t_grad:.1f} s), scaled to one step ({est_step:.1f} s)"),
        "step_s_estimate": est_step,
        "grad_elements_per_s": wl.pop * m / t_grad,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import virtual_noise_perturbed_amd as vn
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    device = torch.device("cuda:0")
    wl = workloads.make(args.workload)
    step = Step(wl, torch, vn, device)

    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()

    events = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step.run(events)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps

    per_kernel = {}
    for name, a, b in events:
        per_kernel.setdefault(name, []).append(a.elapsed_time(b))
    avg_ms = {k: float(np.mean(v)) for k, v in per_kernel.items()}
    fwd_ms = sum(v for k, v in avg_ms.items() if k.startswith("forward"))
    grad_ms = sum(v for k, v in avg_ms.items() if k.startswith("grad"))

    # dominant kernel: the launch with the largest average duration
    dom = max(avg_ms, key=avg_ms.get)
    li = int(dom[-1])
    L = wl.layers[li]
    if dom.startswith("forward"):
        units = wl.pop * (L.out_features * L.in_features + (L.out_features if L.bias is not None else 0))
        kind = "forward"
    elif dom.startswith("grad_w"):
        units = wl.pop * L.out_features * L.in_features
        kind = "gradient"
    else:
        units = wl.pop * L.out_features
        kind = "gradient"
    achieved = units / (avg_ms[dom] * 1e-3) / 1e9
    peak = hash_peak_per_s(kind) / 1e9
    roofline = {
        "bound": "alu",
        "kernel": dom,
        "achieved": round(achieved, 2),
        "peak": round(peak, 2),
        "unit": "Ghash/s",
        "frac": round(achieved / peak, 4),
        "traffic": None,
        "units_per_launch": units,
        "avg_launch_ms": round(avg_ms[dom], 4),
    }

    value = flops_of(wl) / (ms_per_step * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "pop": wl.pop,
            "batch": wl.batch,
            "layers": [[L.in_features, L.out_features] for L in wl.layers],
            "sigma": wl.sigma,
            "step": "forward of every layer + weight and bias gradient of every block",
        },
        "breakdown": {
            "forward_ms": round(fwd_ms, 4),
            "gradient_ms": round(grad_ms, 4),
            "forward_tflops": round(flops_of(wl) / (fwd_ms * 1e-3) / 1e12, 3),
            "forward_noise_elements_per_s": fwd_hashes(wl) / (fwd_ms * 1e-3),
            "gradient_elements_per_s": grad_elems(wl) / (grad_ms * 1e-3),
            "gradient_frac_of_hash_peak": round(grad_elems(wl) / (grad_ms * 1e-3) / hash_peak_per_s("gradient"), 4),
            "forward_frac_of_hash_peak": round(fwd_hashes(wl) / (fwd_ms * 1e-3) / hash_peak_per_s("forward"), 4),
            "per_launch_ms": {k: round(v, 4) for k, v in avg_ms.items()},
        },
    }
    if wl.dtype == "f32":
        # side measurement: the same forward on the fp32 matrix cores (math mode "f32")
        for _ in range(2):
            step.forward_only("f32")
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            step.forward_only("f32")
        b.record()
        torch.cuda.synchronize()
        result["breakdown"]["forward_ms_fp32_matrix_cores"] = round(a.elapsed_time(b) / args.steps, 4)
        result["config"]["forward_math"] = "fp32 operands as three bf16 matrix-core products, fp32 accumulation"
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget_s)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
