#!/usr/bin/env python3
"""Throughput of the virtual-noise ES linear layer on one MI355X.

One step = the whole hot path over one batch of synthetic input: the
perturbed-linear forward of every layer of the workload, then the weight and
bias gradient estimators of every parameter block.  Inputs are resident in
HBM before the timed region.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload 5] [--no-cpu-baseline]

The default workload is the largest of the five reference configurations, the
transformer-width projection (pop 128, batch 256 per individual, 4096 -> 4096,
bf16 operands with fp32 accumulation).  Per-kernel durations come from HIP events
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

# ---------------------------------------------------------------------------
# ALU roofline of the noise hash on MI355X (gfx950).
#
# Every kernel has to produce each noise element: the state step, the
# finalizer (2 x [v_lshrrev_b64, 2 v_xor_b32, v_mul_lo_u32, 2 v_mad_u64_u32,
# v_mov_b32], then v_alignbit_b32 + v_bitop3_b32 for the low word with the
# sign flip), v_ashrrev_i32 for N * 2^24 and v_cvt_f32_i32 -- and consume it
# with at least one fma.  virtual_noise_perturbed_amd/vn_probe measures that
# exact sequence (nothing else in the loop, independent Weyl-stepped chains
# per lane, 2 to 8 waves per SIMD) and reads the shader clock of each launch
# (which moves between 2.0 and 2.43 GHz under load).  The peak prices the
# lowest per-cycle cost in the committed probe runs (profiles/vn_probe_gfx950.txt:
# 16.69 lane-cycles per element, one chain per lane at 8 waves per SIMD; the
# same runs give 16.69-17.28 over occupancies of 8 waves) at the nominal
# 2.4 GHz on 256 CUs x 64 lanes.
CLOCK_HZ = 2.4e9
NOISE_LANE_CYCLES = 16.69   # per element per CU lane, at the measured clock (vn_probe, lowest committed)
HASH_PEAK_PER_S = 256 * 64 * CLOCK_HZ / NOISE_LANE_CYCLES
# The same sequence priced by the sum of its 20 instructions' isolated issue
# costs (the per-instruction rates of the same probe runs): a floor set by
# instruction counts alone.  Mixed, the instructions overlap a little, so this
# peak is lower than the measured one above.
ISSUE_SUM_LANE_CYCLES = 18.57
ISSUE_SUM_PEAK_PER_S = 256 * 64 * CLOCK_HZ / ISSUE_SUM_LANE_CYCLES
HBM_PEAK_GBS = 8000.0
HBM_PEAK = HBM_PEAK_GBS * 1e9   # bytes/s
MFMA_BF16_PEAK = 2.5e15    # dense bf16 matrix-core FLOP/s

KERNEL_SRC = os.path.join(ROOT, "virtual_noise_perturbed_amd", "csrc", "vn_kernels.hip")
GEMM_SRC = os.path.join(ROOT, "virtual_noise_perturbed_amd", "csrc", "vn_gemm.hip")
DEVICE_SRC = os.path.join(ROOT, "virtual_noise_perturbed_amd", "csrc", "vn_device.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def code_without_comments(text: str) -> str:
    """C++ source with // and /* */ comments and blank lines removed, so that
    only code changes count as changes of a kernel (string literals in the
    kernel sources hold no comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in (KERNEL_SRC, GEMM_SRC, DEVICE_SRC):
        with open(f, encoding="utf-8") as fh:
            h.update(code_without_comments(fh.read()).encode())
    return h.hexdigest()[:16]


def recorded_traffic(workload_key: int, kernel: str):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none for this kernel or the kernel source changed since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    ent = rec.get("entries", {}).get(f"{workload_key}:{kernel}")
    return None if ent is None else ent.get("hbm_bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=5, choices=[1, 2, 3, 4, 5, 6])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0,
                    help="approximate CPU seconds for the oracle baseline sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (to scale memory counters)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="only time the vendor bf16 GEMM (torch linear -> hipBLASLt) on the large-batch "
                         "workload's products, for context beside the materialized path")
    ap.add_argument("--fused-chain", action="store_true",
                    help="run a multi-layer workload's forward through the fused chain entry point")
    ap.add_argument("--only", choices=["forward", "gradient", "metric"], default=None,
                    help="run only one kernel family in the timed steps (for profiling runs)")
    return ap.parse_args()


class Step:
    """The workload's tensors on the device and one pass of the hot path."""

    def __init__(self, wl, torch, vn, device, fused=False):
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
        # --fused-chain: all layers in one vn_perturbed_mlp launch (outputs at
        # most 256 wide, batch at most 64).  Off by default: at the 3-layer
        # MLP's shape one launch per layer is as fast or faster.
        fits = all(L.out_features <= 256 for L in wl.layers) and wl.batch <= 64
        self.chain_from = 0 if (fused and len(wl.layers) > 1 and fits) else None
        # Gradient blocks.  When the parameter blocks tile one flat range of
        # noise offsets (weights then bias of each layer, layer after layer),
        # the whole gradient is one launch over that range and each block is a
        # view of it; otherwise one launch per block.
        blocks = []
        for L in wl.layers:
            blocks.append((L.w_offset, L.out_features * L.in_features))
            if L.bias is not None:
                blocks.append((L.b_offset, L.out_features))
        blocks.sort()
        self.flat_base = blocks[0][0]
        self.flat_n = sum(n for _, n in blocks)
        self.flat = all(blocks[k][0] + blocks[k][1] == blocks[k + 1][0] for k in range(len(blocks) - 1))
        if self.flat:
            self.gflat = torch.empty(self.flat_n, dtype=torch.float32, device=device)
            view = lambda off, n: self.gflat[off - self.flat_base: off - self.flat_base + n]
        else:
            view = lambda off, n: torch.empty(n, dtype=torch.float32, device=device)
        self.gws = [view(L.w_offset, L.out_features * L.in_features) for L in wl.layers]
        self.gbs = [None if L.bias is None else view(L.b_offset, L.out_features) for L in wl.layers]

    def forward_launches(self, math="default"):
        """(name, fn) for each forward launch of the step: one per layer, or
        one fused chain ("forward_chain") under --fused-chain; math mode "f32"
        keeps one launch per layer."""
        wl, vn = self.wl, self.vn
        n = len(self.layers)
        out = []
        h = self.x
        chain_from = self.chain_from if math == "default" else None
        for li, (L, w, b) in enumerate(self.layers):
            if chain_from is not None and li == chain_from:
                rest = self.layers[li:]
                out.append(("forward_chain", lambda h=h, rest=rest: vn.virtual_perturbed_mlp(
                    h, [w_ for _, w_, _ in rest], [b_ for _, _, b_ in rest], self.seeds, wl.sigma,
                    [L_.w_offset for L_, _, _ in rest], activation="relu" if wl.relu_between else None,
                    out=self.ys[-1])))
                break
            act = "relu" if (wl.relu_between and li < n - 1) else None
            y = self.ys[li]
            out.append((f"forward{li}", lambda h=h, w=w, b=b, L=L, y=y, act=act: vn.virtual_perturbed_linear(
                h, w, b, self.seeds, wl.sigma, L.w_offset, activation=act, out=y, math=math)))
            h = y
        return out

    def forward_only(self, math):
        """Forward of every layer in the given math mode (for a side measurement)."""
        for _, fn in self.forward_launches(math):
            fn()

    def metric_setup(self):
        """The flat parameter vector (weights then bias of each layer) as the
        centre of the reduce-metric side measurement."""
        torch, wl = self.torch, self.wl
        parts = []
        for L, w, b in self.layers:
            parts.append(w.float().reshape(-1))
            if b is not None:
                parts.append(b.float())
        self.center = torch.cat(parts).contiguous()
        self.metric_out = None

    def metric(self):
        wl = self.wl
        self.metric_out = self.vn.virtual_reduce_metric(self.center, self.seeds, wl.sigma, self.center.numel(), 0)

    def gradient_launches(self):
        """(name, fn) for each gradient launch of the step."""
        wl, vn = self.wl, self.vn
        if self.flat:
            return [("grad_flat", lambda: vn.virtual_flat_gradient(
                self.fit, self.seeds, self.flat_n, wl.sigma, wl.pop, self.flat_base, out=self.gflat))]
        out = []
        for li, (L, w, b) in enumerate(self.layers):
            out.append((f"grad_w{li}", lambda L=L, g=self.gws[li]: vn.virtual_flat_gradient(
                self.fit, self.seeds, L.out_features * L.in_features, wl.sigma, wl.pop, L.w_offset, out=g)))
            if b is not None:
                out.append((f"grad_b{li}", lambda L=L, g=self.gbs[li]: vn.virtual_flat_gradient(
                    self.fit, self.seeds, L.out_features, wl.sigma, wl.pop, L.b_offset, out=g)))
        return out

    def gradients_only(self):
        for _, fn in self.gradient_launches():
            fn()

    def run(self, events=None, only=None):
        """events: optional EventLog; launches are bracketed by its events (all
        of them, or only the launch named `only`)."""
        wl, vn = self.wl, self.vn

        def timed(name, fn):
            if events is None or (only is not None and name != only):
                fn()
                return
            a, b = events.pair(name)
            a.record()
            fn()
            b.record()

        for name, fn in self.forward_launches():
            timed(name, fn)
        for name, fn in self.gradient_launches():
            timed(name, fn)


class EventLog:
    """Timing events created before the timed region (creating an event costs
    about as much host time as a launch), handed out in pairs per launch."""

    def __init__(self, torch, n_pairs):
        E = torch.cuda.Event
        self.free = [(E(enable_timing=True), E(enable_timing=True)) for _ in range(n_pairs)]
        self.used = []

    def pair(self, name):
        a, b = self.free.pop()
        self.used.append((name, a, b))
        return a, b

    def averages(self):
        per = {}
        for name, a, b in self.used:
            per.setdefault(name, []).append(a.elapsed_time(b))
        return {k: float(np.mean(v)) for k, v in per.items()}


def copy_calibration(torch, device):
    """A plain device-to-device copy of a known number of bytes, under the same
    counters as the kernels, to scale FETCH_SIZE / WRITE_SIZE."""
    n = 256 * 1024 * 1024 // 4            # 256 MiB of fp32
    a = torch.ones(n, dtype=torch.float32, device=device)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                      "launches": 3}))


def vendor_gemm(torch, device, workload, steps):
    """The vendor GEMM on the products the large-batch workload's materialized
    path computes: Y_g = X W_g^T (bf16 operands and output) for 8 weight
    matrices of the workload's shape, back to back; a reference point for the
    matrix-core kernel, not part of the hot path."""
    L = workload.layers[0]
    gen = torch.Generator(device="cpu").manual_seed(7)
    x = torch.randn((workload.batch, L.in_features), generator=gen).to(torch.bfloat16).to(device)
    ws = [torch.randn((L.out_features, L.in_features), generator=gen).to(torch.bfloat16).to(device) for _ in range(8)]
    for _ in range(3):
        for w in ws:
            torch.nn.functional.linear(x, w)
    torch.cuda.synchronize()
    times = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for w in ws:
            torch.nn.functional.linear(x, w)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    times.sort()
    ms = times[len(times) // 2]
    flops = 8 * 2.0 * workload.batch * L.in_features * L.out_features
    print(json.dumps({"vendor_gemm": "torch.nn.functional.linear, bf16, 8 products", "batch": workload.batch,
                      "in": L.in_features, "out": L.out_features, "ms_per_8_products": round(ms, 4),
                      "tflops": round(flops / ms / 1e9, 1), "frac_of_bf16_peak": round(flops / ms / 1e9 / 2500, 4),
                      "steps": steps}))


def flops_of(wl) -> float:
    return float(sum(2.0 * wl.pop * wl.batch * L.in_features * L.out_features for L in wl.layers))


def fwd_hashes(wl) -> float:
    return float(sum(wl.pop * (L.out_features * L.in_features + (L.out_features if L.bias is not None else 0))
                     for L in wl.layers))


def algorithmic_bytes(wl, dom: str, chain_layers, flat_n: int) -> int:
    """Bytes one launch of `dom` must move at least: every input read once and
    every output written once (X, W, biases, seeds and Y for a forward; the
    fitness, the seeds and the gradient for the flat gradient)."""
    esz = 2 if wl.dtype == "bf16" else 4
    seeds = wl.pop * 8
    if dom.startswith("grad"):
        return wl.pop * 4 + seeds + flat_n * 4
    layers = chain_layers if dom == "forward_chain" else [wl.layers[int(dom[-1])]]
    first = layers[0]
    if dom == "forward_chain" or dom == "forward0":
        x = (wl.x.size if wl.x.ndim == 2 else wl.pop * wl.batch * first.in_features) * esz
    else:
        x = wl.pop * wl.batch * first.in_features * 4      # fp32 activations of the previous layer
    w = sum(L.out_features * L.in_features * esz + (L.out_features * 4 if L.bias is not None else 0)
            for L in layers)
    y = wl.pop * wl.batch * layers[-1].out_features * 4
    return int(x + w + seeds + y)


def grad_elems(wl) -> float:
    return float(sum(wl.pop * (L.out_features * L.in_features + (L.out_features if L.bias is not None else 0))
                     for L in wl.layers))


_CPU_WL = None


def _cpu_worker_init(key: int):
    """Pool worker: one BLAS thread, the workload built once."""
    global _CPU_WL
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass
    import workloads
    _CPU_WL = workloads.make(key)


def _cpu_forward_job(i: int) -> float:
    """The oracle forward of individual i through every layer; seconds taken."""
    import oracle
    wl = _CPU_WL
    t0 = time.perf_counter()
    sig = float(np.float32(wl.sigma))
    h = (wl.x[None] if wl.x.ndim == 2 else wl.x[i:i + 1]).astype(np.float64)
    for li, L in enumerate(wl.layers):
        h = oracle.perturbed_linear(h, L.weight, L.bias, wl.seeds[i:i + 1], sig, L.w_offset)
        if wl.relu_between and li < len(wl.layers) - 1:
            h = np.maximum(h, 0.0)
    return time.perf_counter() - t0


def _cpu_gradient_job(start_count) -> float:
    """The oracle gradient estimator over `count` flat elements from `start`, all individuals."""
    import oracle
    wl = _CPU_WL
    start, count = start_count
    t0 = time.perf_counter()
    oracle.weight_gradient_at(wl.fitness.astype(np.float64), wl.seeds, float(np.float32(wl.sigma)), wl.pop, 0,
                              np.arange(start, start + count))
    return time.perf_counter() - t0


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(wl, budget_s: float, max_procs: int = 16):
    """Time the CPU oracle on the host's cores on a bounded sample of the same
    workload and scale it to one step of the metric's unit.  One process per
    core (at most `max_procs`, the host share of one GPU), each running the
    oracle with one BLAS thread; half the budget goes to whole individuals
    through the forward (in turn, cycling over the population), half to runs
    of 4096 gradient elements at random starts over the full population."""
    import multiprocessing as mp
    procs = max(1, min(os.cpu_count() or 1, max_procs))
    ctx = mp.get_context("spawn")          # the workers never touch the GPU or inherit its state
    rng = np.random.default_rng(0)
    total = wl.total_params
    chunk = min(4096, total)
    with ctx.Pool(procs, initializer=_cpu_worker_init, initargs=(wl.key,)) as pool:
        pool.map(_cpu_forward_job, [0] * procs)          # workers built and warm before timing
        # forward: rounds of `procs` individuals until half the budget is spent
        t0 = time.perf_counter()
        k = 0
        while k == 0 or time.perf_counter() - t0 < budget_s / 2:
            pool.map(_cpu_forward_job, [(k + q) % wl.pop for q in range(procs)])
            k += procs
        t_fwd = time.perf_counter() - t0
        # gradients: rounds of `procs` runs of `chunk` flat elements
        t1 = time.perf_counter()
        m = 0
        while m == 0 or time.perf_counter() - t1 < budget_s / 2:
            starts = [int(rng.integers(0, max(total - chunk, 1))) for _ in range(procs)]
            pool.map(_cpu_gradient_job, [(st, chunk) for st in starts])
            m += procs * chunk
        t_grad = time.perf_counter() - t1
    fwd_per_indiv = t_fwd / k                   # wall seconds per individual with all workers busy
    grad_per_elem = t_grad / m
    est_step = fwd_per_indiv * wl.pop + grad_per_elem * total
    return {
        "value": flops_of(wl) / est_step / 1e12,
        "unit": "TFLOP/s",
        "cores": procs,
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "host_cpus": os.cpu_count(),
        "sample": (f"numpy oracle in {procs} processes x 1 BLAS thread: forward of {k} individuals (in turn over "
                   f"the population of {wl.pop}) through all layers ({t_fwd:.1f} s wall) and gradients of "
                   f"{m // chunk} runs of {chunk} flat elements at random starts (of {total}) over all "
                   f"{wl.pop} individuals ({t_grad:.1f} s wall), scaled to one step ({est_step:.2f} s)"),
        "step_s_estimate": est_step,
        "forward_s_per_step": fwd_per_indiv * wl.pop,
        "gradient_s_per_step": grad_per_elem * total,
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
    if args.copy_calibration:
        copy_calibration(torch, device)
        return
    if args.vendor_gemm:
        vendor_gemm(torch, device, workloads.make(6), max(args.steps // 5, 5))
        return
    wl = workloads.make(args.workload)
    step = Step(wl, torch, vn, device, fused=args.fused_chain)
    if args.only is not None:
        # profiling aid: the timed steps of one kernel family only
        if args.only == "metric":
            step.metric_setup()
        for _ in range(args.warmup + args.steps):
            if args.only == "forward":
                step.forward_only("default")
            elif args.only == "metric":
                step.metric()
            else:
                step.gradients_only()
        torch.cuda.synchronize()
        print(json.dumps({"only": args.only, "workload": wl.name, "launches": args.warmup + args.steps}))
        return

    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()

    # Per-launch durations of every kernel family, from event-bracketed steps
    # outside the timed region (an event pair on the stream costs the GPU
    # several microseconds, which would inflate the step time).
    n_launch = len(step.forward_launches()) + len(step.gradient_launches())
    cal = EventLog(torch, n_launch * max(args.steps // 5, 4))
    for _ in range(max(args.steps // 5, 4)):
        step.run(cal)
    torch.cuda.synchronize()
    avg_ms = cal.averages()
    # dominant kernel: the launch with the largest average duration
    dom = max(avg_ms, key=avg_ms.get)

    # Timed region: K whole steps; only the dominant launch is bracketed by
    # events, for the roofline.
    live = EventLog(torch, args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step.run(live, only=dom)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    avg_ms[dom] = live.averages()[dom]
    fwd_ms = sum(v for k, v in avg_ms.items() if k.startswith("forward"))
    grad_ms = sum(v for k, v in avg_ms.items() if k.startswith("grad"))
    chain_layers = wl.layers[step.chain_from:] if step.chain_from is not None else []
    if dom == "grad_flat":
        units = wl.pop * step.flat_n
    elif dom == "forward_chain":
        units = wl.pop * sum(L.out_features * L.in_features + (L.out_features if L.bias is not None else 0)
                             for L in chain_layers)
    else:
        L = wl.layers[int(dom[-1])]
        if dom.startswith("forward"):
            units = wl.pop * (L.out_features * L.in_features + (L.out_features if L.bias is not None else 0))
        elif dom.startswith("grad_w"):
            units = wl.pop * L.out_features * L.in_features
        else:
            units = wl.pop * L.out_features
    achieved = units / (avg_ms[dom] * 1e-3)
    traffic = recorded_traffic(args.workload, dom)
    # The binding unit of the dominant launch: the hash on the VALU, or -- for
    # a forward with enough rows per individual -- the matrix cores.  fp32
    # operands run as three bf16 products, so their matrix-core work is 3x.
    mfma_work = 0.0
    if dom.startswith("forward"):
        Ls = chain_layers if dom == "forward_chain" else [wl.layers[int(dom[-1])]]
        mfma_work = sum(2.0 * wl.pop * wl.batch * L.in_features * L.out_features for L in Ls) * \
            (1 if wl.dtype == "bf16" else 3)
    t_hash = units / HASH_PEAK_PER_S
    t_mfma = mfma_work / MFMA_BF16_PEAK
    # The three bounds of the dominant launch as fractions of its measured
    # duration (the binding one is `frac`): noise generation, matrix cores, and
    # HBM on its algorithmic bytes (and on the measured traffic when recorded).
    t_launch = avg_ms[dom] * 1e-3
    alg_bytes = algorithmic_bytes(wl, dom, chain_layers, step.flat_n)
    fractions = {
        "hash": round(t_hash / t_launch, 4),
        "mfma": round(t_mfma / t_launch, 4),
        "hbm_algorithmic": round(alg_bytes / HBM_PEAK / t_launch, 4),
        "hbm_measured": None if traffic is None else round(traffic / HBM_PEAK / t_launch, 4),
        "algorithmic_bytes_per_launch": alg_bytes,
    }
    if t_mfma > t_hash:
        roofline = {
            "bound": "mfma",
            "kernel": dom,
            "achieved": round(mfma_work / (avg_ms[dom] * 1e-3) / 1e12, 2),
            "peak": round(MFMA_BF16_PEAK / 1e12, 1),
            "unit": "TFLOP/s",
            "frac": round(mfma_work / (avg_ms[dom] * 1e-3) / MFMA_BF16_PEAK, 4),
            "traffic": traffic,
            "flops_per_launch": mfma_work,
            "avg_launch_ms": round(avg_ms[dom], 4),
            "peak_basis": "dense bf16 matrix cores 2.5 PFLOP/s (fp32 operands count their three bf16 products)",
            "hash_frac": round(achieved / HASH_PEAK_PER_S, 4),
            "fractions": fractions,
        }
    else:
        roofline = {
            "bound": "alu",
            "kernel": dom,
            "achieved": round(achieved / 1e9, 2),
            "peak": round(HASH_PEAK_PER_S / 1e9, 2),
            "unit": "G noise elements/s",
            "frac": round(achieved / HASH_PEAK_PER_S, 4),
            "traffic": traffic,
            "units_per_launch": units,
            "avg_launch_ms": round(avg_ms[dom], 4),
            "peak_basis": (f"noise generation bound: {NOISE_LANE_CYCLES} lane-cycles per noise element "
                           f"(state step, hash, N as fp32, one fma; measured per shader-clock cycle), "
                           f"256 CUs x 64 lanes x 2.4 GHz"),
            "frac_vs_issue_sum": round(achieved / ISSUE_SUM_PEAK_PER_S, 4),
            "issue_sum_basis": (f"{ISSUE_SUM_LANE_CYCLES} lane-cycles per element: the isolated issue costs of "
                                f"the sequence's 20 instructions summed"),
            "fractions": fractions,
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
        "roofline": roofline,
        "breakdown": {
            "forward_ms": round(fwd_ms, 4),
            "gradient_ms": round(grad_ms, 4),
            "forward_tflops": round(flops_of(wl) / (fwd_ms * 1e-3) / 1e12, 3),
            "forward_noise_elements_per_s": fwd_hashes(wl) / (fwd_ms * 1e-3),
            "gradient_elements_per_s": grad_elems(wl) / (grad_ms * 1e-3),
            "gradient_frac_of_hash_peak": round(grad_elems(wl) / (grad_ms * 1e-3) / HASH_PEAK_PER_S, 4),
            "forward_frac_of_hash_peak": round(fwd_hashes(wl) / (fwd_ms * 1e-3) / HASH_PEAK_PER_S, 4),
            # matrix-core work actually issued (fp32 operands: three bf16 products) vs 2.5 PFLOP/s bf16 dense
            "forward_mfma_utilization": round(flops_of(wl) * (1 if wl.dtype == "bf16" else 3) /
                                              (fwd_ms * 1e-3) / 2.5e15, 4),
            "per_launch_ms": {k: round(v, 4) for k, v in avg_ms.items()},
            "per_launch_note": ("event-bracketed steps outside the timed region; the dominant launch "
                                "from events inside the timed region. A bracketed launch also takes the gap "
                                "between its event records and the kernel (a few us, more after a forward), "
                                "so the per-launch times add up to more than ms_per_step, whose unbracketed "
                                "steps are the sum of the kernel times"),
        },
    }
    # side measurement: the dominant launch with cold caches -- a 512 MiB
    # buffer (more than L2 and Infinity Cache together) is written before each
    # repetition, outside the launch's event pair
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=device)
    dom_fn = dict(step.forward_launches() + step.gradient_launches())[dom]
    reps = min(args.steps, 20)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for r, (a, b) in enumerate(pairs):
        flush.fill_(float(r))
        a.record()
        dom_fn()
        b.record()
    torch.cuda.synchronize()
    cold_ms = float(np.mean([a.elapsed_time(b) for a, b in pairs]))
    del flush
    result["breakdown"]["dominant_cold_cache_ms"] = round(cold_ms, 4)
    result["breakdown"]["dominant_cold_cache_note"] = (
        f"{dom}, mean of {reps} launches each after a 512 MiB write; the timed steps run warm, "
        f"back to back")
    # side measurement: the whole step captured once as a HIP graph and
    # replayed, so no host work stands between launches (what launch-bound
    # shapes cost on the device alone); every output is preallocated
    side = torch.cuda.Stream(device=device)            # default priority
    side.wait_stream(torch.cuda.current_stream(device))
    with torch.cuda.stream(side):
        step.run()
    torch.cuda.current_stream(device).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step.run()
    graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    result["breakdown"]["graph_step_ms"] = round(a.elapsed_time(b) / args.steps, 4)
    result["breakdown"]["graph_step_note"] = (
        f"the step captured once as a HIP graph, {args.steps} replays back to back; value and ms_per_step "
        f"are the eager steps")
    del graph
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
    # side measurement: the reduce metric over the flat parameter vector
    step.metric_setup()
    for _ in range(2):
        step.metric()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        step.metric()
    b.record()
    torch.cuda.synchronize()
    m_ms = a.elapsed_time(b) / args.steps
    m_units = wl.pop * step.center.numel()
    result["breakdown"]["reduce_metric"] = {
        "n_params": step.center.numel(), "ms": round(m_ms, 4),
        "elements_per_s": m_units / (m_ms * 1e-3),
        "frac_of_hash_peak": round(m_units / (m_ms * 1e-3) / HASH_PEAK_PER_S, 4),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget_s)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
