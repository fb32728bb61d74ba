"""Calls from several host threads, each on a stream of its own.

The library keeps no state across calls (only a per-thread error string), and
every entry point is asynchronous on the stream it is given, so concurrent
calls on different streams must give exactly what the same calls give one
after another on the default stream (every kernel sums in a fixed order).
"""

import threading

import pytest
import torch

import virtual_noise_perturbed_amd as vn
from gpu_util import device

pytestmark = pytest.mark.gpu


def _problem(k: int, dev):
    g = torch.Generator().manual_seed(100 + k)
    pop, batch, fin, fout = 16 + 8 * k, 24 + 40 * k, 200 + 56 * k, 96 + 64 * k
    dt = torch.bfloat16 if k % 2 else torch.float32
    x = torch.randn(pop, batch, fin, generator=g).to(dt).to(dev)
    w = (torch.randn(fout, fin, generator=g) / fin ** 0.5).to(dt).to(dev)
    b = torch.randn(fout, generator=g).to(dev)
    seeds = torch.arange(pop, device=dev) * 3 + k
    fit = torch.randn(pop, generator=g).to(dev)
    center = torch.randn(fout * fin + fout, generator=g).to(dev)
    return x, w, b, seeds, fit, center


def _run(prob, sigma=0.03):
    x, w, b, seeds, fit, center = prob
    pop = seeds.numel()
    y = vn.virtual_perturbed_linear(x, w, b, seeds, sigma, 7)
    gw = vn.virtual_weight_gradient(fit, seeds, w.shape, sigma, pop, 7)
    gb = vn.virtual_bias_gradient(fit, seeds, b.shape, sigma, pop, 7 + w.numel())
    m = vn.virtual_reduce_metric(center, seeds, sigma, center.numel(), 7)
    return y, gw, gb, m


def test_threads_on_own_streams_match_sequential():
    print("two host threads, one stream each", flush=True)
    dev = device()
    probs = [_problem(k, dev) for k in range(2)]
    ref = [_run(p) for p in probs]
    torch.cuda.synchronize()

    reps = 6
    results = [[None] * reps for _ in probs]
    errors = []

    def worker(k):
        try:
            stream = torch.cuda.Stream(device=dev)   # default priority
            with torch.cuda.stream(stream):
                for r in range(reps):
                    results[k][r] = _run(probs[k])
            stream.synchronize()
        except Exception as exc:  # reported in the main thread
            errors.append(exc)

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(len(probs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for k in range(len(probs)):
        for r in range(reps):
            for got, want in zip(results[k][r], ref[k]):
                assert torch.equal(got, want), f"problem {k} repeat {r}"
