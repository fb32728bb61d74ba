"""The hot path under HIP graph capture.

Every entry point launches on the caller's current stream and allocates
nothing when its outputs are given, so a forward and a gradient can be
captured into one graph.  Replays, with eager work and synchronizations in
between and a new fitness vector written in place before one of them, must
give exactly what eager calls give (the same kernels in a fixed order)."""

import numpy as np
import pytest
import torch

import virtual_noise_perturbed_amd as vn
from gpu_util import device

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    print("graph capture: two-layer forward + flat gradient", flush=True)
    dev = device()
    g = torch.Generator().manual_seed(7)
    pop, batch, d0, d1, d2 = 24, 5, 70, 48, 10
    x = torch.randn(pop, batch, d0, generator=g).to(dev)
    w1 = (torch.randn(d1, d0, generator=g) / d0 ** 0.5).to(dev)
    b1 = torch.randn(d1, generator=g).to(dev)
    w2 = (torch.randn(d2, d1, generator=g) / d1 ** 0.5).to(dev)
    seeds = (torch.arange(pop) * 1009 - 5).to(dev)
    fit = torch.randn(pop, generator=g).to(dev)
    offs = vn.compute_offsets([(d1, d0), (d1,), (d2, d1)])
    n = offs[-1] + d2 * d1
    h = torch.empty(pop, batch, d1, device=dev)
    y = torch.empty(pop, batch, d2, device=dev)
    grad = torch.empty(n, device=dev)
    sigma = 0.05

    def step():
        vn.virtual_perturbed_linear(x, w1, b1, seeds, sigma, offs[0], activation="relu", out=h)
        vn.virtual_perturbed_linear(h, w2, None, seeds, sigma, offs[2], out=y)
        vn.virtual_flat_gradient(fit, seeds, n, sigma, pop, 0, out=grad)

    def eager():
        step()
        torch.cuda.synchronize()
        return h.clone(), y.clone(), grad.clone()

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    want = eager()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    new_fit = torch.randn(pop, generator=g).to(dev)
    for r in range(4):
        h.zero_(), y.zero_(), grad.zero_()
        if r == 2:                              # new inputs, written in place
            fit.copy_(new_fit)
            want = eager()
            h.zero_(), y.zero_(), grad.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _ = (torch.ones(1000, device=dev) * r).sum().item()    # eager work between replays
        for got, exp, name in zip((h, y, grad), want, ("hidden", "output", "gradient")):
            assert torch.equal(got, exp), f"replay {r}: {name}"
    assert not np.array_equal(want[2].cpu().numpy(), np.zeros(n, dtype=np.float32))


def test_graph_replays_match_eager_large_batch():
    """The large-batch bf16 forward (perturbed weights formed in a workspace the
    binding allocates, two groups of individuals, so four kernels per call) and
    the reduce metric, captured together: replays equal eager calls."""
    print("graph capture: materialized large-batch forward + reduce metric", flush=True)
    dev = device()
    g = torch.Generator().manual_seed(11)
    pop, batch, fin, fout = 9, 2048, 4096, 4096          # 8 individuals per 256 MiB group
    x = torch.randn(batch, fin, generator=g).to(torch.bfloat16).to(dev)
    w = (torch.randn(fout, fin, generator=g) / 64).to(torch.bfloat16).to(dev)
    b = torch.randn(fout, generator=g).to(dev)
    seeds = (torch.arange(pop) * 7919 + 3).to(dev)
    center = torch.randn(fout * fin, generator=g).to(dev)
    y = torch.empty(pop, batch, fout, device=dev)
    res = {}
    sigma = 0.01

    def step():
        vn.virtual_perturbed_linear(x, w, b, seeds, sigma, 17, out=y)
        res["met"] = vn.virtual_reduce_metric(center, seeds, sigma, fout * fin, 17)

    def eager():
        step()
        torch.cuda.synchronize()
        return y.clone(), res["met"].clone()

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    want = eager()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    met = res["met"]                            # the graph's own output of the metric
    for r in range(3):
        y.zero_(), met.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _ = (torch.ones(1000, device=dev) * r).sum().item()    # eager work between replays
        assert torch.equal(y, want[0]), f"replay {r}: output"
        assert torch.equal(met, want[1]), f"replay {r}: metric"
