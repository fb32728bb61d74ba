"""The allocation-free reduce metric (vn_reduce_metric_noalloc) against the
entry point that takes a caller workspace (vn_reduce_metric): the same kernels
in the same summation order, so the means must agree bit for bit; both are
also held to the fp32 bar against the oracle.  Two calls in a row, the second
on a smaller input, so that partial sums a first call left in the GPU's fixed
array cannot leak into the second."""

import numpy as np
import pytest
import torch

import oracle
import virtual_noise_perturbed_amd as vn
from gpu_util import TOL_F32, assert_close, device, sigma32, to_dev

pytestmark = pytest.mark.gpu


def _case(pop, n, offset, seed):
    rng = np.random.default_rng(seed)
    center = rng.standard_normal(n).astype(np.float32)
    seeds = (np.arange(pop, dtype=np.int64) * 7919 - 13) * (1 if seed % 2 else -1)
    return center, seeds, offset


@pytest.mark.parametrize("first,second", [
    ((300, 1 << 21, 5), (3, 200_003, 77)),      # 300 x 4 segments, then 3 x 3 segments
    ((7, 1_000_003, 0), (2, 131_075, 2**33)),   # 7 x 15 segments, then 2 x 2 segments
])
def test_noalloc_matches_workspace_entry_point(first, second):
    dev = device()
    sig = 0.25
    for k, (pop, n, offset) in enumerate((first, second)):
        print(f"no-alloc reduce metric call {k}: pop={pop} n={n} offset={offset}", flush=True)
        center, seeds, offset = _case(pop, n, offset, seed=pop + n)
        c, s = to_dev(center), to_dev(seeds)
        out = torch.full((pop,), float("nan"), dtype=torch.float32, device=dev)
        got = vn.virtual_reduce_metric_noalloc(c, s, sig, n, offset, out=out)
        ref = vn.virtual_reduce_metric(c, s, sig, n, offset)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got, ref), f"call {k}: not bit-identical to vn_reduce_metric"
        want = oracle.reduce_metric(center, seeds, sigma32(sig), n, offset)
        assert_close(got.cpu().numpy(), want, TOL_F32, f"call {k} against the oracle")


def test_noalloc_without_partial_sums():
    """A population of 512 or more needs no partial sums: the array is not used."""
    dev = device()
    center, seeds, offset = _case(512, 4099, 3, seed=11)
    c, s = to_dev(center), to_dev(seeds)
    got = vn.virtual_reduce_metric_noalloc(c, s, 0.5, 4099, offset)
    ref = vn.virtual_reduce_metric(c, s, 0.5, 4099, offset)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


def test_noalloc_under_graph_capture():
    """The callers it is for: a graph captured around the allocation-free call
    (output given, so the call allocates nothing) replays to the bits of the
    workspace entry point, with other calls on the same GPU in between that use
    the fixed array for a different shape."""
    dev = device()
    pop, n, offset = 5, 600_001, 9
    print(f"no-alloc reduce metric under graph capture: pop={pop} n={n}", flush=True)
    center, seeds, _ = _case(pop, n, offset, seed=21)
    c, s = to_dev(center), to_dev(seeds)
    out = torch.empty((pop,), dtype=torch.float32, device=dev)
    ref = vn.virtual_reduce_metric(c, s, 0.125, n, offset)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):                 # warm-up off the capture stream
        vn.virtual_reduce_metric_noalloc(c, s, 0.125, n, offset, out=out)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        vn.virtual_reduce_metric_noalloc(c, s, 0.125, n, offset, out=out)
    c2, s2 = to_dev(_case(3, 70_001, 0, seed=4)[0]), to_dev(_case(3, 70_001, 0, seed=4)[1])
    for r in range(3):
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {r}"
        vn.virtual_reduce_metric_noalloc(c2, s2, 0.5, 70_001, 0)   # another shape through the array
        torch.cuda.synchronize()
