"""Ragged shapes, every kernel variant, degenerate sizes and the reduce metric,
each against the full CPU oracle."""

import numpy as np
import pytest
import torch

import oracle
import virtual_noise_perturbed_amd as vn
import workloads
from gpu_util import TOL_BF16, TOL_F32, assert_close, device, sigma32, to_dev

pytestmark = pytest.mark.gpu

# (pop, batch, in, out, dtype, bias, shared_x, offset)
CASES = [
    (3, 5, 13, 10, "f32", True, False, 0),          # in not a multiple of 4: scalar loads
    (7, 33, 784, 10, "f32", True, False, 200960),   # rows 33 -> two 32-row blocks, out 10
    (5, 1, 7, 300, "f32", False, False, 3),         # batch 1, in below one k-chunk
    (2, 300, 70, 40, "f32", True, False, 11),       # batch > 256: two row tiles
    (4, 64, 256, 256, "f32", True, True, 2**40),    # shared x, huge offset
    (6, 100, 96, 129, "f32", True, False, 5),       # 128-row variant, ragged out
    (3, 200, 64, 65, "f32", False, False, 0),       # 256-row variant
    (2, 16, 100, 300, "f32", True, False, 8),       # 16-row variant with k tail (100 = 64 + 36)
    (3, 3, 130, 20, "bf16", True, True, 2),         # 16-row bf16 variant with k tail
    (3, 5, 24, 10, "bf16", True, False, 0),
    (4, 32, 136, 70, "bf16", False, False, 9),
    (2, 64, 1000, 33, "bf16", True, True, 1 << 33),
    (3, 130, 72, 50, "bf16", True, False, 4),
    (2, 260, 48, 20, "bf16", False, False, 1),
    # narrow outputs: 16-wide column tiles, waves past `out` idle
    (4, 64, 256, 10, "f32", True, False, 266752),   # the 256->10 layer shape
    (3, 50, 100, 16, "bf16", True, False, 6),       # out exactly one 16-wide block, k tail
    (3, 40, 64, 17, "f32", False, False, 0),        # one past a 16-wide block
    (2, 64, 96, 128, "bf16", True, True, 12),       # single-column-block tile, full width
    (2, 60, 72, 129, "f32", True, False, 3),        # two-block tile, second tile mostly idle
    (5, 20, 40, 3, "f32", True, False, 1),          # 32-row tile, out 3
    # 17..32 rows on wide layers: 8-wave workgroups over 256 columns
    (3, 32, 200, 300, "f32", True, False, 5),       # second 256-column tile mostly idle, k tail
    (2, 17, 1000, 129, "bf16", True, False, 2**20), # one row past a 16-row tile, k tail
    (3, 24, 64, 257, "f32", False, True, 2**35),    # shared x, one column past a 256 tile
    (11, 32, 64, 1100, "f32", True, False, 3),      # 5 column tiles, 11 individuals: a last group of 3
    (9, 60, 40, 700, "bf16", False, False, 1),      # 3 column tiles, 9 individuals: a last group of 1
    # one or two fp32 rows: the vector-ALU kernel
    (3, 2, 100, 70, "f32", True, False, 4),         # k tail within a chunk, ragged columns
    (2, 2, 1024, 513, "f32", False, True, 2**36),   # shared x, one column past a tile
    (4, 1, 130, 17, "f32", True, False, 0),         # two chunks, the second partial
    (2, 1, 6, 3, "f32", False, False, 1),           # in not a multiple of 4: element loads
    (3, 3, 260, 140, "f32", True, False, 7),        # three rows
    (2, 4, 64, 200, "f32", False, True, 0),         # four rows, shared x
    # large batches: 512-row workgroups sharing one generated weight tile
    (2, 600, 200, 300, "f32", True, False, 3),      # two row tiles, ragged column tile
    (3, 1030, 136, 130, "bf16", True, True, 2**34), # three row tiles, shared x
    (1, 513, 16, 128, "f32", False, False, 0),      # one k-chunk, one row past a tile
    (2, 700, 17, 5, "f32", True, False, 8),         # in not a multiple of 4: element loads
    (2, 300, 1000, 260, "bf16", False, True, 5),    # dead waves in the row tile
    (2, 520, 300, 100, "bf16", True, False, 17),    # own x; 7 of 8 waves past the batch in tile 2
]


CASES_EXACT = [c for c in CASES if c[4] == "f32"]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[4]}-p{c[0]}b{c[1]}i{c[2]}o{c[3]}{'-shared' if c[6] else ''}"
                                             for c in CASES])
def test_ragged_forward(case):
    _ragged(case, "default")


@pytest.mark.parametrize("case", CASES_EXACT, ids=[f"exact-p{c[0]}b{c[1]}i{c[2]}o{c[3]}" for c in CASES_EXACT])
def test_ragged_forward_exact_f32(case):
    _ragged(case, "f32")


def _ragged(case, math):
    pop, batch, fin, fout, dt, bias, shared, offset = case
    print(f"ragged forward {case} math={math}", flush=True)
    wl = workloads.make_custom(pop, batch, fin, fout, dtype=dt, bias=bias, shared_x=shared, sigma=0.05,
                               offset=offset, seed=fin + fout, seed_base=-2)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    L = wl.layers[0]
    y = vn.virtual_perturbed_linear(to_dev(wl.x, tdt), to_dev(L.weight, tdt),
                                    None if L.bias is None else to_dev(L.bias), to_dev(wl.seeds),
                                    wl.sigma, offset, math=math).cpu().numpy()
    ref = oracle.perturbed_linear(wl.x, L.weight, L.bias, wl.seeds, sigma32(wl.sigma), offset)
    assert_close(y, ref, TOL_BF16 if dt == "bf16" else TOL_F32, str(case))


def test_misaligned_base_pointer_path():
    """in a multiple of 4 but x not 16-byte aligned: the kernel takes element loads."""
    dev = device()
    pop, batch, fin, fout = 3, 8, 32, 24
    wl = workloads.make_custom(pop, batch, fin, fout, seed=3)
    L = wl.layers[0]
    buf = torch.empty(pop * batch * fin + 1, device=dev)
    x = buf[1:].view(pop, batch, fin)
    x.copy_(to_dev(wl.x))
    assert x.data_ptr() % 16 != 0
    y = vn.virtual_perturbed_linear(x, to_dev(L.weight), to_dev(L.bias), to_dev(wl.seeds), wl.sigma, 0)
    ref = oracle.perturbed_linear(wl.x, L.weight, L.bias, wl.seeds, sigma32(wl.sigma), 0)
    assert_close(y.cpu().numpy(), ref, TOL_F32, "misaligned x")


def test_relu_int32_seeds():
    pop, batch, fin, fout = 5, 20, 40, 30
    wl = workloads.make_custom(pop, batch, fin, fout, seed=9, seed_base=-100)
    L = wl.layers[0]
    s32 = to_dev(wl.seeds.astype(np.int32))
    y = vn.virtual_perturbed_linear(to_dev(wl.x), to_dev(L.weight), to_dev(L.bias), s32, wl.sigma, 17,
                                    activation="relu").cpu().numpy()
    ref = np.maximum(oracle.perturbed_linear(wl.x, L.weight, L.bias, wl.seeds, sigma32(wl.sigma), 17), 0)
    assert_close(y, ref, TOL_F32, "relu / int32 seeds")
    assert (y >= 0).all()


def test_sigma_zero_is_plain_linear():
    pop, batch, fin, fout = 4, 9, 50, 20
    wl = workloads.make_custom(pop, batch, fin, fout, seed=10)
    L = wl.layers[0]
    y = vn.virtual_perturbed_linear(to_dev(wl.x), to_dev(L.weight), to_dev(L.bias), to_dev(wl.seeds), 0.0, 0)
    ref = np.einsum("pbk,jk->pbj", wl.x.astype(np.float64), L.weight.astype(np.float64)) + L.bias
    assert_close(y.cpu().numpy(), ref, TOL_F32, "sigma 0")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_negative_sigma(dt):
    """sigma < 0 is a valid perturbation scale: the forward adds sigma * N, the
    gradients divide by P * sigma (a negative scale) and the reduce metric
    takes |c + sigma * N|; everything against the oracle at sigma = -0.3."""
    print(f"negative sigma {dt}", flush=True)
    pop, batch, fin, fout, offset = 5, 40, 96, 70, 11
    wl = workloads.make_custom(pop, batch, fin, fout, dtype=dt, bias=True, sigma=-0.3, offset=offset, seed=31)
    L = wl.layers[0]
    tol = TOL_BF16 if dt == "bf16" else TOL_F32
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    sig = sigma32(wl.sigma)
    seeds = to_dev(wl.seeds)
    y = vn.virtual_perturbed_linear(to_dev(wl.x, tdt), to_dev(L.weight, tdt), to_dev(L.bias), seeds, wl.sigma,
                                    offset).cpu().numpy()
    assert_close(y, oracle.perturbed_linear(wl.x, L.weight, L.bias, wl.seeds, sig, offset), tol, "forward")
    fit = to_dev(wl.fitness)
    f64 = wl.fitness.astype(np.float64)
    gw = vn.virtual_weight_gradient(fit, seeds, (fout, fin), wl.sigma, pop, offset).cpu().numpy()
    assert_close(gw, oracle.weight_gradient(f64, wl.seeds, (fout, fin), sig, pop, offset), TOL_F32, "grad W")
    gb = vn.virtual_bias_gradient(fit, seeds, (fout,), wl.sigma, pop, offset + fout * fin).cpu().numpy()
    assert_close(gb, oracle.bias_gradient(f64, wl.seeds, (fout,), sig, pop, offset + fout * fin), TOL_F32, "grad b")
    center = np.random.default_rng(3).standard_normal(5000).astype(np.float32)
    m = vn.virtual_reduce_metric(to_dev(center), seeds, wl.sigma, 5000, offset).cpu().numpy()
    assert_close(m, oracle.reduce_metric(center, wl.seeds, sig, 5000, offset), TOL_F32, "reduce metric")


def test_degenerate_sizes():
    dev = device()
    s = to_dev(np.arange(3, dtype=np.int64))
    # in = 0: only the bias term remains (b + sigma nb)
    b = torch.ones(5, device=dev)
    y = vn.virtual_perturbed_linear(torch.empty((3, 2, 0), device=dev), torch.empty((5, 0), device=dev), b,
                                    s, 0.5, 7).cpu().numpy()
    nb = oracle.noise(np.arange(3), 5, 7)
    assert_close(y, np.broadcast_to((1 + np.float64(np.float32(0.5)) * nb)[:, None, :], (3, 2, 5)), TOL_F32, "in=0")
    # empty population / batch / out
    assert vn.virtual_perturbed_linear(torch.zeros((0, 2, 4), device=dev), torch.zeros((3, 4), device=dev), None,
                                       torch.zeros(0, dtype=torch.int64, device=dev), 0.1, 0).shape == (0, 2, 3)
    assert vn.virtual_perturbed_linear(torch.zeros((0, 4), device=dev), torch.zeros((3, 4), device=dev), None,
                                       s, 0.1, 0).shape == (3, 0, 3)
    assert vn.virtual_perturbed_linear(torch.zeros((2, 4), device=dev), torch.zeros((0, 4), device=dev), None,
                                       s, 0.1, 0).shape == (3, 2, 0)
    f = torch.ones(3, device=dev)
    assert vn.virtual_weight_gradient(f, s, (0, 4), 0.1, 3, 0).shape == (0, 4)
    # pop 1, one element
    g = vn.virtual_flat_gradient(torch.tensor([2.0], device=dev), s[:1], 1, 0.25, 1, 123).cpu().numpy()
    assert_close(g, oracle.weight_gradient_at(np.array([2.0]), np.array([0]), 0.25, 1, 123, [0]), TOL_F32, "1x1")


# The last three split the population over 16 waves per workgroup (few
# workgroups, long parts of the population): one element per lane with a
# population that 16 does not divide, four per lane, and four per lane at the
# largest element count that still takes the split.
@pytest.mark.parametrize("pop,n", [(1, 5), (63, 1000), (64, 16384), (65, 16385), (1000, 3000), (3, 70001),
                                   (4099, 17385), (1030, 2**20 + 100), (1024, 2**21 - 300)])
def test_gradient_shapes(pop, n):
    print(f"gradient pop={pop} n={n}", flush=True)
    rng = np.random.default_rng(pop + n)
    seeds = rng.integers(-2**62, 2**62, size=pop)
    fit = rng.standard_normal(pop).astype(np.float32)
    sig = 0.03
    g = vn.virtual_flat_gradient(to_dev(fit), to_dev(seeds), n, sig, pop, 999).cpu().numpy()
    idx = np.unique(np.concatenate([np.arange(min(n, 50)), n - 1 - np.arange(min(n, 50)), rng.integers(0, n, 500)]))
    ref = oracle.weight_gradient_at(fit.astype(np.float64), seeds, sigma32(sig), pop, 999, idx)
    assert_close(g[idx], ref, TOL_F32, f"pop {pop} n {n}")


def test_binding_checks_pop_size():
    dev = device()
    s = to_dev(np.arange(4, dtype=np.int64))
    with pytest.raises(ValueError):
        vn.virtual_weight_gradient(torch.ones(4, device=dev), s, (2, 3), 0.1, 5, 0)
    with pytest.raises(ValueError):
        vn.virtual_weight_gradient(torch.ones(4, device=dev), s, (2, 3), 0.0, 4, 0)


@pytest.mark.parametrize("pop,n,offset", [(6, 1000, 0), (3, 269322, 5), (1, 1, 2**35), (40, 4097, 77), (2, 3, 9),
                                          (5, 4096 * 3 + 2, 1), (300, 2051, 13), (1, (1 << 20) + 3, 3),
                                          (200, 140000, 0), (511, 131076, 2), (512, 131076, 2)])
def test_reduce_metric(pop, n, offset):
    # (511, 131076): the largest population that still splits (two segments);
    # (512, 131076): the smallest that takes one workgroup per individual
    print(f"reduce metric pop={pop} n={n}", flush=True)
    rng = np.random.default_rng(n)
    center = rng.standard_normal(n).astype(np.float32)
    seeds = np.arange(pop, dtype=np.int64) * 31 - 7
    sig = 0.3
    got = vn.virtual_reduce_metric(to_dev(center), to_dev(seeds), sig, n, offset).cpu().numpy()
    ref = oracle.reduce_metric(center, seeds, sigma32(sig), n, offset)
    assert_close(got, ref, TOL_F32, "reduce metric")


def test_reduce_metric_repeat_bit_identical():
    """Segmented (small population, long vector): partial sums in a fixed order."""
    pop, n = 3, 600001
    center = to_dev(np.random.default_rng(1).standard_normal(n).astype(np.float32))
    seeds = to_dev(np.array([4, 5, 6], dtype=np.int64))
    a = vn.virtual_reduce_metric(center, seeds, 0.1, n, 7)
    b = vn.virtual_reduce_metric(center, seeds, 0.1, n, 7)
    assert torch.equal(a, b)


@pytest.mark.parametrize("sig", [0.3, 2.0 ** -101])
def test_reduce_metric_unaligned_center_and_tiny_sigma(sig):
    """center starting one float past a 16-byte boundary takes the scalar loads;
    sigma below 2^-100 takes the kernel that forms sigma * N directly."""
    pop, n, offset = 4, 300003, 21
    rng = np.random.default_rng(5)
    center = rng.standard_normal(n + 1).astype(np.float32)
    seeds = np.arange(pop, dtype=np.int64) + 100
    buf = to_dev(center)
    got = vn.virtual_reduce_metric(buf[1:], to_dev(seeds), sig, n, offset).cpu().numpy()
    ref = oracle.reduce_metric(center[1:], seeds, sigma32(sig), n, offset)
    assert_close(got, ref, TOL_F32, "reduce metric")
