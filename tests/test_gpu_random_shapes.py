"""A seeded sweep of random shapes through every entry point, against the
oracle: the hand-picked edge cases aim at known boundaries, this aims at the
combinations nobody thought of (population, rows, widths, dtype, shared x,
bias, offset, ragged everything).  Sizes stay small enough for the CPU oracle."""

import numpy as np
import pytest
import torch

import oracle
import virtual_noise_perturbed_amd as vn
import workloads
from gpu_util import TOL_BF16, TOL_F32, assert_close, sigma32, to_dev

pytestmark = pytest.mark.gpu


def _cases(n=30, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        batch = int(rng.choice([1, 2, 3, 4, int(rng.integers(5, 65)), int(rng.integers(65, 300)),
                                int(rng.integers(513, 700))], p=[.1, .08, .06, .06, .4, .2, .1]))
        pop = int(rng.integers(1, 41)) if batch < 300 else int(rng.integers(1, 4))
        fin = int(rng.integers(1, 700))
        fout = int(rng.integers(1, 600))
        dt = "bf16" if rng.random() < 0.4 else "f32"
        bias = bool(rng.random() < 0.6)
        shared = bool(rng.random() < 0.3)
        offset = int(rng.choice([0, int(rng.integers(1, 1 << 20)), int(rng.integers(1 << 32, 1 << 40))]))
        sigma = float(rng.choice([0.02, 0.3, 1.5]))
        out.append((pop, batch, fin, fout, dt, bias, shared, offset, sigma))
    return out


CASES = _cases()


def _id(c):
    return f"{c[4]}-p{c[0]}b{c[1]}i{c[2]}o{c[3]}{'-bias' if c[5] else ''}{'-shared' if c[6] else ''}-off{c[7]}"


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_random_shape(case):
    pop, batch, fin, fout, dt, bias, shared, offset, sigma = case
    print(f"random shape {_id(case)} sigma={sigma}", flush=True)
    wl = workloads.make_custom(pop, batch, fin, fout, dtype=dt, bias=bias, shared_x=shared, sigma=sigma,
                               offset=offset, seed=pop * 1000 + fin, seed_base=-7)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    L = wl.layers[0]
    sig = sigma32(wl.sigma)
    seeds = to_dev(wl.seeds)

    # forward, every output
    y = vn.virtual_perturbed_linear(to_dev(wl.x, tdt), to_dev(L.weight, tdt),
                                    None if L.bias is None else to_dev(L.bias), seeds, wl.sigma, offset)
    ref = oracle.perturbed_linear(wl.x, L.weight, L.bias, wl.seeds, sig, offset)
    assert_close(y.cpu().numpy(), ref, TOL_BF16 if dt == "bf16" else TOL_F32, "forward " + _id(case))

    # gradients of the whole parameter block in one launch (weights, then the bias region)
    n = fout * fin + (fout if bias else 0)
    fit = wl.fitness.astype(np.float32)
    g = vn.virtual_flat_gradient(to_dev(fit), seeds, n, wl.sigma, pop, offset).cpu().numpy()
    f64 = fit.astype(np.float64)
    want = oracle.weight_gradient(f64, wl.seeds, (fout, fin), sig, pop, offset).reshape(-1)
    if bias:
        want = np.concatenate([want, oracle.bias_gradient(f64, wl.seeds, (fout,), sig, pop, offset + fout * fin)])
    assert_close(g, want, TOL_F32, "gradient " + _id(case))

    # reduce metric over the same block, centred on the weights (and bias)
    center = np.concatenate([L.weight.astype(np.float32).reshape(-1)] +
                            ([L.bias.astype(np.float32)] if bias else []))
    m = vn.virtual_reduce_metric(to_dev(center), seeds, wl.sigma, n, offset).cpu().numpy()
    assert_close(m, oracle.reduce_metric(center, wl.seeds, sig, n, offset), TOL_F32, "metric " + _id(case))
