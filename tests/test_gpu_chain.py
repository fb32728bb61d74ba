"""The fused chain of layers (vn_perturbed_mlp) against the oracle applied
layer after layer, with ReLU between layers as the 3-layer workload uses it."""

import numpy as np
import pytest
import torch

import oracle
import virtual_noise_perturbed_amd as vn
import workloads
from gpu_util import TOL_BF16, TOL_F32, assert_close, device, sigma32, to_dev

pytestmark = pytest.mark.gpu


def _oracle_chain(x, weights, biases, seeds, sig, offsets, relu, ids):
    """x: (batch, in) shared or (pop, batch, in); float64 chain over individuals ids."""
    h = np.asarray(x, dtype=np.float64)
    h = h if h.ndim == 2 else h[ids]
    for l, (w, b) in enumerate(zip(weights, biases)):
        h = oracle.perturbed_linear(h, w, b, seeds[ids], sig, offsets[l])
        if relu and l < len(weights) - 1:
            h = np.maximum(h, 0.0)
    return h


CASES = [
    # pop, batch, dims, dtype, biases, shared x, relu, offsets
    (3, 5, [40, 33, 7], "f32", [True, True], False, True, [0, 5000]),
    (2, 64, [256, 256, 10], "f32", [True, True], False, True, [200960, 266752]),
    (4, 1, [17, 256, 3, 9], "f32", [False, True, True], True, False, [7, 20000, 90000]),
    (2, 63, [100], "f32", [], False, True, []),                       # no layer: rejected below
    (3, 64, [64, 64], "bf16", [True], False, True, [11]),             # one layer = one linear call
    (2, 37, [250, 129, 255, 32], "bf16", [True, False, True], True, True, [0, 2**33, 2**34]),
    (5, 16, [8, 8, 8, 8, 8, 8, 8, 8, 8], "f32", [True] * 8, False, True, [1000 * k for k in range(8)]),
    # wide first layers (streamed input): the 3-layer workload's shape, ragged widths, unaligned rows
    (3, 64, [784, 256, 256, 10], "f32", [True, True, True], False, True, [0, 200960, 266752]),
    (2, 33, [1000, 100, 7], "bf16", [True, True], False, True, [5, 10**6]),
    (3, 20, [301, 256, 40], "f32", [False, True], True, True, [0, 77101]),
    (2, 64, [4096, 64], "bf16", [True], True, False, [3]),
    (2, 7, [33, 31, 1], "f32", [True, True], False, False, [0, 9]),
]


@pytest.mark.parametrize("case", [c for c in CASES if len(c[2]) > 1],
                         ids=[f"{c[3]}-p{c[0]}b{c[1]}-{'x'.join(map(str, c[2]))}" for c in CASES if len(c[2]) > 1])
def test_chain_matches_oracle(case):
    _check_chain(case)


def _random_chain_cases(n=16, seed=7):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        n_layers = int(rng.integers(2, 5))
        dims = [int(rng.integers(1, 900))] + [int(rng.integers(1, 257)) for _ in range(n_layers)]
        out.append((int(rng.integers(1, 9)), int(rng.integers(1, 65)), dims,
                    "bf16" if rng.random() < 0.4 else "f32", [bool(rng.random() < 0.7) for _ in range(n_layers)],
                    bool(rng.random() < 0.3), bool(rng.random() < 0.7),
                    [int(rng.integers(0, 1 << 36)) for _ in range(n_layers)]))
    return out


RANDOM_CASES = _random_chain_cases()


@pytest.mark.parametrize("case", RANDOM_CASES,
                         ids=[f"{c[3]}-p{c[0]}b{c[1]}-{'x'.join(map(str, c[2]))}" for c in RANDOM_CASES])
def test_random_chain_matches_oracle(case):
    """Seeded random chains: widths, depth, rows, dtype, biases, shared x, ReLU, offsets."""
    _check_chain(case)


def _check_chain(case):
    pop, batch, dims, dt, has_b, shared, relu, offsets = case
    print(f"chain {case}", flush=True)
    rng = np.random.default_rng(sum(dims) + batch)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    rb = workloads.round_to_bf16 if dt == "bf16" else (lambda a: a)
    xshape = (batch, dims[0]) if shared else (pop, batch, dims[0])
    x = rb(rng.uniform(-1.0, 1.0, size=xshape).astype(np.float32))
    weights = [rb((rng.standard_normal((o, i)) / np.sqrt(i)).astype(np.float32)) for i, o in zip(dims[:-1], dims[1:])]
    biases = [(0.1 * rng.standard_normal(o)).astype(np.float32) if hb else None for o, hb in zip(dims[1:], has_b)]
    seeds = np.arange(pop, dtype=np.int64) * 17 - 3
    sigma = 0.05
    y = vn.virtual_perturbed_mlp(to_dev(x, tdt), [to_dev(w, tdt) for w in weights],
                                 [None if b is None else to_dev(b) for b in biases], to_dev(seeds), sigma, offsets,
                                 activation="relu" if relu else None).cpu().numpy()
    assert y.shape == (pop, batch, dims[-1])
    if dt == "bf16":
        # the chain rounds intermediate activations to bf16, as a caller feeding bf16 layers does
        h = np.asarray(x, dtype=np.float64)
        h = h if h.ndim == 2 else h
        for l, (w, b) in enumerate(zip(weights, biases)):
            h = oracle.perturbed_linear(h, w, b, seeds, sigma32(sigma), offsets[l])
            if relu and l < len(weights) - 1:
                h = np.maximum(h, 0.0)
            if l < len(weights) - 1:
                h = workloads.round_to_bf16(h.astype(np.float32)).astype(np.float64)
        ref = h
        tol = TOL_BF16
    else:
        ref = _oracle_chain(x, weights, biases, seeds, sigma32(sigma), offsets, relu, np.arange(pop))
        tol = TOL_F32
    assert_close(y, ref, tol, str(case))


def test_chain_one_layer_equals_linear():
    """n_layers = 1 is the perturbed linear layer."""
    pop, batch, fin, fout = 3, 40, 96, 50
    rng = np.random.default_rng(3)
    x = to_dev(rng.standard_normal((pop, batch, fin)).astype(np.float32))
    w = to_dev((rng.standard_normal((fout, fin)) / 10).astype(np.float32))
    b = to_dev(rng.standard_normal(fout).astype(np.float32))
    s = to_dev(np.array([4, 5, 6], dtype=np.int64))
    y1 = vn.virtual_perturbed_mlp(x, [w], [b], s, 0.1, [77])
    y2 = vn.virtual_perturbed_linear(x, w, b, s, 0.1, 77)
    assert_close(y1.cpu().numpy(), y2.cpu().numpy().astype(np.float64), TOL_F32, "one layer")


@pytest.mark.parametrize("split", [0, 1])
def test_three_layer_workload(split):
    """The 3-layer workload: all three layers in one chain (split 0) or layer 1
    through the linear entry point and layers 2-3 through the chain (split 1),
    sampled individuals against the oracle chain."""
    print(f"workload 4, chain from layer {split}", flush=True)
    wl = workloads.make(4)
    sig = sigma32(wl.sigma)
    L = wl.layers
    s = to_dev(wl.seeds)
    h = to_dev(wl.x)
    if split:
        h = vn.virtual_perturbed_linear(h, to_dev(L[0].weight), to_dev(L[0].bias), s, wl.sigma, L[0].w_offset,
                                        activation="relu")
    y = vn.virtual_perturbed_mlp(h, [to_dev(Ly.weight) for Ly in L[split:]], [to_dev(Ly.bias) for Ly in L[split:]],
                                 s, wl.sigma, [Ly.w_offset for Ly in L[split:]], activation="relu")
    torch.cuda.synchronize()
    ids = [0, 17, 255, 511]
    h = wl.x[ids].astype(np.float64)
    for li, Ly in enumerate(L):
        h = oracle.perturbed_linear(h, Ly.weight, Ly.bias, wl.seeds[ids], sig, Ly.w_offset)
        if li < 2:
            h = np.maximum(h, 0.0)
    assert_close(y[ids].cpu().numpy(), h, TOL_F32, f"3-layer, chain from layer {split}")


def test_chain_repeat_bit_identical():
    wl = workloads.make(4)
    L = wl.layers
    rng = np.random.default_rng(9)
    h1 = to_dev(rng.uniform(0, 1, size=(wl.pop, wl.batch, 256)).astype(np.float32))
    args = ([to_dev(L[1].weight), to_dev(L[2].weight)], [to_dev(L[1].bias), to_dev(L[2].bias)], to_dev(wl.seeds),
            wl.sigma, [L[1].w_offset, L[2].w_offset])
    a = vn.virtual_perturbed_mlp(h1, *args)
    b = vn.virtual_perturbed_mlp(h1, *args)
    assert torch.equal(a, b)
    x = to_dev(wl.x)
    full = ([to_dev(Ly.weight) for Ly in L], [to_dev(Ly.bias) for Ly in L], to_dev(wl.seeds), wl.sigma,
            [Ly.w_offset for Ly in L])
    assert torch.equal(vn.virtual_perturbed_mlp(x, *full), vn.virtual_perturbed_mlp(x, *full))
