"""The HIP path against the CPU oracle on the five synthetic workloads, at
their full sizes and in the launch configuration the bench times.

Small workloads are checked element by element against the full oracle.
Large ones are checked on whole individuals (every output of a few
individuals, first/middle/last) plus random output elements spread over all
individuals, and on sampled gradient elements including the first and last
rows; the oracle evaluates exactly those elements.
"""

import numpy as np
import pytest
import torch

import oracle
import virtual_noise_perturbed_amd as vn
import workloads
from gpu_util import TOL_BF16, TOL_F32, assert_close, device, sigma32, to_dev

pytestmark = pytest.mark.gpu


def _dev_inputs(wl):
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    x = to_dev(wl.x, dt)
    layers = []
    for L in wl.layers:
        layers.append((to_dev(L.weight, dt), None if L.bias is None else to_dev(L.bias)))
    return x, layers, to_dev(wl.seeds), to_dev(wl.fitness)


def _pick_individuals(pop, k=3):
    return sorted(set([0, pop // 2, pop - 1][:k]))


def _sample_outputs(rng, pop, batch, out, n):
    return rng.integers(0, pop, n), rng.integers(0, batch, n), rng.integers(0, out, n)


def _sample_flat(rng, n_el, fin, n):
    idx = np.concatenate([np.arange(min(64, n_el)), n_el - 1 - np.arange(min(64, n_el)),
                          rng.integers(0, n_el, n)])
    if fin:
        idx = np.concatenate([idx, np.arange(fin) + (n_el // fin // 2) * fin])  # a whole middle row
    return np.unique(idx)


@pytest.mark.parametrize("key", [1, 2, 3, 5, 6])
def test_single_layer_forward(key):
    print(f"workload {key} forward", flush=True)
    wl = workloads.make(key)
    tol = TOL_BF16 if wl.dtype == "bf16" else TOL_F32
    L = wl.layers[0]
    sig = sigma32(wl.sigma)
    x, layers, seeds, _ = _dev_inputs(wl)
    w, b = layers[0]
    y = vn.virtual_perturbed_linear(x, w, b, seeds, wl.sigma, L.w_offset)
    torch.cuda.synchronize()
    assert y.shape == (wl.pop, wl.batch, L.out_features)
    ids = list(range(wl.pop)) if wl.pop <= 8 else _pick_individuals(wl.pop)
    shared = wl.x.ndim == 2
    # whole rows (every output column) of a few individuals; all rows unless
    # the batch is large, then the first, middle and last rows of both row
    # tiles they fall in
    rows = np.arange(wl.batch) if wl.batch <= 256 else np.array([0, 1, 511, 512, wl.batch // 2, wl.batch - 1])
    xs = wl.x[rows] if shared else wl.x[ids][:, rows]
    ref = oracle.perturbed_linear(xs, L.weight, L.bias, wl.seeds[ids], sig, L.w_offset)
    got = y[ids][:, torch.as_tensor(rows)].cpu().numpy()
    assert_close(got, ref, tol, f"workload {key} whole rows of individuals {ids}")
    rng = np.random.default_rng(key)
    ii, bb, jj = _sample_outputs(rng, wl.pop, wl.batch, L.out_features, 400)
    ref_s = oracle.perturbed_linear_at(wl.x, L.weight, L.bias, wl.seeds, sig, L.w_offset, ii, bb, jj)
    got_s = y[torch.as_tensor(ii), torch.as_tensor(bb), torch.as_tensor(jj)].cpu().numpy()
    assert_close(got_s, ref_s, tol, f"workload {key} sampled outputs")


@pytest.mark.parametrize("key", [1, 2, 3, 5, 6])
def test_single_layer_gradients(key):
    print(f"workload {key} gradients", flush=True)
    wl = workloads.make(key)
    L = wl.layers[0]
    sig = sigma32(wl.sigma)
    _, _, seeds, fit = _dev_inputs(wl)
    fit64 = wl.fitness.astype(np.float64)
    gw = vn.virtual_weight_gradient(fit, seeds, (L.out_features, L.in_features), wl.sigma, wl.pop,
                                    L.w_offset).cpu().numpy()
    n_el = L.out_features * L.in_features
    if n_el * wl.pop <= 4_000_000:
        ref = oracle.weight_gradient(fit64, wl.seeds, (L.out_features, L.in_features), sig, wl.pop, L.w_offset)
        assert_close(gw, ref, TOL_F32, f"workload {key} grad_W (full)")
    else:
        idx = _sample_flat(np.random.default_rng(100 + key), n_el, L.in_features, 3000)
        ref = oracle.weight_gradient_at(fit64, wl.seeds, sig, wl.pop, L.w_offset, idx)
        assert_close(gw.reshape(-1)[idx], ref, TOL_F32, f"workload {key} grad_W (sampled)")
    if L.bias is not None:
        gb = vn.virtual_bias_gradient(fit, seeds, (L.out_features,), wl.sigma, wl.pop, L.b_offset).cpu().numpy()
        refb = oracle.bias_gradient(fit64, wl.seeds, (L.out_features,), sig, wl.pop, L.b_offset)
        assert_close(gb, refb, TOL_F32, f"workload {key} grad_b")


def test_three_layer_chain():
    """784->256->256->10 with ReLU between layers, blocks chained by flat offsets."""
    print("workload 4 forward chain", flush=True)
    wl = workloads.make(4)
    sig = sigma32(wl.sigma)
    x, layers, seeds, _ = _dev_inputs(wl)
    assert [L.w_offset for L in wl.layers] == [0, 200960, 266752]
    assert vn.compute_offsets(wl.shapes) == [0, 200704, 200960, 266496, 266752, 269312]
    h = x
    outs = []
    for li, (L, (w, b)) in enumerate(zip(wl.layers, layers)):
        act = "relu" if li < len(wl.layers) - 1 else None
        h = vn.virtual_perturbed_linear(h, w, b, seeds, wl.sigma, L.w_offset, activation=act)
        outs.append(h)
    torch.cuda.synchronize()
    ids = _pick_individuals(wl.pop) + [17]
    h_ref = wl.x[ids].astype(np.float64)
    for li, L in enumerate(wl.layers):
        h_ref = oracle.perturbed_linear(h_ref, L.weight, L.bias, wl.seeds[ids], sig, L.w_offset)
        if li < len(wl.layers) - 1:
            h_ref = np.maximum(h_ref, 0.0)
        assert_close(outs[li][ids].cpu().numpy(), h_ref, TOL_F32, f"layer {li + 1}")


def test_three_layer_gradients():
    print("workload 4 gradients", flush=True)
    wl = workloads.make(4)
    sig = sigma32(wl.sigma)
    _, _, seeds, fit = _dev_inputs(wl)
    fit64 = wl.fitness.astype(np.float64)
    rng = np.random.default_rng(44)
    for L in wl.layers:
        gw = vn.virtual_weight_gradient(fit, seeds, (L.out_features, L.in_features), wl.sigma, wl.pop,
                                        L.w_offset).cpu().numpy()
        n_el = L.out_features * L.in_features
        idx = _sample_flat(rng, n_el, L.in_features, 1500)
        ref = oracle.weight_gradient_at(fit64, wl.seeds, sig, wl.pop, L.w_offset, idx)
        assert_close(gw.reshape(-1)[idx], ref, TOL_F32, f"grad_W at {L.w_offset}")
        gb = vn.virtual_bias_gradient(fit, seeds, (L.out_features,), wl.sigma, wl.pop, L.b_offset).cpu().numpy()
        refb = oracle.bias_gradient(fit64, wl.seeds, (L.out_features,), sig, wl.pop, L.b_offset)
        assert_close(gb, refb, TOL_F32, f"grad_b at {L.b_offset}")
    # the whole chained parameter vector in one launch equals the per-block results
    total = wl.total_params
    flat = vn.virtual_flat_gradient(fit, seeds, total, wl.sigma, wl.pop, 0).cpu().numpy()
    idx = _sample_flat(rng, total, 0, 2000)
    ref = oracle.weight_gradient_at(fit64, wl.seeds, sig, wl.pop, 0, idx)
    assert_close(flat[idx], ref, TOL_F32, "flat gradient of the chained vector")


@pytest.mark.parametrize("key", [1, 2, 3])
def test_single_layer_forward_exact_f32(key):
    """The fp32 matrix-core math mode on the fp32 workloads."""
    print(f"workload {key} forward, fp32 matrix cores", flush=True)
    wl = workloads.make(key)
    L = wl.layers[0]
    sig = sigma32(wl.sigma)
    x, layers, seeds, _ = _dev_inputs(wl)
    w, b = layers[0]
    y = vn.virtual_perturbed_linear(x, w, b, seeds, wl.sigma, L.w_offset, math="f32")
    ids = list(range(wl.pop)) if wl.pop <= 8 else _pick_individuals(wl.pop)
    ref = oracle.perturbed_linear(wl.x[ids], L.weight, L.bias, wl.seeds[ids], sig, L.w_offset)
    assert_close(y[ids].cpu().numpy(), ref, TOL_F32, f"workload {key} exact fp32")


@pytest.mark.parametrize("key", [2, 5])
def test_repeat_calls_bit_identical(key):
    print(f"workload {key} determinism", flush=True)
    wl = workloads.make(key)
    L = wl.layers[0]
    x, layers, seeds, fit = _dev_inputs(wl)
    w, b = layers[0]
    y1 = vn.virtual_perturbed_linear(x, w, b, seeds, wl.sigma, L.w_offset)
    y2 = vn.virtual_perturbed_linear(x, w, b, seeds, wl.sigma, L.w_offset)
    assert torch.equal(y1, y2)
    g1 = vn.virtual_weight_gradient(fit, seeds, L.weight.shape, wl.sigma, wl.pop, L.w_offset)
    g2 = vn.virtual_weight_gradient(fit, seeds, L.weight.shape, wl.sigma, wl.pop, L.w_offset)
    assert torch.equal(g1, g2)
