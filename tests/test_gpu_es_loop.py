"""End-to-end use of the hot path: a few evolution-strategies iterations on a
synthetic regression, everything through the library.

Each iteration evaluates the population with the perturbed forward, turns the
per-individual losses into centered-rank fitness, estimates the gradient with
the weight and bias estimators at the blocks' offsets from compute_offsets,
and takes an ascent step (the estimator points towards higher fitness).  The
loss of the unperturbed layer must fall steadily, and the estimate must point
the same way as the exact gradient of the smoothed loss.
"""

import numpy as np
import pytest
import torch

import virtual_noise_perturbed_amd as vn
from gpu_util import device

pytestmark = pytest.mark.gpu


def _centered_ranks(x: torch.Tensor) -> torch.Tensor:
    ranks = torch.empty_like(x)
    ranks[torch.argsort(x)] = torch.arange(x.numel(), device=x.device, dtype=x.dtype)
    return ranks / (x.numel() - 1) - 0.5


def test_es_loop_reduces_loss():
    print("ES loop on a synthetic regression", flush=True)
    dev = device()
    g = torch.Generator().manual_seed(7)
    fin, fout, batch, pop, sigma, lr = 32, 8, 64, 256, 0.05, 0.06
    x = torch.randn(batch, fin, generator=g).to(dev)
    w_true = (torch.randn(fout, fin, generator=g) / fin ** 0.5).to(dev)
    b_true = (0.1 * torch.randn(fout, generator=g)).to(dev)
    target = x @ w_true.T + b_true
    w = torch.zeros(fout, fin, device=dev)
    b = torch.zeros(fout, device=dev)
    offsets = vn.compute_offsets([(fout, fin), (fout,)])
    assert offsets == [0, fout * fin]

    def loss(w_, b_):
        return float(((x @ w_.T + b_ - target) ** 2).mean())

    losses = [loss(w, b)]
    for gen in range(40):
        seeds = torch.arange(gen * pop, (gen + 1) * pop, device=dev)
        y = vn.virtual_perturbed_linear(x, w, b, seeds, sigma, offsets[0])        # shared x: (pop, batch, fout)
        per = ((y - target) ** 2).mean(dim=(1, 2))
        fit = _centered_ranks(-per)                                                # higher is better
        gw = vn.virtual_weight_gradient(fit, seeds, w.shape, sigma, pop, offsets[0])
        gb = vn.virtual_bias_gradient(fit, seeds, b.shape, sigma, pop, offsets[1])
        if gen == 0:
            # the whole parameter vector in one launch gives the same estimate
            flat = vn.virtual_flat_gradient(fit, seeds, fout * fin + fout, sigma, pop, 0)
            both = torch.cat([gw.flatten(), gb])
            assert float((flat - both).abs().max()) <= 1e-5 * float(both.abs().max())
        step = torch.cat([gw.flatten(), gb])
        step = lr * step / (step.norm() + 1e-12)                                   # fixed-length ascent step
        w = w + step[: fout * fin].view(fout, fin)
        b = b + step[fout * fin:]
        losses.append(loss(w, b))
    torch.cuda.synchronize()
    print("losses", [round(v, 4) for v in losses[::8]], flush=True)
    assert losses[-1] < 0.5 * losses[0]
    # mostly monotone: at most a few small upticks
    ups = sum(1 for a, c in zip(losses, losses[1:]) if c > a * 1.02)
    assert ups <= 4


def test_es_estimate_aligns_with_exact_gradient():
    """With fitness = -loss_i (no ranks) and a large population, the weight
    estimate is a positive multiple of -d loss / dW up to sampling noise: the
    cosine with the exact gradient at the unperturbed weights must be clearly
    positive."""
    dev = device()
    g = torch.Generator().manual_seed(11)
    fin, fout, batch, pop, sigma = 16, 4, 32, 8192, 0.01
    x = torch.randn(batch, fin, generator=g).to(dev)
    target = torch.randn(batch, fout, generator=g).to(dev)
    w = (torch.randn(fout, fin, generator=g) / 4).to(dev)
    seeds = torch.arange(pop, device=dev)
    y = vn.virtual_perturbed_linear(x, w, None, seeds, sigma, 0)
    fit = -((y - target) ** 2).mean(dim=(1, 2))
    fit = fit - fit.mean()
    gw = vn.virtual_weight_gradient(fit, seeds, w.shape, sigma, pop, 0)
    exact = -(2.0 / (batch * fout)) * ((x @ w.T - target).T @ x)            # -d loss / dW
    cos = float((gw * exact).sum() / (gw.norm() * exact.norm()))
    print(f"cosine(estimate, -grad) = {cos:.3f}", flush=True)
    assert cos > 0.8
    # scale: E[f N]/sigma = Var(N) * (-dL/dW) = (1/12) (-dL/dW) for small sigma
    ratio = float((gw * exact).sum() / (exact * exact).sum())
    assert 0.5 / 12 < ratio < 2.0 / 12
