"""Noise-sensitive parity at the full sizes of the two bf16 projections
(pop 128 x batch 256 x 4096 -> 4096 with per-individual inputs, and the
large-batch 4096 x 4096 shared-input layer), in the launch configurations the
bench times.

At sigma = 0.001 and in = 4096 the noise term of those workloads is smaller
than the bf16 tolerance, so a normwise check of their outputs cannot tell
whether the noise is there.  These tests make it visible:

* readouts (the forward/gradient consistency requirement of the module
  introduction on the EvoX virtual_noise page): W = 0, sigma = 1, no bias and
  one-hot input rows, so that every output is exactly bf16(N_i[j, k]) for a
  known (j, k) -- compared element for element with the oracle's noise over
  whole outputs;
* the same shapes with random data at a sigma where the oracle's noise term is
  several times the tolerance (asserted), compared normwise.

A kernel that dropped sigma * N, or mis-indexed the seed, the offset, a
column tile or an individual, fails every one of them.
"""

import numpy as np
import pytest
import torch

import oracle
import virtual_noise_perturbed_amd as vn
import workloads
from gpu_util import TOL_BF16, assert_close, bf16_round_cpu, device, normwise_err, sigma32, to_dev

pytestmark = pytest.mark.gpu

FIN = FOUT = 4096
# Individuals past one group of eight: the per-individual launch order places
# groups of eight individuals on the eight XCDs and spaces a last, partial
# group differently, so 11 individuals cover both.
WIDE_SEEDS = np.array([0, 1, 2, 3, 4, 5, 6, 7, 127, -1, 2**40 + 3], dtype=np.int64)


def _windows(pop, batch):
    """Start of the k-window individual i reads: different for every
    individual, the first at 0 and the last ending at FIN."""
    starts = (np.arange(pop, dtype=np.int64) * 1543) % (FIN - batch + 1)
    starts[0] = 0
    starts[-1] = FIN - batch
    return starts


def test_wide_forward_readout_full_size():
    """pop 11, batch 256, 4096 -> 4096, bf16, own X per individual (the
    wide workload's launch configuration): X[i][b, k] = 1 for
    k = start_i + b, W = 0, sigma = 1, offset 12345.  Then
    Y[i][b, j] = bf16(N_i[j, start_i + b]) exactly."""
    print("wide readout: pop 11, batch 256, 4096->4096, bf16, own X", flush=True)
    dev = device()
    pop, batch, offset = len(WIDE_SEEDS), 256, 12345
    starts = _windows(pop, batch)
    x = torch.zeros((pop, batch, FIN), dtype=torch.bfloat16, device=dev)
    rows = torch.arange(batch, device=dev)
    for i in range(pop):
        x[i, rows, int(starts[i]) + rows] = 1.0
    w = torch.zeros((FOUT, FIN), dtype=torch.bfloat16, device=dev)
    y = vn.virtual_perturbed_linear(x, w, None, to_dev(WIDE_SEEDS), 1.0, offset)
    torch.cuda.synchronize()
    assert y.shape == (pop, batch, FOUT)
    jj = np.arange(FOUT, dtype=np.int64)
    for i in range(pop):
        ks = int(starts[i]) + np.arange(batch, dtype=np.int64)
        idx = offset + (jj[None, :] * FIN + ks[:, None])          # (batch, out): element (j, k) of row b
        want = bf16_round_cpu(oracle.noise_at(WIDE_SEEDS[i:i + 1], idx.reshape(-1))[0]).reshape(batch, FOUT)
        got = y[i].cpu().numpy().astype(np.float64)
        bad = np.argwhere(got != want)
        assert bad.size == 0, (f"individual {i} (seed {WIDE_SEEDS[i]}): {len(bad)} mismatches, first at "
                               f"(row, col) {tuple(bad[0])}: got {got[tuple(bad[0])]}, want {want[tuple(bad[0])]}")


def test_large_batch_forward_readout_full_size():
    """pop 10, batch 4096, 4096 -> 4096, bf16, one X shared by all (the
    large-batch workload's launch configuration): X = I, W = 0, sigma = 1,
    offset 777.  Then Y[i][b, j] = bf16(N_i[j, b]): whole outputs of three
    individuals and 256 random rows of every other one."""
    print("large-batch readout: pop 10, batch 4096, 4096->4096, bf16, shared X", flush=True)
    dev = device()
    seeds = np.array([9, 8, 7, 6, 5, 4, 3, 2, 1, -2**63], dtype=np.int64)
    pop, offset = len(seeds), 777
    x = torch.eye(FIN, dtype=torch.bfloat16, device=dev)
    w = torch.zeros((FOUT, FIN), dtype=torch.bfloat16, device=dev)
    y = vn.virtual_perturbed_linear(x, w, None, to_dev(seeds), 1.0, offset)
    torch.cuda.synchronize()
    assert y.shape == (pop, FIN, FOUT)
    rng = np.random.default_rng(606)
    jj = np.arange(FOUT, dtype=np.int64)
    for i in range(pop):
        if i in (0, 4, pop - 1):
            rows = np.arange(FIN, dtype=np.int64)
        else:
            rows = np.unique(np.concatenate([[0, 511, 512, FIN - 1], rng.integers(0, FIN, 252)]))
        got = y[i][torch.as_tensor(rows, device=dev)].cpu().numpy().astype(np.float64)
        for r0 in range(0, len(rows), 512):
            rr = rows[r0:r0 + 512]
            idx = offset + (jj[None, :] * FIN + rr[:, None])
            want = bf16_round_cpu(oracle.noise_at(seeds[i:i + 1], idx.reshape(-1))[0]).reshape(len(rr), FOUT)
            g = got[r0:r0 + 512]
            bad = np.argwhere(g != want)
            assert bad.size == 0, (f"individual {i}: {len(bad)} mismatches, first at row {rr[bad[0][0]]}, "
                                   f"col {bad[0][1]}")


def _noise_visible(x, L, seeds, sig, ii, bb, jj, tol):
    """Oracle outputs at the sampled elements, after checking that the noise
    term moves them by more than five times the tolerance."""
    ref = oracle.perturbed_linear_at(x, L.weight, L.bias, seeds, sig, L.w_offset, ii, bb, jj)
    ref0 = oracle.perturbed_linear_at(x, L.weight, L.bias, seeds, 0.0, L.w_offset, ii, bb, jj)
    term = normwise_err(ref0, ref)
    assert term > 5 * tol, f"noise term {term:.3e} is not visible at tolerance {tol:.1e}"
    return ref, term


@pytest.mark.parametrize("key", [5, 6])
def test_bf16_projection_noise_visible(key):
    """The wide and large-batch workloads' data and shapes at sigma = 0.05,
    where the noise term is about as large as X W^T: sampled outputs over all
    individuals and rows, plus whole rows of the first and last individual."""
    wl = workloads.make(key)
    sigma = 0.05
    sig = sigma32(sigma)
    print(f"workload {key} at sigma {sigma}", flush=True)
    L = wl.layers[0]
    x = to_dev(wl.x, torch.bfloat16)
    y = vn.virtual_perturbed_linear(x, to_dev(L.weight, torch.bfloat16), None, to_dev(wl.seeds), sigma, L.w_offset)
    torch.cuda.synchronize()
    rng = np.random.default_rng(50 + key)
    n = 600
    ii = np.concatenate([rng.integers(0, wl.pop, n), np.zeros(64, np.int64), np.full(64, wl.pop - 1)])
    bb = np.concatenate([rng.integers(0, wl.batch, n), np.full(64, wl.batch - 1), np.zeros(64, np.int64)])
    jj = np.concatenate([rng.integers(0, L.out_features, n), rng.integers(0, L.out_features, 128)])
    ref, term = _noise_visible(wl.x, L, wl.seeds, sig, ii, bb, jj, TOL_BF16)
    got = y[torch.as_tensor(ii), torch.as_tensor(bb), torch.as_tensor(jj)].cpu().numpy()
    err = assert_close(got, ref, TOL_BF16, f"workload {key} at sigma {sigma} (noise term {term:.2f})")
    print(f"workload {key}: noise term {term:.3f}, error {err:.2e}", flush=True)


@pytest.mark.parametrize("pop", [128, 16])
def test_reduce_metric_full_size_sampled(pop):
    """The reduce metric at the sizes of the two bf16 projections (4096 * 4096
    parameters; pop 128: eight segments per individual, pop 16: 64 -- the
    launches the bench times), sampled: the oracle computes three whole
    individuals (first, middle, last).  At sigma = 0.5 the noise moves each
    mean by about 1%, twenty times the tolerance (asserted against the mean
    without noise)."""
    device()
    n, offset, sig = FIN * FOUT, 3, 0.5
    print(f"reduce metric full size: pop={pop} n={n}", flush=True)
    rng = np.random.default_rng(20261202 + 5)
    center = rng.standard_normal(n, dtype=np.float32)
    seeds = np.arange(pop, dtype=np.int64)
    got = vn.virtual_reduce_metric(to_dev(center), to_dev(seeds), sig, n, offset).cpu().numpy()
    pick = np.array([0, pop // 2 - 1, pop - 1])
    want = oracle.reduce_metric(center, seeds[pick], sigma32(sig), n, offset)
    plain = np.full(len(pick), np.mean(np.abs(center.astype(np.float64))))
    assert normwise_err(want, plain) > 20 * 1e-4, "the noise must move the means"
    assert_close(got[pick], want, 1e-4, "reduce metric, sampled individuals")
