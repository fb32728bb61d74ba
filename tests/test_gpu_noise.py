"""Bit-exact noise on the GPU: the hash words, the u values, and the noise as
seen through the forward kernel and the gradient kernel (the page's
requirement that both regenerate identical noise)."""

import numpy as np
import pytest
import torch

import oracle
import virtual_noise_perturbed_amd as vn
from gpu_util import bf16_round_cpu, device, to_dev, u32

pytestmark = pytest.mark.gpu

SEEDS = np.array([0, 7, 1000, -1, 3, 2**63 - 1, -2**63, 123456789012345, -987654321], dtype=np.int64)


@pytest.mark.parametrize("n,offset", [(1, 0), (1000, 0), (65537, 12345), (3000, 2**32 - 1500),
                                      (777, 2**40), (513, 2**62 + 7)])
def test_noise_u32_and_f32_bit_exact(n, offset):
    print(f"noise n={n} offset={offset}", flush=True)
    s = to_dev(SEEDS)
    r = u32(vn.noise_u32(s, n, offset))
    want = oracle.noise_u32(SEEDS, n, offset)
    assert np.array_equal(r, want)
    f = vn.noise_f32(s, n, offset).cpu().numpy()
    assert np.array_equal(f.astype(np.float64), oracle.noise(SEEDS, n, offset))
    assert f.min() >= -0.5 and f.max() < 0.5


def test_int32_seeds_sign_extended():
    s32 = np.array([-5, 5, -2**31, 2**31 - 1], dtype=np.int32)
    r = u32(vn.noise_u32(to_dev(s32), 300, 77))
    assert np.array_equal(r, oracle.noise_u32(s32.astype(np.int64), 300, 77))


def test_last_indices_of_largest_workloads():
    # transformer-width block: last weight element of individual 127; 3-layer MLP: last bias element
    for seed, idx in [(127, 4096 * 4096 - 1), (511, 269321), (4095, 256 * 512 - 1)]:
        s = np.array([seed], dtype=np.int64)
        r = u32(vn.noise_u32(to_dev(s), 1, idx))
        assert r[0, 0] == oracle.noise_u32_at(s, [idx])[0, 0]


def split_bf16_cpu(a):
    """hi = bf16(a), lo = bf16(a - hi), returned as hi + lo (exact in float64)."""
    hi = bf16_round_cpu(a)
    lo = bf16_round_cpu(np.asarray(a, dtype=np.float64) - hi)
    return hi + lo


@pytest.mark.parametrize("mode", ["bf16", "f32-default", "f32-exact"])
@pytest.mark.parametrize("fin,fout", [(16, 37), (40, 33), (100, 70), (256, 130), (13, 9)])
def test_forward_readout(mode, fin, fout):
    """X = I, W = 0, sigma = 1, no bias: Y[i] = N_i^T as the operand precision keeps
    it -- exactly N (fp32 matrix cores), bf16(N) (bf16 operands), or the two-term
    bf16 split of N (fp32 operands on the bf16 matrix cores)."""
    print(f"readout {mode} in={fin} out={fout}", flush=True)
    dev = device()
    dtype = torch.bfloat16 if mode == "bf16" else torch.float32
    pop, offset = 3, 1000
    seeds = np.array([11, -3, 2**40], dtype=np.int64)
    x = torch.eye(fin, dtype=dtype, device=dev)                 # shared (batch=in, in)
    w = torch.zeros((fout, fin), dtype=dtype, device=dev)
    y = vn.virtual_perturbed_linear(x, w, None, to_dev(seeds), 1.0, offset,
                                    math="f32" if mode == "f32-exact" else "default").cpu().numpy()
    n = oracle.noise(seeds, fout * fin, offset).reshape(pop, fout, fin)
    want = np.transpose(n, (0, 2, 1))
    if mode == "bf16":
        want = bf16_round_cpu(want)
    elif mode == "f32-default":
        want = split_bf16_cpu(want)
    assert np.array_equal(y.astype(np.float64), want)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_forward_readout_tiny_sigma(dt):
    """sigma = 2^-101: sigma * 2^-24 is subnormal, so the call takes the kernels
    that form sigma * N in floating point; X = I, W = 0 reads back sigma * N
    (exact in fp32, rounded once to bf16 for bf16 operands)."""
    dev = device()
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    fin, fout, offset = 40, 24, 77
    seeds = np.array([3, -9], dtype=np.int64)
    sigma = 2.0 ** -101
    x = torch.eye(fin, dtype=dtype, device=dev)
    w = torch.zeros((fout, fin), dtype=dtype, device=dev)
    y = vn.virtual_perturbed_linear(x, w, None, to_dev(seeds), sigma, offset).cpu().numpy()
    n = oracle.noise(seeds, fout * fin, offset).reshape(2, fout, fin)
    want = np.transpose(n, (0, 2, 1)) * sigma
    if dt == "bf16":
        want = bf16_round_cpu(want)
    assert np.array_equal(y.astype(np.float64), want)


def test_forward_bias_readout():
    """X = 0, W = 0, b = 0, sigma = 1: Y[i, b, j] = nb_i[j] at offset + out*in + j."""
    dev = device()
    pop, batch, fin, fout, offset = 4, 3, 24, 50, 31
    seeds = np.arange(pop, dtype=np.int64) * 1000 - 1500
    x = torch.zeros((pop, batch, fin), device=dev)
    w = torch.zeros((fout, fin), device=dev)
    b = torch.zeros((fout,), device=dev)
    y = vn.virtual_perturbed_linear(x, w, b, to_dev(seeds), 1.0, offset).cpu().numpy()
    nb = oracle.noise(seeds, fout, offset + fout * fin)
    assert np.array_equal(y.astype(np.float64), np.broadcast_to(nb[:, None, :], y.shape))


@pytest.mark.parametrize("n", [300, 20000, (1 << 20) + 300])   # population-major, element-major E=1 and E=4
def test_gradient_readout_one_hot(n):
    """fitness = e_i, sigma = 1/pop (pop a power of two): grad = N_i exactly."""
    print(f"gradient readout n={n}", flush=True)
    pop, offset = 8, 555
    seeds = np.array([5, 4, 3, 2, 1, 0, -1, -2], dtype=np.int64) * 7919
    s = to_dev(seeds)
    for i in (0, 5, 7):
        f = np.zeros(pop, dtype=np.float32)
        f[i] = 1.0
        g = vn.virtual_flat_gradient(to_dev(f), s, n, 1.0 / pop, pop, offset).cpu().numpy()
        want = oracle.noise_at(seeds[i:i + 1], offset + np.arange(n))[0]
        assert np.array_equal(g.astype(np.float64), want), f"individual {i}"


def test_forward_and_gradient_see_the_same_noise():
    """Readout through the forward kernel equals readout through the weight and
    bias gradient kernels, element for element."""
    dev = device()
    pop, fin, fout, offset = 4, 48, 20, 2**33 + 5
    seeds = np.array([1, 2, 3, 4], dtype=np.int64)
    s = to_dev(seeds)
    x = torch.eye(fin, device=dev)
    y = vn.virtual_perturbed_linear(x, torch.zeros((fout, fin), device=dev), None, s, 1.0, offset, math="f32")
    yb = vn.virtual_perturbed_linear(torch.zeros((1, fin), device=dev), torch.zeros((fout, fin), device=dev),
                                     torch.zeros((fout,), device=dev), s, 1.0, offset)
    for i in range(pop):
        f = torch.zeros(pop, device=dev)
        f[i] = 1.0
        gw = vn.virtual_weight_gradient(f, s, (fout, fin), 1.0 / pop, pop, offset)
        gb = vn.virtual_bias_gradient(f, s, (fout,), 1.0 / pop, pop, offset + fout * fin)
        assert torch.equal(y[i].T, gw)
        assert torch.equal(yb[i, 0], gb)
