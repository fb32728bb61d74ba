"""Large-batch bf16 forward through materialized perturbed weights: the path a
workspace enables must give the same bits as the fused kernels (same perturbed
weights, same MFMA accumulation order), and match the oracle."""

import numpy as np
import pytest
import torch

import oracle
import virtual_noise_perturbed_amd as vn
import workloads
from virtual_noise_perturbed_amd import _lib
from gpu_util import TOL_BF16, assert_close, normwise_err, sigma32, to_dev

pytestmark = pytest.mark.gpu


def _ws_bytes(pop, batch, fin, fout):
    need = __import__("ctypes").c_int64(0)
    st = _lib.load().vn_perturbed_linear_workspace_size(_lib.VN_BF16, pop, batch, fin, fout, 0,
                                                        __import__("ctypes").byref(need))
    assert st == _lib.VN_OK
    return need.value


# (pop, batch, in, out, bias, shared_x, relu, int32 seeds, offset)
CASES = [
    (3, 2048, 256, 384, True, False, True, False, 7),       # ragged column tile, bias + relu
    (2, 2100, 192, 256, False, True, False, False, 2**33),  # ragged row tile, shared x
    (2, 2304, 128, 300, True, True, False, True, 3),        # two k-stages only; int32 seeds
    (1, 2048, 640, 257, True, False, True, False, 0),       # last column tile of one column, moved back
    (4, 2560, 320, 512, False, False, False, False, 11),    # odd number of k-stages (5)
]


def _check_same_bits(case):
    pop, batch, fin, fout, bias, shared, relu, s32, offset = case
    print(f"materialized vs fused {case}", flush=True)
    assert _ws_bytes(pop, batch, fin, fout) > 0, "shape should take the materialized path"
    wl = workloads.make_custom(pop, batch, fin, fout, dtype="bf16", bias=bias, shared_x=shared, sigma=0.05,
                               offset=offset, seed=fin + fout, seed_base=-5)
    L = wl.layers[0]
    seeds = to_dev(wl.seeds.astype(np.int32) if s32 else wl.seeds)
    args = (to_dev(wl.x, torch.bfloat16), to_dev(L.weight, torch.bfloat16),
            None if L.bias is None else to_dev(L.bias), seeds, wl.sigma, offset)
    act = "relu" if relu else None
    ym = vn.virtual_perturbed_linear(*args, activation=act, materialize=True)
    yf = vn.virtual_perturbed_linear(*args, activation=act, materialize=False)
    torch.cuda.synchronize()
    assert torch.equal(ym, yf), f"max |diff| {(ym - yf).abs().max().item():.3e}"


@pytest.mark.parametrize("case", CASES, ids=[f"p{c[0]}b{c[1]}i{c[2]}o{c[3]}" for c in CASES])
def test_materialized_same_bits_as_fused(case):
    _check_same_bits(case)


@pytest.mark.parametrize("pop,batch,fin,fout,offset", [
    (2, 2048, 128, 272, 5),      # ragged last column tile (moved back by 240 columns)
    (1, 2100, 192, 300, 2**35),  # ragged last row tile and column tile
])
def test_materialized_against_oracle(pop, batch, fin, fout, offset):
    print(f"materialized vs oracle {(pop, batch, fin, fout, offset)}", flush=True)
    assert _ws_bytes(pop, batch, fin, fout) > 0
    wl = workloads.make_custom(pop, batch, fin, fout, dtype="bf16", bias=True, shared_x=False, sigma=0.05,
                               offset=offset, seed=44)
    L = wl.layers[0]
    y = vn.virtual_perturbed_linear(to_dev(wl.x, torch.bfloat16), to_dev(L.weight, torch.bfloat16),
                                    to_dev(L.bias), to_dev(wl.seeds), wl.sigma, offset).cpu().numpy()
    ref = oracle.perturbed_linear(wl.x, L.weight, L.bias, wl.seeds, sigma32(wl.sigma), offset)
    ref0 = oracle.perturbed_linear(wl.x, L.weight, L.bias, wl.seeds, 0.0, offset)
    assert normwise_err(ref0, ref) > 5 * TOL_BF16, "the noise must be visible at this sigma"
    assert_close(y, ref, TOL_BF16, "materialized forward")


@pytest.mark.parametrize("fout", [255, 256])
def test_output_width_boundary(fout):
    """Fewer than 256 outputs keep the noise inside the product (no workspace);
    256 take the materialized path.  Both against the oracle, and the
    materialized result against the fused one bit for bit."""
    pop, batch, fin, offset = 1, 2048, 128, 77
    print(f"output width {fout}", flush=True)
    ws = _ws_bytes(pop, batch, fin, fout)
    assert (ws > 0) == (fout >= 256)
    wl = workloads.make_custom(pop, batch, fin, fout, dtype="bf16", bias=True, shared_x=False, sigma=0.05,
                               offset=offset, seed=fout)
    L = wl.layers[0]
    args = (to_dev(wl.x, torch.bfloat16), to_dev(L.weight, torch.bfloat16), to_dev(L.bias), to_dev(wl.seeds),
            wl.sigma, offset)
    ym = vn.virtual_perturbed_linear(*args, materialize=True)
    yf = vn.virtual_perturbed_linear(*args, materialize=False)
    torch.cuda.synchronize()
    assert torch.equal(ym, yf)
    ref = oracle.perturbed_linear(wl.x, L.weight, L.bias, wl.seeds, sigma32(wl.sigma), offset)
    assert_close(ym.cpu().numpy(), ref, TOL_BF16, f"forward, {fout} outputs")


def test_materialized_several_groups():
    """4096 x 4096 weights: 8 individuals per 256 MiB group, so 9 individuals
    take two groups (the second with one individual)."""
    pop, batch, fin, fout = 9, 2048, 4096, 4096
    print("materialized, two groups", flush=True)
    assert _ws_bytes(pop, batch, fin, fout) == 8 * fin * fout * 2
    gen = torch.Generator(device="cpu").manual_seed(123)
    x = (torch.randn((pop, batch, fin), generator=gen) * 0.5).to(torch.bfloat16).to("cuda:0")
    w = (torch.randn((fout, fin), generator=gen) / 64).to(torch.bfloat16).to("cuda:0")
    b = torch.randn((fout,), generator=gen).to("cuda:0")
    seeds = torch.arange(pop, dtype=torch.int64, device="cuda:0") * 1000003 - 7
    ym = vn.virtual_perturbed_linear(x, w, b, seeds, 0.05, 99, materialize=True)
    yf = vn.virtual_perturbed_linear(x, w, b, seeds, 0.05, 99, materialize=False)
    torch.cuda.synchronize()
    assert torch.equal(ym, yf), f"max |diff| {(ym - yf).abs().max().item():.3e}"


def _random_cases(n, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        pop = int(rng.integers(1, 4))
        batch = int(rng.integers(2048, 2700))
        fin = int(rng.integers(2, 12)) * 64
        fout = int(rng.integers(256, 700))
        cases.append((pop, batch, fin, fout, bool(rng.integers(2)), bool(rng.integers(2)),
                      bool(rng.integers(2)), bool(rng.integers(2)), int(rng.integers(0, 2**40))))
    return cases


RANDOM_CASES = _random_cases(8)


@pytest.mark.parametrize("case", RANDOM_CASES, ids=[f"r{k}" for k in range(len(RANDOM_CASES))])
def test_materialized_random_shapes_same_bits(case):
    """Seeded random shapes (ragged batch and out, any in that is a multiple of
    64, bias / relu / shared x / int32 seeds at random): same bits as the fused
    kernels."""
    _check_same_bits(case)
