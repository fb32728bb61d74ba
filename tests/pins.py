"""Checks that pin the CPU oracle to facts other than itself.

Each ``check_*`` raises AssertionError when the oracle disagrees with what the
EvoX ``virtual_noise`` API page or the mathematics fixes.  They run against the
real oracle in ``test_oracle_pins.py`` and against deliberately broken copies
of it in ``test_oracle_mutations.py`` (every planted mistake must trip at
least one check).

The independent reference used here is ``TextbookSplitMix``: a sequential
splitmix64 generator on Python big integers (state += GAMMA, then mix) that
never touches numpy, and pure-Python brute-force loops on tiny shapes.
"""

from __future__ import annotations

import ast
import math
import os

import numpy as np

import oracle.vn_oracle as vo

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
MASK64 = (1 << 64) - 1


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([p.strip() for p in line.split("|")])
    return rows


def page_gamma() -> int:
    return int(read_golden("gamma.txt")[0][0])


class TextbookSplitMix:
    """Sequential splitmix64 on Python ints: the n-th call returns
    mix(seed + (n+1)*GAMMA), produced by repeated Weyl additions."""

    def __init__(self, seed: int, m1: int, m2: int, gamma: int):
        self.state = seed & MASK64
        self.m1, self.m2, self.gamma = m1, m2, gamma

    def next(self) -> int:
        self.state = (self.state + self.gamma) & MASK64
        z = self.state
        z ^= z >> 30
        z = (z * self.m1) & MASK64
        z ^= z >> 27
        z = (z * self.m2) & MASK64
        z ^= z >> 31
        return z

    def stream(self, n):
        return [self.next() for _ in range(n)]


def textbook_noise_stream(seed: int, n: int):
    """The method's noise for indices 0..n-1 under readings A1-A3, from the
    sequential big-int generator and plain Python floats."""
    g = page_gamma()
    gen = TextbookSplitMix(seed, g, g, g)
    out = []
    for _ in range(n):
        r = gen.next() & 0xFFFFFFFF
        out.append((r >> 8) / 16777216.0 - 0.5)
    return out


# ----------------------------------------------------------------------------- constants

def check_gamma_constant():
    g = page_gamma()
    assert vo.GAMMA == g
    # floor(2^64 / phi) = floor(2^64 * (sqrt(5) - 1) / 2), by integer square root
    assert (math.isqrt(5 << 128) - (1 << 64)) // 2 == g
    assert g % 2 == 1  # odd, so the Weyl sequence has full period


def check_published_splitmix_vector():
    rows = read_golden("splitmix64_seed0.txt")
    idx = np.array([int(r[0]) for r in rows], dtype=np.int64)
    want = [int(r[1], 16) for r in rows]
    got = vo.noise_bits_at(np.array([0], dtype=np.int64), idx, vo.CANONICAL_M1, vo.CANONICAL_M2)[0]
    assert [int(v) for v in got] == want


def check_counter_matches_sequential():
    """Reading A1: the counter form equals stepping the textbook generator."""
    g = page_gamma()
    seeds = [0, 7, 1000, -1, 3, 2**63 - 1, -2**63, 123456789012345]
    n = 40
    got = vo.noise_u32(np.array(seeds, dtype=np.int64), n, 0)
    for row, seed in zip(got, seeds):
        ref = [v & 0xFFFFFFFF for v in TextbookSplitMix(seed, g, g, g).stream(n)]
        assert [int(v) for v in row] == ref
    # int32 seeds are sign-extended (reading A4)
    got32 = vo.noise_u32(np.array([-5, 5], dtype=np.int32), 3, 11)
    ref = [[v & 0xFFFFFFFF for v in TextbookSplitMix(s, g, g, g).stream(14)[11:]] for s in (-5, 5)]
    assert got32.tolist() == ref


def check_large_index_wrap():
    """Offsets far beyond 2^32: state = seed + (idx+1)*GAMMA mod 2^64 done in
    exact big-int arithmetic, mixed by the (published-vector-pinned) finalizer."""
    g = page_gamma()
    cases = [(3, 2**32 + 5), (0, 2**40), (1000, 266752), (511, 269321),
             (-7, 2**62 + 12345), (2**63 - 1, 2**63 - 2)]
    for seed, idx in cases:
        z0 = ((seed & MASK64) + (idx + 1) * g) & MASK64
        want = int(vo.splitmix_finalize(np.array([z0], dtype=np.uint64))[0]) & 0xFFFFFFFF
        got = int(vo.noise_u32_at(np.array([seed], dtype=np.int64), [idx])[0, 0])
        assert got == want


# ----------------------------------------------------------------------------- u mapping

def check_u_mapping_edges():
    r = np.array([0, 0xFF, 0x100, 0x80000000, 0xFFFFFFFF, 0x7FFFFFFF], dtype=np.uint32)
    n = vo.noise_from_bits(r)
    assert n[0] == -0.5 and n[1] == -0.5                 # r < 256 -> u = 0
    assert n[2] == -0.5 + 2.0 ** -24                      # one step of 2^-24
    assert n[3] == 0.0                                    # r = 2^31 -> u = 1/2
    assert n[4] == 0.5 - 2.0 ** -24                       # largest value, strictly below 0.5
    assert n[5] == -2.0 ** -24
    assert np.all(n.astype(np.float32).astype(np.float64) == n)   # exact in fp32


def check_range_and_statistics():
    """Page section "RNG: fast centered-uniform approximation": values in
    [-0.5, 0.5), mean ~0, variance 1/12.  5-sigma bounds at n = 2^22."""
    n = 1 << 22
    for seed in (0, 12345):
        r = vo.noise_u32(np.array([seed], dtype=np.int64), n, 0)[0]
        x = vo.noise_from_bits(r)
        assert np.all(np.isfinite(x)) and x.min() >= -0.5 and x.max() < 0.5
        assert abs(x.mean()) < 5 * math.sqrt(1 / (12 * n))
        assert abs(x.var() - 1 / 12) < 5 * math.sqrt(1 / (180 * n))
        u = (r >> np.uint32(24)).astype(np.int64)             # 256 equal bins of u
        counts = np.bincount(u, minlength=256)
        e = n / 256
        chi2 = float(((counts - e) ** 2 / e).sum())
        assert chi2 < 255 + 5 * math.sqrt(2 * 255)
        lag1 = np.corrcoef(x[:-1], x[1:])[0, 1]
        assert abs(lag1) < 5 / math.sqrt(n)
    a = vo.noise(np.array([1], dtype=np.int64), n, 0)[0]
    b = vo.noise(np.array([2], dtype=np.int64), n, 0)[0]
    assert abs(np.corrcoef(a, b)[0, 1]) < 5 / math.sqrt(n)


def check_determinism_and_shift():
    seeds = np.array([4, -9, 77], dtype=np.int64)
    a = vo.noise(seeds, 300, 1234)
    b = vo.noise(seeds, 300, 1234)
    assert np.array_equal(a, b)
    # N(seed, offset=o, flat=t) == N(seed, offset=o+t, flat=0)
    c = vo.noise(seeds, 200, 1334)
    assert np.array_equal(a[:, 100:], c[:, :200])


# ----------------------------------------------------------------------------- offsets

def check_compute_offsets_example():
    for shapes_txt, want_txt in read_golden("compute_offsets_example.txt"):
        assert vo.compute_offsets(ast.literal_eval(shapes_txt)) == ast.literal_eval(want_txt)
    assert vo.compute_offsets([]) == []
    assert vo.compute_offsets([(), (3,), (2, 2)]) == [0, 1, 4]
    assert vo.compute_offsets([(0, 5), (4,)]) == [0, 0]


# ----------------------------------------------------------------------------- forward

def _brute_forward(x, w, b, seeds, sigma, offset):
    """Pure-Python loops with noise from the sequential big-int generator."""
    pop = len(seeds)
    out_f, in_f = len(w), len(w[0])
    shared = np.asarray(x).ndim == 2
    n_stream = offset + out_f * in_f + out_f
    y = []
    for i in range(pop):
        nz = textbook_noise_stream(int(seeds[i]), n_stream)
        xi = x if shared else x[i]
        rows = []
        for bb in range(len(xi)):
            row = []
            for j in range(out_f):
                acc = 0.0
                for k in range(in_f):
                    acc += float(xi[bb][k]) * (float(w[j][k]) + sigma * nz[offset + j * in_f + k])
                if b is not None:
                    acc += float(b[j]) + sigma * nz[offset + out_f * in_f + j]
                row.append(acc)
            rows.append(row)
        y.append(rows)
    return np.array(y)


def check_forward_brute_force():
    rng = np.random.default_rng(5)
    for (pop, batch, fin, fout, offset, bias, shared) in [
        (3, 2, 5, 3, 0, True, False),
        (2, 3, 4, 6, 37, True, False),
        (2, 1, 7, 2, 5, False, False),
        (4, 2, 3, 5, 11, True, True),
    ]:
        x = rng.standard_normal((batch, fin) if shared else (pop, batch, fin))
        w = rng.standard_normal((fout, fin))
        b = rng.standard_normal(fout) if bias else None
        seeds = rng.integers(-1000, 1000, size=pop)
        sigma = 0.37
        got = vo.perturbed_linear(x, w, b, seeds, sigma, offset)
        want = _brute_forward(x.tolist(), w.tolist(), None if b is None else b.tolist(),
                              seeds, sigma, offset)
        assert got.shape == (pop, batch, fout)
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
        ii = rng.integers(0, pop, 6)
        bb = rng.integers(0, batch, 6)
        jj = rng.integers(0, fout, 6)
        at = vo.perturbed_linear_at(x, w, b, seeds, sigma, offset, ii, bb, jj)
        assert np.allclose(at, want[ii, bb, jj], rtol=1e-12, atol=1e-12)


def check_sigma_zero_is_linear():
    """sigma = 0 reduces to the textbook linear layer (torch.nn.functional.linear)."""
    import torch
    rng = np.random.default_rng(6)
    pop, batch, fin, fout = 3, 4, 9, 7
    x = rng.standard_normal((pop, batch, fin))
    w = rng.standard_normal((fout, fin))
    b = rng.standard_normal(fout)
    got = vo.perturbed_linear(x, w, b, np.arange(pop), 0.0, 3)
    want = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w),
                                      torch.from_numpy(b)).numpy()
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def check_shared_x_equals_replicated():
    rng = np.random.default_rng(7)
    pop, batch, fin, fout = 4, 3, 6, 5
    x = rng.standard_normal((batch, fin))
    w = rng.standard_normal((fout, fin))
    b = rng.standard_normal(fout)
    seeds = np.array([9, 8, 7, 6])
    a = vo.perturbed_linear(x, w, b, seeds, 0.1, 2)
    r = vo.perturbed_linear(np.broadcast_to(x, (pop, batch, fin)).copy(), w, b, seeds, 0.1, 2)
    assert np.array_equal(a, r)


def check_bias_none_vs_zero():
    """Reading A5: bias=None drops the bias noise, a zero bias keeps it."""
    x = np.zeros((1, 1, 2))
    w = np.zeros((3, 2))
    seeds = np.array([42])
    y_none = vo.perturbed_linear(x, w, None, seeds, 1.0, 0)
    y_zero = vo.perturbed_linear(x, w, np.zeros(3), seeds, 1.0, 0)
    assert np.all(y_none == 0.0)
    assert np.array_equal(y_zero[0, 0], np.array(textbook_noise_stream(42, 9)[6:9]))


# ----------------------------------------------------------------------------- gradients

def _brute_grad(fitness, seeds, n, sigma, offset):
    pop = len(seeds)
    streams = [textbook_noise_stream(int(s), offset + n) for s in seeds]
    return [sum(float(fitness[i]) * streams[i][offset + e] for i in range(pop)) / (pop * sigma)
            for e in range(n)]


def check_gradients_brute_force():
    rng = np.random.default_rng(8)
    for pop, fout, fin, offset in [(5, 3, 4, 0), (3, 2, 6, 29), (1, 1, 1, 3)]:
        fit = rng.standard_normal(pop)
        seeds = rng.integers(-50, 50, size=pop)
        sigma = 0.3
        gw = vo.weight_gradient(fit, seeds, (fout, fin), sigma, pop, offset)
        want = np.array(_brute_grad(fit, seeds, fout * fin, sigma, offset)).reshape(fout, fin)
        assert gw.shape == (fout, fin)
        assert np.allclose(gw, want, rtol=1e-12, atol=1e-12)
        boff = offset + fout * fin
        gb = vo.bias_gradient(fit, seeds, (fout,), sigma, pop, boff)
        wantb = np.array(_brute_grad(fit, seeds, fout, sigma, boff))
        assert np.allclose(gb, wantb, rtol=1e-12, atol=1e-12)
        flat = rng.integers(0, fout * fin, 5)
        at = vo.weight_gradient_at(fit, seeds, sigma, pop, offset, flat)
        assert np.allclose(at, want.reshape(-1)[flat], rtol=1e-12, atol=1e-12)


def check_one_hot_and_linearity():
    rng = np.random.default_rng(9)
    pop, fout, fin, offset, sigma = 8, 3, 5, 17, 0.125
    seeds = rng.integers(0, 10**6, size=pop)
    for i in (0, 5):
        f = np.zeros(pop)
        f[i] = 1.0
        g = vo.weight_gradient(f, seeds, (fout, fin), sigma, pop, offset)
        ni = np.array(textbook_noise_stream(int(seeds[i]), offset + fout * fin)[offset:])
        assert np.array_equal(g.reshape(-1), ni / (pop * sigma))
    f1, f2 = rng.standard_normal(pop), rng.standard_normal(pop)
    a, c = 0.7, -2.5
    g1 = vo.weight_gradient(f1, seeds, (fout, fin), sigma, pop, offset)
    g2 = vo.weight_gradient(f2, seeds, (fout, fin), sigma, pop, offset)
    g12 = vo.weight_gradient(a * f1 + c * f2, seeds, (fout, fin), sigma, pop, offset)
    assert np.allclose(g12, a * g1 + c * g2, rtol=1e-12, atol=1e-12)


def check_forward_gradient_consistency():
    """Page's requirement that forward and gradient regenerate the same noise:
    X = I, W = 0, sigma = 1, no bias gives Y[i] = N_i^T, which must equal the
    one-hot gradient readout; the forward's bias noise must equal the bias
    gradient's noise at the bias-region offset."""
    pop, fout, fin, offset = 4, 3, 5, 123
    seeds = np.array([3, -3, 99, 2**40])
    y = vo.perturbed_linear(np.eye(fin), np.zeros((fout, fin)), None, seeds, 1.0, offset)
    yb = vo.perturbed_linear(np.zeros((1, fin)), np.zeros((fout, fin)), np.zeros(fout),
                             seeds, 1.0, offset)
    for i in range(pop):
        f = np.zeros(pop)
        f[i] = 1.0
        g = vo.weight_gradient(f, seeds, (fout, fin), 1.0 / pop, pop, offset)
        assert np.array_equal(y[i].T, g)
        gb = vo.bias_gradient(f, seeds, (fout,), 1.0 / pop, pop, offset + fout * fin)
        assert np.array_equal(yb[i, 0], gb)


def check_reduce_metric_brute_force():
    rng = np.random.default_rng(10)
    n, offset, sigma = 13, 7, 0.4
    center = rng.standard_normal(n)
    seeds = [5, -1, 77]
    got = vo.reduce_metric(center, np.array(seeds), sigma, n, offset)
    for i, s in enumerate(seeds):
        nz = textbook_noise_stream(s, offset + n)
        want = sum(abs(center[k] + sigma * nz[offset + k]) for k in range(n)) / n
        assert abs(got[i] - want) < 1e-12


ALL_CHECKS = [
    check_gamma_constant,
    check_published_splitmix_vector,
    check_counter_matches_sequential,
    check_large_index_wrap,
    check_u_mapping_edges,
    check_range_and_statistics,
    check_determinism_and_shift,
    check_compute_offsets_example,
    check_forward_brute_force,
    check_sigma_zero_is_linear,
    check_shared_x_equals_replicated,
    check_bias_none_vs_zero,
    check_gradients_brute_force,
    check_one_hot_and_linearity,
    check_forward_gradient_consistency,
    check_reduce_metric_brute_force,
]
