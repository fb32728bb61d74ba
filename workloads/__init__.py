"""Seeded synthetic inputs for the virtual-noise ES linear layer.

This module only draws inputs (activations, weights, biases, fitness, seeds);
it holds none of the method's arithmetic, so both the oracle-side tests and
the HIP-side tests and bench can use it without sharing any of the method.

The five workloads mirror the shapes and value distributions of the
population-ES linear layer described on the EvoX ``virtual_noise`` API page
(per-individual (pop, batch, in) inputs, (out, in) weights, blocks chained by
flat offsets as in the page's ``compute_offsets`` example).  No public dataset
is involved; every array comes from ``numpy.random.default_rng(20261202 + k)``
for workload k, drawn in the order X, weights, biases, raw fitness.  ``N(m, v)``
means mean m and variance v.  bf16 workloads draw fp32 values and round them
to the nearest bf16 (ties to even) here, so every consumer sees the same
bf16-representable values.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

BASE_SEED = 20261202


@dataclass
class Layer:
    weight: np.ndarray            # (out, in) float32 (bf16-representable for bf16 workloads)
    bias: Optional[np.ndarray]    # (out,) float32 or None
    w_offset: int                 # flat noise offset of the weight block
    b_offset: int                 # flat noise offset of the bias block (= w_offset + out*in)

    @property
    def out_features(self) -> int:
        return int(self.weight.shape[0])

    @property
    def in_features(self) -> int:
        return int(self.weight.shape[1])


@dataclass
class Workload:
    key: int
    name: str
    pop: int
    batch: int
    dtype: str                    # "f32" or "bf16": dtype of x and the weights
    seeds: np.ndarray             # (pop,) int64
    sigma: float
    x: np.ndarray                 # (pop, batch, in0) float32, or (batch, in0) when shared
    layers: List[Layer]
    fitness: np.ndarray           # (pop,) float32
    relu_between: bool = False
    notes: str = ""
    shapes: list = field(default_factory=list)   # parameter block shapes in flat order

    @property
    def total_params(self) -> int:
        return sum(int(np.prod(s)) for s in self.shapes)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 value (ties to even), returned as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = ((bits + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
    return rounded.view(np.float32)


def _normal(rng, shape, var=1.0):
    z = rng.standard_normal(size=shape, dtype=np.float32)
    if var != 1.0:
        z *= np.float32(np.sqrt(var))
    return z


def _uniform(rng, shape, lo, hi):
    return rng.uniform(lo, hi, size=shape).astype(np.float32)


def centered_ranks(raw: np.ndarray) -> np.ndarray:
    """rank_i / (P - 1) - 0.5 with ranks from a stable argsort of raw scores."""
    p = raw.shape[0]
    ranks = np.empty(p, dtype=np.float64)
    ranks[np.argsort(raw, kind="stable")] = np.arange(p, dtype=np.float64)
    if p == 1:
        return np.zeros(1, dtype=np.float32)
    return (ranks / (p - 1) - 0.5).astype(np.float32)


# Flat noise offsets of every parameter block, written out (weights then bias
# of each layer, back to back, as the page's compute_offsets example lays out
# an MLP's blocks): per layer (weight offset, bias offset).  Written as
# literals so that this module computes no part of the method; the tests check
# them against compute_offsets of the block shapes.
LAYER_OFFSETS = {
    1: [(0, 2048)],                                          # 64 -> 32 with bias
    2: [(0, 1048576)],                                       # 1024 -> 1024 with bias
    3: [(0, 131072)],                                        # 512 -> 256, no bias
    4: [(0, 200704), (200960, 266496), (266752, 269312)],   # 784 -> 256 -> 256 -> 10, biases
    5: [(0, 16777216)],                                      # 4096 -> 4096, no bias
    6: [(0, 16777216)],                                      # 4096 -> 4096, no bias
}


def _block_shapes(shapes_io, biases):
    """[(out, in), (out,)?, ...] in flat order."""
    shapes = []
    for (i, o), has_b in zip(shapes_io, biases):
        shapes.append((o, i))
        if has_b:
            shapes.append((o,))
    return shapes


DESCRIPTIONS = {
    1: "tiny single layer: pop 8, batch 4, 64->32, fp32",
    2: "MLP hidden layer: pop 256, batch 32, 1024->1024, fp32",
    3: "RL policy single observation: pop 4096, batch 1, 512->256, fp32",
    4: "3-layer MLP 784->256->256->10 chained by flat offsets: pop 512, batch 64, fp32",
    5: "transformer-width projection: pop 128, batch 256, 4096->4096, bf16 operands",
    6: "large-batch shared-input projection: pop 16, batch 4096 (one X for all), 4096->4096, bf16 operands",
}


def make(key: int) -> Workload:
    """Full-size workload ``key`` (1..6)."""
    rng = np.random.default_rng(BASE_SEED + key)
    if key == 1:
        pop, batch, fin, fout = 8, 4, 64, 32
        x = _normal(rng, (pop, batch, fin))
        w = _normal(rng, (fout, fin), 1.0 / fin)
        b = _normal(rng, (fout,), 0.01)
        fit = _normal(rng, (pop,))
        per, shapes = LAYER_OFFSETS[1], _block_shapes([(fin, fout)], [True])
        return Workload(1, DESCRIPTIONS[1], pop, batch, "f32", np.arange(pop, dtype=np.int64),
                        0.02, x, [Layer(w, b, *per[0])], fit, shapes=shapes)
    if key == 2:
        pop, batch, fin, fout = 256, 32, 1024, 1024
        x = _normal(rng, (pop, batch, fin))
        w = _normal(rng, (fout, fin), 1.0 / fin)
        b = np.zeros(fout, dtype=np.float32)
        fit = centered_ranks(_normal(rng, (pop,)))
        per, shapes = LAYER_OFFSETS[2], _block_shapes([(fin, fout)], [True])
        return Workload(2, DESCRIPTIONS[2], pop, batch, "f32",
                        1000 + np.arange(pop, dtype=np.int64), 0.01, x,
                        [Layer(w, b, *per[0])], fit, shapes=shapes)
    if key == 3:
        pop, batch, fin, fout = 4096, 1, 512, 256
        x = _uniform(rng, (pop, batch, fin), -1.0, 1.0)
        w = _normal(rng, (fout, fin), 1.0 / fin)
        fit = _normal(rng, (pop,))
        per, shapes = LAYER_OFFSETS[3], _block_shapes([(fin, fout)], [False])
        return Workload(3, DESCRIPTIONS[3], pop, batch, "f32", np.arange(pop, dtype=np.int64),
                        0.05, x, [Layer(w, None, *per[0])], fit, shapes=shapes)
    if key == 4:
        pop, batch = 512, 64
        dims = [(784, 256), (256, 256), (256, 10)]
        x = _uniform(rng, (pop, batch, 784), 0.0, 1.0)
        ws = [_normal(rng, (o, i), 1.0 / i) for i, o in dims]
        bs = [np.zeros(o, dtype=np.float32) for _, o in dims]
        fit = _normal(rng, (pop,))
        per, shapes = LAYER_OFFSETS[4], _block_shapes(dims, [True, True, True])
        layers = [Layer(w, b, *p) for w, b, p in zip(ws, bs, per)]
        return Workload(4, DESCRIPTIONS[4], pop, batch, "f32", np.arange(pop, dtype=np.int64),
                        0.02, x, layers, fit, relu_between=True, shapes=shapes)
    if key == 5:
        pop, batch, fin, fout = 128, 256, 4096, 4096
        x = round_to_bf16(_normal(rng, (pop, batch, fin)))
        w = round_to_bf16(_normal(rng, (fout, fin), 1.0 / fin))
        fit = _normal(rng, (pop,))
        per, shapes = LAYER_OFFSETS[5], _block_shapes([(fin, fout)], [False])
        return Workload(5, DESCRIPTIONS[5], pop, batch, "bf16", np.arange(pop, dtype=np.int64),
                        0.001, x, [Layer(w, None, *per[0])], fit, shapes=shapes)
    if key == 6:
        # the large-batch regime: one (batch, in) input shared by every
        # individual, enough rows per individual for the matrix cores to bind
        pop, batch, fin, fout = 16, 4096, 4096, 4096
        x = round_to_bf16(_normal(rng, (batch, fin)))
        w = round_to_bf16(_normal(rng, (fout, fin), 1.0 / fin))
        fit = _normal(rng, (pop,))
        per, shapes = LAYER_OFFSETS[6], _block_shapes([(fin, fout)], [False])
        return Workload(6, DESCRIPTIONS[6], pop, batch, "bf16", np.arange(pop, dtype=np.int64),
                        0.001, x, [Layer(w, None, *per[0])], fit, shapes=shapes)
    raise ValueError(f"unknown workload {key}")


def make_custom(pop: int, batch: int, fin: int, fout: int, *, dtype: str = "f32",
                bias: bool = True, shared_x: bool = False, sigma: float = 0.05,
                offset: int = 0, seed: int = 0, seed_base: int = 0,
                seeds: Optional[np.ndarray] = None) -> Workload:
    """A single-layer workload of arbitrary (possibly ragged) shape for tests."""
    rng = np.random.default_rng(BASE_SEED + 1000 + seed)
    xshape = (batch, fin) if shared_x else (pop, batch, fin)
    x = _normal(rng, xshape)
    w = _normal(rng, (fout, fin), 1.0 / max(fin, 1))
    b = _normal(rng, (fout,), 0.01) if bias else None
    fit = _normal(rng, (pop,))
    if dtype == "bf16":
        x = round_to_bf16(x)
        w = round_to_bf16(w)
    if seeds is None:
        seeds = seed_base + np.arange(pop, dtype=np.int64)
    layer = Layer(w, b, offset, offset + fout * fin)
    shapes = [(fout, fin)] + ([(fout,)] if bias else [])
    return Workload(0, f"custom {pop}x{batch} {fin}->{fout} {dtype}", pop, batch, dtype,
                    np.asarray(seeds, dtype=np.int64), sigma, x, [layer], fit, shapes=shapes)
