"""Plain numpy oracle of the virtual-noise ES linear layer (test infrastructure only).

Everything here follows the EvoX API documentation page
``evox.triton_kernels.kernels.virtual_noise`` and is written for a reader to
check against it by eye: integers are ``numpy.uint64`` (products wrap mod
2**64), floating point is float64 from the exact input values, and the noise
is materialized one individual at a time, as the page's entry
``virtual_perturbed_linear`` says its CPU fallback does.

Readings of the page (where it is silent or loose) that fix the bit patterns:

A1  state: ``z0 = s + (idx + 1) * GAMMA  (mod 2**64)``.  This is the idx-th
    output (0-based) of the textbook splitmix64 sequence seeded with ``s``;
    the page says only that the value comes from a splitmix64 hash of
    (seed, element index).
A2  finalizer multipliers: GAMMA in both rounds, as the page's
    ``_splitmix64_step`` entry prints the formula (the word "canonical" there
    is read loosely; the textbook finalizer uses two other constants, kept
    here only as ``CANONICAL_M1/M2`` for pinning the structure).
A3  uint32 -> u: ``u = (r >> 8) * 2**-24``, exact in fp32 and strictly below
    1, so the page's half-open range [-0.5, 0.5) holds for every draw.
A4  seeds are two's-complement int64 reinterpreted as uint64 (int32 seeds are
    sign-extended first); negative seeds are legal.
A5  ``bias=None`` means no bias term and no bias noise; a zero bias tensor
    still receives ``sigma * nb_i``.
"""

from __future__ import annotations

import numpy as np

# Page entry ``_SPLITMIX64_GAMMA``: 11400714819323198485 (= 0x9E3779B97F4A7C15).
GAMMA = 11400714819323198485
# Textbook splitmix64 finalizer multipliers (Steele, Lea & Flood, "Fast
# splittable pseudorandom number generators", OOPSLA 2014, variant used by
# Vigna's splitmix64.c).  Not used by the method; only for pinning structure.
CANONICAL_M1 = 0xBF58476D1CE4E5B9
CANONICAL_M2 = 0x94D049BB133111EB

_MASK32 = np.uint64(0xFFFFFFFF)


def _u64(v) -> np.ndarray:
    return np.asarray(v, dtype=np.uint64)


def splitmix_finalize(z, m1: int = GAMMA, m2: int = GAMMA) -> np.ndarray:
    """Page entry ``_splitmix64_step``: two xor-shift/multiply rounds, then a
    final xor-shift, all mod 2**64 with logical shifts (uint64 shifts are
    logical, which is what the page's ``_cpu_logical_rshift`` emulates on
    signed int64)."""
    z = _u64(z)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(m1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(m2)
        z = z ^ (z >> np.uint64(31))
    return z


def canonical_seeds(seeds) -> np.ndarray:
    """Reading A4: int seeds -> uint64 two's-complement bit patterns."""
    s = np.asarray(seeds)
    if s.ndim != 1:
        raise ValueError("seeds must be 1-D")
    if not np.issubdtype(s.dtype, np.integer):
        raise TypeError("seeds must be an integer array")
    if s.dtype == np.uint64:
        return s
    return s.astype(np.int64).view(np.uint64)


def initial_state(seeds, idx) -> np.ndarray:
    """Reading A1: ``z0[i, t] = s_i + (idx_t + 1) * GAMMA  (mod 2**64)``.

    ``idx`` are absolute element indices (offset + flat index, page section
    "Noise indexing scheme"); they must be non-negative.
    """
    s = canonical_seeds(seeds)
    idx = np.asarray(idx, dtype=np.int64).reshape(-1)
    if idx.size and idx.min() < 0:
        raise ValueError("element indices must be non-negative")
    with np.errstate(over="ignore"):
        step = (idx.astype(np.uint64) + np.uint64(1)) * np.uint64(GAMMA)
        return s[:, None] + step[None, :]


def noise_bits_at(seeds, idx, m1: int = GAMMA, m2: int = GAMMA) -> np.ndarray:
    """Full 64-bit finalizer output for every (seed, index) pair: (P, len(idx))."""
    return splitmix_finalize(initial_state(seeds, idx), m1, m2)


def noise_u32_at(seeds, idx) -> np.ndarray:
    """Page entry ``_cpu_normal_noise``: the low 32 bits of the splitmix64
    hash, as uint32, shape (P, len(idx))."""
    return (noise_bits_at(seeds, idx) & _MASK32).astype(np.uint32)


def noise_from_bits(r_u32) -> np.ndarray:
    """Reading A3 and page section "RNG: fast centered-uniform approximation":
    ``u = (r >> 8) * 2**-24`` in [0, 1), noise ``= u - 0.5`` in [-0.5, 0.5)."""
    r = np.asarray(r_u32, dtype=np.uint32).astype(np.int64)
    u = (r >> 8).astype(np.float64) * 2.0 ** -24
    return u - 0.5


def noise_u32(seeds, n_elements: int, offset: int) -> np.ndarray:
    """(P, n) uint32 words for indices ``offset + [0, n)`` (page entry
    ``_cpu_normal_noise``: element index = offset + flat_index)."""
    return noise_u32_at(seeds, offset + np.arange(int(n_elements), dtype=np.int64))


def noise_at(seeds, idx) -> np.ndarray:
    """(P, len(idx)) float64 centered-uniform noise at absolute indices."""
    return noise_from_bits(noise_u32_at(seeds, idx))


def noise(seeds, n_elements: int, offset: int) -> np.ndarray:
    """Mirror of the page's ``_cpu_normal_noise(seeds, n_elements, offset)``:
    (P, n) noise in [-0.5, 0.5) (float64 here; every value is exact in fp32)."""
    return noise_at(seeds, offset + np.arange(int(n_elements), dtype=np.int64))


def compute_offsets(param_shapes) -> list[int]:
    """Page entry ``compute_offsets``: the starting flat offset of each block is
    the element count of all preceding blocks; a block holds prod(shape)
    elements (an empty shape is a scalar, one element)."""
    offsets = []
    running = 0
    for shape in param_shapes:
        offsets.append(running)
        count = 1
        for d in shape:
            d = int(d)
            if d < 0:
                raise ValueError("negative dimension")
            count *= d
        running += count
    return offsets


def _per_individual_x(x, pop: int) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    if x.ndim == 2:  # (batch, in), shared by every individual
        return np.broadcast_to(x, (pop,) + x.shape)
    if x.ndim == 3 and x.shape[0] == pop:
        return x
    raise ValueError("x must be (batch, in) or (pop, batch, in)")


def perturbed_linear(x, weight, bias, seeds, sigma: float, offset: int) -> np.ndarray:
    """Page entry ``virtual_perturbed_linear`` and the module's model equation:
    ``Y[i] = X[i] @ (W + sigma*N_i)^T + (b + sigma*nb_i)``.

    Weight element (j, k) takes the noise at ``offset + j*in + k``, bias element
    j the noise at ``offset + out*in + j`` (section "Noise indexing scheme").
    Returns (pop, batch, out) float64.
    """
    s = canonical_seeds(seeds)
    pop = s.shape[0]
    w = np.asarray(weight, dtype=np.float64)
    out_f, in_f = w.shape
    xs = _per_individual_x(x, pop)
    if xs.shape[2] != in_f:
        raise ValueError("x and weight disagree on in_features")
    y = np.empty((pop, xs.shape[1], out_f), dtype=np.float64)
    w_idx = offset + np.arange(out_f * in_f, dtype=np.int64)
    b_idx = offset + out_f * in_f + np.arange(out_f, dtype=np.int64)
    for i in range(pop):
        n_i = noise_at(s[i:i + 1], w_idx)[0].reshape(out_f, in_f)
        w_i = w + sigma * n_i
        y[i] = xs[i] @ w_i.T
        if bias is not None:
            nb_i = noise_at(s[i:i + 1], b_idx)[0]
            y[i] += np.asarray(bias, dtype=np.float64) + sigma * nb_i
    return y


def perturbed_linear_at(x, weight, bias, seeds, sigma: float, offset: int,
                        ii, bb, jj) -> np.ndarray:
    """The same model evaluated only at the output elements Y[ii[t], bb[t], jj[t]]
    (one row of noise per sample), for checking very large workloads."""
    s = canonical_seeds(seeds)
    pop = s.shape[0]
    w = np.asarray(weight)
    out_f, in_f = w.shape
    xs = np.asarray(x)
    shared = xs.ndim == 2
    ks = np.arange(in_f, dtype=np.int64)
    res = np.empty(len(ii), dtype=np.float64)
    for t, (i, b, j) in enumerate(zip(ii, bb, jj)):
        i, b, j = int(i), int(b), int(j)
        if not (0 <= i < pop):
            raise IndexError("individual out of range")
        n_row = noise_at(s[i:i + 1], offset + j * in_f + ks)[0]
        x_row = np.asarray(xs[b] if shared else xs[i, b], dtype=np.float64)
        w_row = np.asarray(w[j], dtype=np.float64) + sigma * n_row
        val = float(np.dot(x_row, w_row))
        if bias is not None:
            nb = noise_at(s[i:i + 1], [offset + out_f * in_f + j])[0, 0]
            val += float(np.asarray(bias, dtype=np.float64)[j]) + sigma * nb
        res[t] = val
    return res


def _check_pop(fitness, seeds, pop_size: int):
    f = np.asarray(fitness, dtype=np.float64).reshape(-1)
    s = canonical_seeds(seeds)
    if not (f.shape[0] == s.shape[0] == int(pop_size)):
        raise ValueError("pop_size must equal len(fitness) and len(seeds)")
    if int(pop_size) <= 0:
        raise ValueError("pop_size must be positive")
    return f, s


def weight_gradient(fitness, seeds, weight_shape, sigma: float, pop_size: int,
                    offset: int) -> np.ndarray:
    """Page entry ``virtual_weight_gradient`` / the module's gradient equation:
    ``grad[j, k] = sum_i fitness_i * N_i[j, k] / (pop_size * sigma)`` with the
    weight noise at ``offset + j*in + k``."""
    f, s = _check_pop(fitness, seeds, pop_size)
    n = int(np.prod(weight_shape, dtype=np.int64))
    noise_mat = noise(s.view(np.int64), n, offset)  # (pop, n)
    g = (f @ noise_mat) / (pop_size * sigma)
    return g.reshape(tuple(weight_shape))


def weight_gradient_at(fitness, seeds, sigma: float, pop_size: int, offset: int,
                       flat_index) -> np.ndarray:
    """The same estimator at chosen flat elements only (any block shape)."""
    f, s = _check_pop(fitness, seeds, pop_size)
    idx = offset + np.asarray(flat_index, dtype=np.int64).reshape(-1)
    noise_mat = noise_at(s.view(np.int64), idx)
    return (f @ noise_mat) / (pop_size * sigma)


def bias_gradient(fitness, seeds, bias_shape, sigma: float, pop_size: int,
                  offset: int) -> np.ndarray:
    """Page entry ``virtual_bias_gradient``:
    ``grad[j] = sum_i fitness_i * nb_i[j] / (pop_size * sigma)``, where
    ``offset`` already points at the bias region (weight offset + out*in)."""
    f, s = _check_pop(fitness, seeds, pop_size)
    n = int(np.prod(bias_shape, dtype=np.int64))
    noise_mat = noise(s.view(np.int64), n, offset)
    g = (f @ noise_mat) / (pop_size * sigma)
    return g.reshape(tuple(bias_shape))


def reduce_metric(center, seeds, sigma: float, n_params: int, offset: int = 0) -> np.ndarray:
    """Page entry ``virtual_reduce_metric``:
    ``fitness[i] = mean_k |center[k] + sigma * noise[i, k]|`` with the noise at
    ``offset + k``.  Returns (pop,) float64."""
    c = np.asarray(center, dtype=np.float64).reshape(-1)
    if c.shape[0] != int(n_params) or int(n_params) <= 0:
        raise ValueError("n_params must equal center.numel() and be positive")
    s = canonical_seeds(seeds)
    out = np.empty(s.shape[0], dtype=np.float64)
    for i in range(s.shape[0]):
        n_i = noise(s[i:i + 1].view(np.int64), n_params, offset)[0]
        out[i] = np.mean(np.abs(c + sigma * n_i))
    return out
