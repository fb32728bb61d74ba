"""Plant plausible mistakes in the oracle (on the CPU) and require that the
pins catch every one of them.  Each mutation patches one function of
``oracle.vn_oracle`` for the duration of a test."""

import numpy as np
import pytest

import oracle.vn_oracle as vo
import pins

_real_finalize = vo.splitmix_finalize
_real_initial_state = vo.initial_state
_real_from_bits = vo.noise_from_bits
_real_noise_at = vo.noise_at


def _finalize_wrong_shift(z, m1=vo.GAMMA, m2=vo.GAMMA):
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(31))) * np.uint64(m1)   # 30 -> 31
        z = (z ^ (z >> np.uint64(27))) * np.uint64(m2)
        return z ^ (z >> np.uint64(31))


def _finalize_missing_last_xorshift(z, m1=vo.GAMMA, m2=vo.GAMMA):
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(m1)
        return (z ^ (z >> np.uint64(27))) * np.uint64(m2)


def _finalize_canonical_constants(z, m1=vo.GAMMA, m2=vo.GAMMA):
    if m1 == vo.GAMMA:
        m1, m2 = vo.CANONICAL_M1, vo.CANONICAL_M2
    return _real_finalize(z, m1, m2)


def _state_without_plus_one(seeds, idx):
    # mistake: z0 = s + idx*GAMMA (index 0 would reuse the seed state)
    with np.errstate(over="ignore"):
        return _real_initial_state(seeds, idx) - np.uint64(vo.GAMMA)


def _state_xor(seeds, idx):
    s = vo.canonical_seeds(seeds)
    idx = np.asarray(idx, dtype=np.int64).reshape(-1)
    with np.errstate(over="ignore"):
        return s[:, None] ^ ((idx.astype(np.uint64) + np.uint64(1)) * np.uint64(vo.GAMMA))[None, :]


def _from_bits_23bit(r):
    r = np.asarray(r, dtype=np.uint32).astype(np.int64)
    return (r >> 9).astype(np.float64) * 2.0 ** -23 - 0.5


def _from_bits_sign_flip(r):
    return -_real_from_bits(r)


def _from_bits_float_scale(r):
    r = np.asarray(r, dtype=np.uint32).astype(np.float64)
    return r * 2.0 ** -32 - 0.5


def _noise_at_transposed(seeds, idx):
    # uses index (k*out + j) order by reversing each row's layout: mimics a transposed noise matrix
    n = _real_noise_at(seeds, idx)
    return n[:, ::-1].copy()


MUTATIONS = [
    ("splitmix_finalize", _finalize_wrong_shift),
    ("splitmix_finalize", _finalize_missing_last_xorshift),
    ("splitmix_finalize", _finalize_canonical_constants),
    ("initial_state", _state_without_plus_one),
    ("initial_state", _state_xor),
    ("noise_from_bits", _from_bits_23bit),
    ("noise_from_bits", _from_bits_sign_flip),
    ("noise_from_bits", _from_bits_float_scale),
    ("noise_at", _noise_at_transposed),
]


def _run_all():
    failed = []
    for check in pins.ALL_CHECKS:
        if check is pins.check_range_and_statistics:
            continue  # slow and not aimed at structural mistakes
        try:
            check()
        except AssertionError:
            failed.append(check.__name__)
    return failed


@pytest.mark.parametrize("name,fn", MUTATIONS, ids=[f"{n}:{f.__name__}" for n, f in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(vo, name, fn)
    assert _run_all(), f"no pin caught the planted mistake {fn.__name__}"


def _forward_untransposed(x, weight, bias, seeds, sigma, offset):
    w = np.asarray(weight, dtype=np.float64)
    out_f, in_f = w.shape
    s = vo.canonical_seeds(seeds)
    xs = vo._per_individual_x(x, s.shape[0])
    y = np.empty((s.shape[0], xs.shape[1], out_f))
    for i in range(s.shape[0]):
        # mistake: noise laid out as (in, out) then transposed
        n_i = vo.noise_at(s[i:i + 1], offset + np.arange(out_f * in_f))[0].reshape(in_f, out_f).T
        y[i] = xs[i] @ (w + sigma * n_i).T
        if bias is not None:
            y[i] += np.asarray(bias) + sigma * vo.noise_at(s[i:i + 1], offset + out_f * in_f + np.arange(out_f))[0]
    return y


def _forward_bias_index_off(x, weight, bias, seeds, sigma, offset):
    w = np.asarray(weight, dtype=np.float64)
    out_f, in_f = w.shape
    s = vo.canonical_seeds(seeds)
    xs = vo._per_individual_x(x, s.shape[0])
    y = np.empty((s.shape[0], xs.shape[1], out_f))
    for i in range(s.shape[0]):
        n_i = vo.noise_at(s[i:i + 1], offset + np.arange(out_f * in_f))[0].reshape(out_f, in_f)
        y[i] = xs[i] @ (w + sigma * n_i).T
        if bias is not None:
            # mistake: bias noise taken at offset + j instead of offset + out*in + j
            y[i] += np.asarray(bias) + sigma * vo.noise_at(s[i:i + 1], offset + np.arange(out_f))[0]
    return y


FORWARD_MUTATIONS = [_forward_untransposed, _forward_bias_index_off]


@pytest.mark.parametrize("fn", FORWARD_MUTATIONS, ids=lambda f: f.__name__)
def test_planted_forward_mistake_is_caught(monkeypatch, fn):
    monkeypatch.setattr(vo, "perturbed_linear", fn)
    assert _run_all()


def test_planted_gradient_scale_mistake_is_caught(monkeypatch):
    real = vo.weight_gradient
    monkeypatch.setattr(vo, "weight_gradient",
                        lambda f, s, shp, sig, p, off: real(f, s, shp, sig, p, off) * p)
    assert _run_all()


def _metric_without_abs(center, seeds, sigma, n_params, offset=0):
    c = np.asarray(center, dtype=np.float64).reshape(-1)
    s = vo.canonical_seeds(seeds)
    return np.array([np.mean(c + sigma * vo.noise(s[i:i + 1].view(np.int64), n_params, offset)[0])
                     for i in range(s.shape[0])])


def _metric_sum_not_mean(center, seeds, sigma, n_params, offset=0):
    c = np.asarray(center, dtype=np.float64).reshape(-1)
    s = vo.canonical_seeds(seeds)
    return np.array([np.sum(np.abs(c + sigma * vo.noise(s[i:i + 1].view(np.int64), n_params, offset)[0]))
                     for i in range(s.shape[0])])


def _metric_offset_ignored(center, seeds, sigma, n_params, offset=0):
    c = np.asarray(center, dtype=np.float64).reshape(-1)
    s = vo.canonical_seeds(seeds)
    return np.array([np.mean(np.abs(c + sigma * vo.noise(s[i:i + 1].view(np.int64), n_params, 0)[0]))
                     for i in range(s.shape[0])])


def _bias_gradient_forward_offsets(fitness, seeds, bias_shape, sigma, pop_size, offset):
    # mistake: `offset` treated as a weight offset and moved past a weight block (here one of
    # out x out elements) before the bias noise is read, where the bias gradient takes the
    # bias-region offset itself
    (out_f,) = bias_shape
    f = np.asarray(fitness, dtype=np.float64)
    n = vo.noise_at(seeds, offset + out_f * out_f + np.arange(out_f))
    return (f @ n) / (pop_size * sigma)


def _weight_gradient_transposed(fitness, seeds, weight_shape, sigma, pop_size, offset):
    out_f, in_f = weight_shape
    f = np.asarray(fitness, dtype=np.float64)
    n = vo.noise_at(seeds, offset + np.arange(out_f * in_f))
    return ((f @ n) / (pop_size * sigma)).reshape(in_f, out_f).T.copy()


def _offsets_inclusive(param_shapes):
    out, acc = [], 0
    for shp in param_shapes:
        acc += int(np.prod(shp)) if len(shp) else 1
        out.append(acc)
    return out


MORE_MUTATIONS = [
    ("reduce_metric", _metric_without_abs),
    ("reduce_metric", _metric_sum_not_mean),
    ("reduce_metric", _metric_offset_ignored),
    ("bias_gradient", _bias_gradient_forward_offsets),
    ("weight_gradient", _weight_gradient_transposed),
    ("compute_offsets", _offsets_inclusive),
]


@pytest.mark.parametrize("name,fn", MORE_MUTATIONS, ids=[f"{n}:{f.__name__}" for n, f in MORE_MUTATIONS])
def test_planted_api_mistake_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(vo, name, fn)
    assert _run_all(), f"no pin caught the planted mistake {fn.__name__}"
