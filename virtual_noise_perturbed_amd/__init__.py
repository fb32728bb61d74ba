"""Virtual-noise evolution-strategies linear layer on AMD MI355X (gfx950).

Python entry points with the signatures of the EvoX API page
``evox.triton_kernels.kernels.virtual_noise`` (entries ``compute_offsets``,
``virtual_perturbed_linear``, ``virtual_weight_gradient``,
``virtual_bias_gradient`` and ``virtual_reduce_metric``).  Each one only
checks and marshals its arguments (device, dtype, contiguity, output
allocation, the current HIP stream) and calls the C ABI of ``libvn.so``;
every step of the method runs in the library's HIP kernels.  Tensors must
live on a ROCm device: there is no CPU path.
"""

from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from . import _lib
from ._lib import VNError, VN_ACT_NONE, VN_ACT_RELU  # noqa: F401

__all__ = [
    "compute_offsets",
    "virtual_perturbed_linear",
    "virtual_perturbed_mlp",
    "virtual_weight_gradient",
    "virtual_bias_gradient",
    "virtual_flat_gradient",
    "virtual_reduce_metric",
    "virtual_reduce_metric_noalloc",
    "noise_u32",
    "noise_f32",
    "VNError",
]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require_device(name: str, t: torch.Tensor, device: Optional[torch.device] = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a ROCm GPU (got {t.device}); there is no CPU path")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _seeds(seeds: torch.Tensor, device):
    _require_device("seeds", seeds, device)
    if seeds.dim() != 1:
        raise ValueError("seeds must be 1-D (pop_size,)")
    if seeds.dtype == torch.int64:
        kind = _lib.VN_I64
    elif seeds.dtype == torch.int32:
        kind = _lib.VN_I32
    else:
        raise TypeError(f"seeds must be int64 or int32, got {seeds.dtype}")
    return seeds.contiguous(), kind


def _fitness(fitness: torch.Tensor, device):
    _require_device("fitness", fitness, device)
    if fitness.dim() != 1:
        raise ValueError("fitness must be 1-D (pop_size,)")
    if not fitness.is_floating_point():
        raise TypeError("fitness must be a floating point tensor")
    return fitness.to(torch.float32).contiguous()


def compute_offsets(param_shapes: Sequence[Sequence[int]]) -> list:
    """Starting flat offset of each parameter block (page entry
    ``compute_offsets``); computed by ``vn_compute_offsets`` on the host."""
    lib = _lib.load()
    shapes = [tuple(int(d) for d in s) for s in param_shapes]
    n = len(shapes)
    dims = [d for s in shapes for d in s]
    ndims = (ctypes.c_int32 * max(n, 1))(*[len(s) for s in shapes])
    dims_arr = (ctypes.c_int64 * max(len(dims), 1))(*dims)
    offs = (ctypes.c_int64 * max(n, 1))()
    total = ctypes.c_int64(0)
    st = lib.vn_compute_offsets(dims_arr, ndims, n, offs, ctypes.byref(total))
    _lib.check("vn_compute_offsets", st)
    return [int(offs[b]) for b in range(n)]


def virtual_perturbed_linear(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor],
                             seeds: torch.Tensor, sigma: float, offset: int,
                             activation: Optional[str] = None,
                             out: Optional[torch.Tensor] = None,
                             math: str = "default", materialize: bool = True) -> torch.Tensor:
    """``Y[i] = X[i] @ (W + sigma*N_i)^T + (b + sigma*nb_i)`` (page entry
    ``virtual_perturbed_linear``).

    x: (batch, in) shared by all individuals, or (pop, batch, in); weight (out, in)
    in the same dtype as x (float32 or bfloat16); bias (out,) or None; seeds
    (pop,) int64/int32.  Returns (pop, batch, out) float32.  ``activation`` may
    be ``"relu"`` to apply max(., 0) in the same kernel.  ``math``: ``"default"``
    (float32 operands as three bf16 matrix-core products, about 2^-16 relative
    per product) or ``"f32"`` (float32 matrix-core products; float32 only).
    ``materialize``: give the library the device workspace it asks for, so
    that large bf16 batches take the materialized-weights path (same bits;
    False keeps the noise inside the product).
    """
    lib = _lib.load()
    _require_device("weight", weight)
    dev = weight.device
    _require_device("x", x, dev)
    if weight.dim() != 2:
        raise ValueError("weight must be (out_features, in_features)")
    if x.dtype != weight.dtype:
        raise TypeError(f"x ({x.dtype}) and weight ({weight.dtype}) must share a dtype")
    if weight.dtype == torch.float32:
        dt = _lib.VN_F32
    elif weight.dtype == torch.bfloat16:
        dt = _lib.VN_BF16
    else:
        raise TypeError(f"unsupported dtype {weight.dtype} (float32 or bfloat16)")
    s, kind = _seeds(seeds, dev)
    pop = s.shape[0]
    out_f, in_f = weight.shape
    if x.dim() == 2:
        batch = x.shape[0]
        stride = 0
    elif x.dim() == 3:
        if x.shape[0] != pop:
            raise ValueError(f"x has {x.shape[0]} individuals, seeds has {pop}")
        batch = x.shape[1]
        stride = batch * in_f
    else:
        raise ValueError("x must be (batch, in) or (pop, batch, in)")
    if x.shape[-1] != in_f:
        raise ValueError("x and weight disagree on in_features")
    b = None
    if bias is not None:
        _require_device("bias", bias, dev)
        if bias.shape != (out_f,):
            raise ValueError("bias must be (out_features,)")
        b = bias.to(torch.float32).contiguous()
    act = {None: _lib.VN_ACT_NONE, "none": _lib.VN_ACT_NONE, "relu": _lib.VN_ACT_RELU}.get(activation)
    if act is None:
        raise ValueError(f"unknown activation {activation!r}")
    mm = {"default": _lib.VN_MATH_DEFAULT, "f32": _lib.VN_MATH_F32}.get(math)
    if mm is None:
        raise ValueError(f"unknown math mode {math!r}")
    xc = x.contiguous()
    wc = weight.contiguous()
    if out is None:
        y = torch.empty((pop, batch, out_f), dtype=torch.float32, device=dev)
    else:
        _require_device("out", out, dev)
        if out.shape != (pop, batch, out_f) or out.dtype != torch.float32 or not out.is_contiguous():
            raise ValueError("out must be a contiguous float32 (pop, batch, out) tensor")
        y = out
    need = ctypes.c_int64(0)
    if materialize:
        _lib.check("vn_perturbed_linear_workspace_size",
                   lib.vn_perturbed_linear_workspace_size(dt, pop, batch, in_f, out_f, mm, ctypes.byref(need)))
    ws = torch.empty((need.value,), dtype=torch.uint8, device=dev) if need.value > 0 else None
    st = lib.vn_perturbed_linear(_ptr(xc), stride, _ptr(wc), dt, _ptr(b), _ptr(s), kind,
                                 pop, batch, in_f, out_f, float(sigma), int(offset), act, mm,
                                 _ptr(y), _ptr(ws), need.value, _stream(dev))
    _lib.check("vn_perturbed_linear", st)
    return y


def virtual_perturbed_mlp(x: torch.Tensor, weights: Sequence[torch.Tensor],
                          biases: Optional[Sequence[Optional[torch.Tensor]]], seeds: torch.Tensor,
                          sigma: float, offsets: Sequence[int], activation: Optional[str] = "relu",
                          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """A chain of narrow perturbed layers in one launch: ``virtual_perturbed_linear``
    applied layer after layer (layer ``l`` with noise offset ``offsets[l]``), the
    activation between layers, the intermediate activations kept on chip.

    x: (batch, in0) shared or (pop, batch, in0); weights[l]: (out_l, in_l) in x's
    dtype with every width in 1..256; biases: None or a list of (out_l,) tensors /
    None; batch <= 64.  Returns (pop, batch, out_last) float32.
    """
    lib = _lib.load()
    n = len(weights)
    if n < 1:
        raise ValueError("at least one layer")
    dev = weights[0].device
    for t in weights:
        _require_device("weights", t, dev)
    _require_device("x", x, dev)
    dtype = weights[0].dtype
    if any(t.dtype != dtype for t in weights) or x.dtype != dtype:
        raise TypeError("x and every weight must share one dtype")
    dt = {torch.float32: _lib.VN_F32, torch.bfloat16: _lib.VN_BF16}.get(dtype)
    if dt is None:
        raise TypeError(f"unsupported dtype {dtype} (float32 or bfloat16)")
    s, kind = _seeds(seeds, dev)
    pop = s.shape[0]
    dims = [int(weights[0].shape[1])] + [int(t.shape[0]) for t in weights]
    for l, t in enumerate(weights):
        if t.dim() != 2 or int(t.shape[1]) != dims[l]:
            raise ValueError(f"weights[{l}] must be (out, {dims[l]})")
    if len(offsets) != n:
        raise ValueError("one offset per layer")
    if x.dim() == 2:
        batch, stride = x.shape[0], 0
    elif x.dim() == 3:
        if x.shape[0] != pop:
            raise ValueError(f"x has {x.shape[0]} individuals, seeds has {pop}")
        batch, stride = x.shape[1], x.shape[1] * dims[0]
    else:
        raise ValueError("x must be (batch, in) or (pop, batch, in)")
    if x.shape[-1] != dims[0]:
        raise ValueError("x and weights[0] disagree on in_features")
    bs = [None] * n if biases is None else list(biases)
    if len(bs) != n:
        raise ValueError("one bias (or None) per layer")
    bc = []
    for l, b in enumerate(bs):
        if b is None:
            bc.append(None)
            continue
        _require_device("bias", b, dev)
        if b.shape != (dims[l + 1],):
            raise ValueError(f"biases[{l}] must be ({dims[l + 1]},)")
        bc.append(b.to(torch.float32).contiguous())
    act = {None: _lib.VN_ACT_NONE, "none": _lib.VN_ACT_NONE, "relu": _lib.VN_ACT_RELU}.get(activation)
    if act is None:
        raise ValueError(f"unknown activation {activation!r}")
    wc = [t.contiguous() for t in weights]
    xc = x.contiguous()
    if out is None:
        y = torch.empty((pop, batch, dims[-1]), dtype=torch.float32, device=dev)
    else:
        _require_device("out", out, dev)
        if out.shape != (pop, batch, dims[-1]) or out.dtype != torch.float32 or not out.is_contiguous():
            raise ValueError("out must be a contiguous float32 (pop, batch, out_last) tensor")
        y = out
    dims_arr = (ctypes.c_int64 * (n + 1))(*dims)
    w_arr = (ctypes.c_void_p * n)(*[t.data_ptr() for t in wc])
    b_arr = (ctypes.c_void_p * n)(*[0 if b is None else b.data_ptr() for b in bc])
    o_arr = (ctypes.c_int64 * n)(*[int(o) for o in offsets])
    st = lib.vn_perturbed_mlp(_ptr(xc), stride, dt, n, dims_arr, w_arr, b_arr, o_arr, _ptr(s), kind, pop,
                              batch, float(sigma), act, _ptr(y), _stream(dev))
    _lib.check("vn_perturbed_mlp", st)
    return y


def _check_pop(fitness, seeds, pop_size):
    if int(pop_size) != fitness.shape[0] or int(pop_size) != seeds.shape[0]:
        raise ValueError(f"pop_size={pop_size} but len(fitness)={fitness.shape[0]}, len(seeds)={seeds.shape[0]}")


def virtual_weight_gradient(fitness: torch.Tensor, seeds: torch.Tensor, weight_shape: Sequence[int],
                            sigma: float, pop_size: int, offset: int) -> torch.Tensor:
    """``grad[j, k] = sum_i fitness_i * N_i[j, k] / (pop_size * sigma)`` (page
    entry ``virtual_weight_gradient``); returns a float32 tensor of
    ``weight_shape`` on the seeds' device."""
    lib = _lib.load()
    s, kind = _seeds(seeds, None)
    dev = s.device
    f = _fitness(fitness, dev)
    _check_pop(f, s, pop_size)
    out_f, in_f = (int(d) for d in weight_shape)
    g = torch.empty((out_f, in_f), dtype=torch.float32, device=dev)
    st = lib.vn_weight_gradient(_ptr(f), _ptr(s), kind, int(pop_size), out_f, in_f, float(sigma),
                                int(offset), _ptr(g), _stream(dev))
    _lib.check("vn_weight_gradient", st)
    return g


def virtual_bias_gradient(fitness: torch.Tensor, seeds: torch.Tensor, bias_shape: Sequence[int],
                          sigma: float, pop_size: int, offset: int) -> torch.Tensor:
    """``grad[j] = sum_i fitness_i * nb_i[j] / (pop_size * sigma)`` (page entry
    ``virtual_bias_gradient``); ``offset`` points at the bias region."""
    lib = _lib.load()
    s, kind = _seeds(seeds, None)
    dev = s.device
    f = _fitness(fitness, dev)
    _check_pop(f, s, pop_size)
    (out_f,) = (int(d) for d in bias_shape)
    g = torch.empty((out_f,), dtype=torch.float32, device=dev)
    st = lib.vn_bias_gradient(_ptr(f), _ptr(s), kind, int(pop_size), out_f, float(sigma), int(offset),
                              _ptr(g), _stream(dev))
    _lib.check("vn_bias_gradient", st)
    return g


def virtual_flat_gradient(fitness: torch.Tensor, seeds: torch.Tensor, n: int, sigma: float,
                          pop_size: int, offset: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The gradient estimator over ``n`` consecutive flat elements starting at
    ``offset`` (a whole ``compute_offsets``-chained parameter vector at once)."""
    lib = _lib.load()
    s, kind = _seeds(seeds, None)
    dev = s.device
    f = _fitness(fitness, dev)
    _check_pop(f, s, pop_size)
    if out is None:
        g = torch.empty((int(n),), dtype=torch.float32, device=dev)
    else:
        _require_device("out", out, dev)
        if out.numel() != int(n) or out.dtype != torch.float32 or not out.is_contiguous():
            raise ValueError("out must be a contiguous float32 tensor with n elements")
        g = out
    st = lib.vn_flat_gradient(_ptr(f), _ptr(s), kind, int(pop_size), int(n), float(sigma), int(offset),
                              _ptr(g), _stream(dev))
    _lib.check("vn_flat_gradient", st)
    return g


def virtual_reduce_metric(center: torch.Tensor, seeds: torch.Tensor, sigma: float, n_params: int,
                          offset: int = 0) -> torch.Tensor:
    """``fitness[i] = mean_k |center[k] + sigma * noise[i, k]|`` with the noise at
    ``offset + k`` (page entry ``virtual_reduce_metric``); (pop,) float32."""
    lib = _lib.load()
    _require_device("center", center)
    dev = center.device
    s, kind = _seeds(seeds, dev)
    if center.dim() != 1 or center.shape[0] != int(n_params):
        raise ValueError("center must be 1-D with n_params elements")
    c = center.to(torch.float32).contiguous()
    o = torch.empty((s.shape[0],), dtype=torch.float32, device=dev)
    need = ctypes.c_int64(0)
    _lib.check("vn_reduce_metric_workspace_size",
               lib.vn_reduce_metric_workspace_size(s.shape[0], int(n_params), ctypes.byref(need)))
    ws = torch.empty((need.value // 4,), dtype=torch.float32, device=dev) if need.value > 0 else None
    st = lib.vn_reduce_metric(_ptr(c), _ptr(s), kind, s.shape[0], int(n_params), float(sigma), int(offset),
                              _ptr(o), _ptr(ws), need.value, _stream(dev))
    _lib.check("vn_reduce_metric", st)
    return o


def virtual_reduce_metric_noalloc(center: torch.Tensor, seeds: torch.Tensor, sigma: float, n_params: int,
                                  offset: int = 0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``virtual_reduce_metric`` through the entry point that allocates nothing:
    its partial sums live in a fixed array on the GPU (``vn_reduce_metric_noalloc``).
    With ``out`` given, the call makes no allocation at all; calls on one GPU that
    may overlap must be ordered by the caller."""
    lib = _lib.load()
    _require_device("center", center)
    dev = center.device
    s, kind = _seeds(seeds, dev)
    if center.dim() != 1 or center.shape[0] != int(n_params):
        raise ValueError("center must be 1-D with n_params elements")
    c = center.to(torch.float32).contiguous()
    if out is None:
        o = torch.empty((s.shape[0],), dtype=torch.float32, device=dev)
    else:
        _require_device("out", out, dev)
        if out.shape != (s.shape[0],) or out.dtype != torch.float32 or not out.is_contiguous():
            raise ValueError("out must be a contiguous float32 (pop,) tensor")
        o = out
    st = lib.vn_reduce_metric_noalloc(_ptr(c), _ptr(s), kind, s.shape[0], int(n_params), float(sigma),
                                      int(offset), _ptr(o), _stream(dev))
    _lib.check("vn_reduce_metric_noalloc", st)
    return o


def noise_u32(seeds: torch.Tensor, n: int, offset: int) -> torch.Tensor:
    """(pop, n) low 32-bit hash words for indices offset + [0, n), as int32
    bit patterns (torch has no uint32 arithmetic); view with ``.numpy().view('u4')``."""
    lib = _lib.load()
    s, kind = _seeds(seeds, None)
    r = torch.empty((s.shape[0], int(n)), dtype=torch.int32, device=s.device)
    st = lib.vn_noise_u32(_ptr(s), kind, s.shape[0], int(n), int(offset), _ptr(r), _stream(s.device))
    _lib.check("vn_noise_u32", st)
    return r


def noise_f32(seeds: torch.Tensor, n: int, offset: int) -> torch.Tensor:
    """(pop, n) centered-uniform noise in [-0.5, 0.5) for indices offset + [0, n)."""
    lib = _lib.load()
    s, kind = _seeds(seeds, None)
    r = torch.empty((s.shape[0], int(n)), dtype=torch.float32, device=s.device)
    st = lib.vn_noise_f32(_ptr(s), kind, s.shape[0], int(n), int(offset), _ptr(r), _stream(s.device))
    _lib.check("vn_noise_f32", st)
    return r
