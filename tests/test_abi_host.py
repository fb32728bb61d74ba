"""Host-side checks of the C ABI: no GPU work is ever launched here.

Every call below either fails validation (which happens before any HIP call)
or has a zero extent (which returns without a launch), so fake pointers are
never dereferenced.
"""

import ctypes
import os
import re

import pytest

from virtual_noise_perturbed_amd import _lib
import virtual_noise_perturbed_amd as vn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vn.h")

FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: every call with it must fail validation
NULL = None


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vn_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert "vn_perturbed_linear" in names and "vn_weight_gradient" in names
    for name in names:
        assert hasattr(lib, name), f"{name} declared in vn.h but not exported"
    # and the binding knows every one of them
    assert set(names) == set(_lib.SIGNATURES)


def test_abi_version_and_status_strings(lib):
    text = open(HEADER).read()
    ver = int(re.search(r"#define VN_ABI_VERSION (\d+)", text).group(1))
    assert lib.vn_abi_version() == ver
    for code in range(8):
        assert lib.vn_status_string(code).decode() not in ("", "unknown status")
    assert lib.vn_status_string(99).decode() == "unknown status"


def test_compute_offsets_page_example():
    # page entry compute_offsets, its printed example
    assert vn.compute_offsets([(256, 784), (256,), (10, 256), (10,)]) == [0, 200704, 200960, 203520]
    assert vn.compute_offsets([(256, 784), (256,), (256, 256), (256,), (10, 256), (10,)]) == \
        [0, 200704, 200960, 266496, 266752, 269312]
    assert vn.compute_offsets([]) == []
    assert vn.compute_offsets([(), (3,), (2, 2)]) == [0, 1, 4]


def test_compute_offsets_errors(lib):
    i64 = ctypes.c_int64
    out = (i64 * 2)()
    dims = (i64 * 2)(2**62, 2**62)
    nd = (ctypes.c_int32 * 2)(1, 1)
    assert lib.vn_compute_offsets(dims, nd, 2, out, None) == _lib.VN_ERR_OVERFLOW   # sum = 2^63
    nd2 = (ctypes.c_int32 * 1)(2)
    assert lib.vn_compute_offsets(dims, nd2, 1, out, None) == _lib.VN_ERR_OVERFLOW  # product = 2^124
    dims = (i64 * 2)(3, -1)
    assert lib.vn_compute_offsets(dims, nd, 2, out, None) == _lib.VN_ERR_SHAPE
    assert lib.vn_compute_offsets(dims, nd, -1, out, None) == _lib.VN_ERR_SHAPE
    assert lib.vn_compute_offsets(dims, None, 2, out, None) == _lib.VN_ERR_NULL
    nd_bad = (ctypes.c_int32 * 2)(1, -2)
    assert lib.vn_compute_offsets(dims, nd_bad, 2, out, None) == _lib.VN_ERR_SHAPE
    assert lib.vn_compute_offsets(None, None, 0, None, None) == _lib.VN_OK
    with pytest.raises(ValueError):
        vn.compute_offsets([(2**40, 2**40)])


def fwd(lib, **kw):
    a = dict(x=FAKE, stride=0, w=FAKE, dtype=_lib.VN_F32, b=NULL, seeds=FAKE, sdt=_lib.VN_I64, pop=4,
             batch=2, i=8, o=3, sigma=0.1, offset=0, act=0, math=0, y=FAKE, ws=NULL, ws_bytes=0, stream=NULL)
    a.update(kw)
    return lib.vn_perturbed_linear(a["x"], a["stride"], a["w"], a["dtype"], a["b"], a["seeds"], a["sdt"],
                                   a["pop"], a["batch"], a["i"], a["o"], a["sigma"], a["offset"], a["act"],
                                   a["math"], a["y"], a["ws"], a["ws_bytes"], a["stream"])


def test_forward_validation(lib):
    E = _lib
    assert fwd(lib, dtype=7) == E.VN_ERR_DTYPE
    assert fwd(lib, sdt=5) == E.VN_ERR_DTYPE
    assert fwd(lib, pop=-1) == E.VN_ERR_SHAPE
    assert fwd(lib, batch=-1) == E.VN_ERR_SHAPE
    assert fwd(lib, i=-1) == E.VN_ERR_SHAPE
    assert fwd(lib, o=-1) == E.VN_ERR_SHAPE
    assert fwd(lib, stride=5) == E.VN_ERR_SHAPE          # neither 0 nor batch*in
    assert fwd(lib, sigma=float("nan")) == E.VN_ERR_VALUE
    assert fwd(lib, sigma=float("inf")) == E.VN_ERR_VALUE
    assert fwd(lib, offset=-1) == E.VN_ERR_VALUE
    assert fwd(lib, act=9) == E.VN_ERR_VALUE
    assert fwd(lib, math=5) == E.VN_ERR_VALUE
    assert fwd(lib, math=E.VN_MATH_F32, dtype=E.VN_BF16) == E.VN_ERR_VALUE   # exact fp32 math needs fp32 operands
    assert fwd(lib, offset=2**63 - 20) == E.VN_ERR_OVERFLOW   # offset + out*in + out > INT64_MAX
    assert fwd(lib, o=2**40, i=2**40) == E.VN_ERR_OVERFLOW
    assert fwd(lib, y=NULL) == E.VN_ERR_NULL
    assert fwd(lib, seeds=NULL) == E.VN_ERR_NULL
    assert fwd(lib, x=NULL) == E.VN_ERR_NULL
    assert fwd(lib, w=NULL) == E.VN_ERR_NULL
    assert fwd(lib, y=ctypes.c_void_p(0x10002)) == E.VN_ERR_ALIGN
    assert fwd(lib, seeds=ctypes.c_void_p(0x10004)) == E.VN_ERR_ALIGN
    assert fwd(lib, x=ctypes.c_void_p(0x10002)) == E.VN_ERR_ALIGN
    assert fwd(lib, ws=FAKE, ws_bytes=-1) == E.VN_ERR_SHAPE
    assert fwd(lib, ws=ctypes.c_void_p(0x10008), ws_bytes=64) == E.VN_ERR_ALIGN   # workspace not 16-byte aligned
    # zero extents: nothing to do, nothing launched, even with NULL outputs
    assert fwd(lib, pop=0, y=NULL, x=NULL, w=NULL, seeds=NULL) == E.VN_OK
    assert fwd(lib, batch=0, y=NULL) == E.VN_OK
    assert fwd(lib, o=0, y=NULL) == E.VN_OK


def grad(lib, fn, **kw):
    a = dict(f=FAKE, seeds=FAKE, sdt=_lib.VN_I64, pop=4, n=6, sigma=0.1, offset=0, out=FAKE)
    a.update(kw)
    if fn == "flat":
        return lib.vn_flat_gradient(a["f"], a["seeds"], a["sdt"], a["pop"], a["n"], a["sigma"], a["offset"],
                                    a["out"], None)
    if fn == "bias":
        return lib.vn_bias_gradient(a["f"], a["seeds"], a["sdt"], a["pop"], a["n"], a["sigma"], a["offset"],
                                    a["out"], None)
    return lib.vn_weight_gradient(a["f"], a["seeds"], a["sdt"], a["pop"], a["n"], 3, a["sigma"], a["offset"],
                                  a["out"], None)


@pytest.mark.parametrize("fn", ["flat", "bias", "weight"])
def test_gradient_validation(lib, fn):
    E = _lib
    assert grad(lib, fn, sdt=3) == E.VN_ERR_DTYPE
    assert grad(lib, fn, n=-1) == E.VN_ERR_SHAPE
    assert grad(lib, fn, pop=0) == E.VN_ERR_VALUE
    assert grad(lib, fn, pop=-3) == E.VN_ERR_VALUE
    assert grad(lib, fn, sigma=0.0) == E.VN_ERR_VALUE      # the estimator divides by sigma
    assert grad(lib, fn, sigma=float("nan")) == E.VN_ERR_VALUE
    assert grad(lib, fn, sigma=1e-45) == E.VN_ERR_VALUE    # 1/(pop*sigma) overflows fp32
    assert grad(lib, fn, offset=-5) == E.VN_ERR_VALUE
    assert grad(lib, fn, offset=2**63 - 2) == E.VN_ERR_OVERFLOW
    assert grad(lib, fn, f=NULL) == E.VN_ERR_NULL
    assert grad(lib, fn, seeds=NULL) == E.VN_ERR_NULL
    assert grad(lib, fn, out=NULL) == E.VN_ERR_NULL
    assert grad(lib, fn, out=ctypes.c_void_p(0x10001)) == E.VN_ERR_ALIGN
    assert grad(lib, fn, n=0, out=NULL) == E.VN_OK


def test_metric_and_noise_validation(lib):
    E = _lib
    m = lambda **kw: lib.vn_reduce_metric(kw.get("c", FAKE), kw.get("s", FAKE), kw.get("sdt", 0),
                                          kw.get("pop", 3), kw.get("n", 5), kw.get("sigma", 0.1),
                                          kw.get("offset", 0), kw.get("out", FAKE), kw.get("ws", NULL),
                                          kw.get("ws_bytes", 0), None)
    assert m(sdt=4) == E.VN_ERR_DTYPE
    assert m(pop=-1) == E.VN_ERR_SHAPE
    assert m(n=0) == E.VN_ERR_SHAPE
    assert m(ws_bytes=-4) == E.VN_ERR_SHAPE
    assert m(sigma=float("inf")) == E.VN_ERR_VALUE
    assert m(offset=-1) == E.VN_ERR_VALUE
    assert m(c=NULL) == E.VN_ERR_NULL
    assert m(ws=ctypes.c_void_p(0x10002), ws_bytes=64) == E.VN_ERR_ALIGN
    assert m(pop=0, c=NULL, out=NULL) == E.VN_OK
    # a small population over a long vector splits into segments and needs the workspace
    need = ctypes.c_int64(-1)
    assert lib.vn_reduce_metric_workspace_size(3, 600001, ctypes.byref(need)) == E.VN_OK
    assert 0 < need.value <= 6 * 1024 and need.value % 4 == 0
    assert m(n=600001) == E.VN_ERR_NULL
    assert m(n=600001, ws=FAKE, ws_bytes=need.value - 4) == E.VN_ERR_SHAPE
    for pop, n in [(512, 10**7), (3, 5), (1, 131071), (0, 10**6), (5, 0)]:
        assert lib.vn_reduce_metric_workspace_size(pop, n, ctypes.byref(need)) == E.VN_OK
        assert need.value == 0, (pop, n)
    worst = 0
    for pop in range(1, 512):
        for n in (131072, 10**6, 2**31):
            assert lib.vn_reduce_metric_workspace_size(pop, n, ctypes.byref(need)) == E.VN_OK
            worst = max(worst, need.value)
    assert worst <= 1535 * 4
    assert lib.vn_reduce_metric_workspace_size(-1, 5, ctypes.byref(need)) == E.VN_ERR_SHAPE
    assert lib.vn_reduce_metric_workspace_size(1, 5, None) == E.VN_ERR_NULL
    # the allocation-free variant validates the same way before any HIP call
    na = lambda **kw: lib.vn_reduce_metric_noalloc(kw.get("c", FAKE), kw.get("s", FAKE), kw.get("sdt", 0),
                                                   kw.get("pop", 3), kw.get("n", 5), kw.get("sigma", 0.1),
                                                   kw.get("offset", 0), kw.get("out", FAKE), None)
    assert na(sdt=4) == E.VN_ERR_DTYPE
    assert na(pop=-1) == E.VN_ERR_SHAPE
    assert na(n=0) == E.VN_ERR_SHAPE
    assert na(sigma=float("nan")) == E.VN_ERR_VALUE
    assert na(offset=-1) == E.VN_ERR_VALUE
    assert na(offset=2**63 - 2) == E.VN_ERR_OVERFLOW
    assert na(out=NULL) == E.VN_ERR_NULL
    assert na(c=ctypes.c_void_p(0x10002)) == E.VN_ERR_ALIGN
    assert na(pop=0, c=NULL, out=NULL) == E.VN_OK
    nz = lambda **kw: lib.vn_noise_u32(kw.get("s", FAKE), kw.get("sdt", 0), kw.get("pop", 2), kw.get("n", 4),
                                       kw.get("offset", 0), kw.get("out", FAKE), None)
    assert nz(sdt=2) == E.VN_ERR_DTYPE
    assert nz(n=-4) == E.VN_ERR_SHAPE
    assert nz(offset=-4) == E.VN_ERR_VALUE
    assert nz(out=NULL) == E.VN_ERR_NULL
    assert nz(s=ctypes.c_void_p(0x10004)) == E.VN_ERR_ALIGN
    assert nz(n=0, out=NULL) == E.VN_OK
    assert lib.vn_noise_f32(FAKE, 0, 2, 4, 2**63 - 1, FAKE, None) == E.VN_ERR_OVERFLOW


def mlp(lib, **kw):
    a = dict(x=FAKE, stride=0, dtype=_lib.VN_F32, dims=[8, 6, 4], w=[FAKE, FAKE], b=None, offsets=[0, 100],
             seeds=FAKE, sdt=_lib.VN_I64, pop=3, batch=5, sigma=0.1, act=_lib.VN_ACT_RELU, y=FAKE)
    a.update(kw)
    n = kw.get("n", 2)
    dims = None if a["dims"] is None else (ctypes.c_int64 * len(a["dims"]))(*a["dims"])
    w = None if a["w"] is None else (ctypes.c_void_p * len(a["w"]))(*[None if p is None else p.value for p in a["w"]])
    b = None if a["b"] is None else (ctypes.c_void_p * len(a["b"]))(*[None if p is None else p.value for p in a["b"]])
    offs = None if a["offsets"] is None else (ctypes.c_int64 * len(a["offsets"]))(*a["offsets"])
    return lib.vn_perturbed_mlp(a["x"], a["stride"], a["dtype"], n, dims, w, b, offs, a["seeds"], a["sdt"],
                                a["pop"], a["batch"], a["sigma"], a["act"], a["y"], None)


def test_mlp_validation(lib):
    """Every call fails validation or has a zero extent: nothing is launched."""
    E = _lib
    assert mlp(lib, dtype=9) == E.VN_ERR_DTYPE
    assert mlp(lib, sdt=9) == E.VN_ERR_DTYPE
    assert mlp(lib, n=0) == E.VN_ERR_SHAPE
    assert mlp(lib, n=9, dims=[4] * 10, w=[FAKE] * 9, offsets=[0] * 9) == E.VN_ERR_SHAPE
    assert mlp(lib, dims=[8, 257, 4]) == E.VN_ERR_SHAPE          # output widths are at most 256
    assert mlp(lib, dims=[8, 4, 257]) == E.VN_ERR_SHAPE
    assert mlp(lib, dims=[0, 4, 4]) == E.VN_ERR_SHAPE
    assert mlp(lib, dims=[2**62, 4, 4]) == E.VN_ERR_OVERFLOW     # batch * dims[0] overflows
    assert mlp(lib, dims=[8, 0, 4]) == E.VN_ERR_SHAPE
    assert mlp(lib, batch=65) == E.VN_ERR_SHAPE                  # batches are at most 64
    assert mlp(lib, pop=-1) == E.VN_ERR_SHAPE
    assert mlp(lib, stride=7) == E.VN_ERR_SHAPE                  # neither 0 nor batch*dims[0]
    assert mlp(lib, dims=None) == E.VN_ERR_NULL
    assert mlp(lib, w=None) == E.VN_ERR_NULL
    assert mlp(lib, offsets=None) == E.VN_ERR_NULL
    assert mlp(lib, sigma=float("nan")) == E.VN_ERR_VALUE
    assert mlp(lib, sigma=2.0 ** -110) == E.VN_ERR_VALUE         # sigma * 2^-24 would be subnormal
    assert mlp(lib, act=4) == E.VN_ERR_VALUE
    assert mlp(lib, offsets=[0, -1]) == E.VN_ERR_VALUE
    assert mlp(lib, offsets=[0, 2**63 - 10]) == E.VN_ERR_OVERFLOW
    assert mlp(lib, x=NULL) == E.VN_ERR_NULL
    assert mlp(lib, y=NULL) == E.VN_ERR_NULL
    assert mlp(lib, seeds=NULL) == E.VN_ERR_NULL
    assert mlp(lib, w=[FAKE, None]) == E.VN_ERR_NULL
    assert mlp(lib, w=[FAKE, ctypes.c_void_p(0x10002)]) == E.VN_ERR_ALIGN
    assert mlp(lib, b=[FAKE, ctypes.c_void_p(0x10002)]) == E.VN_ERR_ALIGN
    assert mlp(lib, y=ctypes.c_void_p(0x10002)) == E.VN_ERR_ALIGN
    assert mlp(lib, x=ctypes.c_void_p(0x10002)) == E.VN_ERR_ALIGN
    assert mlp(lib, pop=0, x=NULL, y=NULL, seeds=NULL) == E.VN_OK
    assert mlp(lib, batch=0, y=NULL) == E.VN_OK


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(2, 3)
    w = torch.zeros(4, 3)
    s = torch.arange(2)
    with pytest.raises(ValueError, match="GPU"):
        vn.virtual_perturbed_linear(x, w, None, s, 0.1, 0)
    with pytest.raises(ValueError, match="GPU"):
        vn.virtual_weight_gradient(torch.zeros(2), s, (4, 3), 0.1, 2, 0)


def ws_size(lib, dtype, pop, batch, i, o, math=0):
    out = ctypes.c_int64(-7)
    st = lib.vn_perturbed_linear_workspace_size(dtype, pop, batch, i, o, math, ctypes.byref(out))
    return st, out.value


def test_forward_workspace_size(lib):
    E = _lib
    mib = 1 << 20
    # bf16 operands, many rows: groups of up to 256 MiB of perturbed weights
    assert ws_size(lib, E.VN_BF16, 16, 4096, 4096, 4096) == (E.VN_OK, 8 * 32 * mib)
    assert ws_size(lib, E.VN_BF16, 3, 2048, 4096, 4096) == (E.VN_OK, 3 * 32 * mib)
    assert ws_size(lib, E.VN_BF16, 2, 2048, 16384, 16384) == (E.VN_OK, 512 * mib)   # one individual per group
    assert ws_size(lib, E.VN_BF16, 1, 2048, 128, 256) == (E.VN_OK, 256 * 128 * 2)
    assert ws_size(lib, E.VN_BF16, 1, 2048, 128, 255) == (E.VN_OK, 0)       # fewer than 256 outputs
    # sizes that keep the noise inside the product: no workspace
    assert ws_size(lib, E.VN_F32, 16, 4096, 4096, 4096) == (E.VN_OK, 0)
    assert ws_size(lib, E.VN_BF16, 16, 2047, 4096, 4096) == (E.VN_OK, 0)
    assert ws_size(lib, E.VN_BF16, 16, 4096, 4000, 4096) == (E.VN_OK, 0)      # in not a multiple of 64
    assert ws_size(lib, E.VN_BF16, 16, 4096, 64, 4096) == (E.VN_OK, 0)        # in below 128
    assert ws_size(lib, E.VN_BF16, 16, 4096, 1 << 22, 8) == (E.VN_OK, 0)     # in too wide
    assert ws_size(lib, E.VN_BF16, 0, 4096, 4096, 4096) == (E.VN_OK, 0)
    assert ws_size(lib, E.VN_BF16, 16, 4096, 4096, 0) == (E.VN_OK, 0)
    # errors
    assert lib.vn_perturbed_linear_workspace_size(E.VN_BF16, 1, 1, 1, 1, 0, None) == E.VN_ERR_NULL
    assert ws_size(lib, 7, 1, 1, 1, 1)[0] == E.VN_ERR_DTYPE
    assert ws_size(lib, E.VN_BF16, -1, 1, 1, 1)[0] == E.VN_ERR_SHAPE
    assert ws_size(lib, E.VN_BF16, 1, 1, -1, 1)[0] == E.VN_ERR_SHAPE
    assert ws_size(lib, E.VN_BF16, 1, 1, 1, 1, math=5)[0] == E.VN_ERR_VALUE
    assert ws_size(lib, E.VN_BF16, 1, 1, 2**62, 2**62)[0] == E.VN_ERR_OVERFLOW
