"""ctypes loader for libvn.so and the status-code plumbing.

The shared library is built in-tree by ``virtual_noise_perturbed_amd.build``;
nothing here computes any part of the method.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int32, c_int64, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvn.so")

VN_OK, VN_ERR_NULL, VN_ERR_SHAPE, VN_ERR_VALUE, VN_ERR_DTYPE, VN_ERR_OVERFLOW, VN_ERR_HIP, VN_ERR_ALIGN = range(8)
VN_F32, VN_BF16 = 0, 1
VN_I64, VN_I32 = 0, 1
VN_ACT_NONE, VN_ACT_RELU = 0, 1
VN_MATH_DEFAULT, VN_MATH_F32 = 0, 1

# name -> argument types, in the order of include/vn.h
SIGNATURES = {
    "vn_status_string": [c_int32],
    "vn_abi_version": [],
    "vn_last_hip_error": [],
    "vn_compute_offsets": [c_void_p, c_void_p, c_int32, c_void_p, c_void_p],
    "vn_perturbed_linear": [c_void_p, c_int64, c_void_p, c_int32, c_void_p, c_void_p, c_int32,
                            c_int64, c_int64, c_int64, c_int64, c_float, c_int64, c_int32, c_int32,
                            c_void_p, c_void_p, c_int64, c_void_p],
    "vn_perturbed_linear_workspace_size": [c_int32, c_int64, c_int64, c_int64, c_int64, c_int32, c_void_p],
    "vn_perturbed_mlp": [c_void_p, c_int64, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                         c_void_p, c_int32, c_int64, c_int64, c_float, c_int32, c_void_p, c_void_p],
    "vn_weight_gradient": [c_void_p, c_void_p, c_int32, c_int64, c_int64, c_int64, c_float, c_int64,
                           c_void_p, c_void_p],
    "vn_bias_gradient": [c_void_p, c_void_p, c_int32, c_int64, c_int64, c_float, c_int64,
                         c_void_p, c_void_p],
    "vn_flat_gradient": [c_void_p, c_void_p, c_int32, c_int64, c_int64, c_float, c_int64,
                         c_void_p, c_void_p],
    "vn_reduce_metric_workspace_size": [c_int64, c_int64, c_void_p],
    "vn_reduce_metric": [c_void_p, c_void_p, c_int32, c_int64, c_int64, c_float, c_int64,
                         c_void_p, c_void_p, c_int64, c_void_p],
    "vn_reduce_metric_noalloc": [c_void_p, c_void_p, c_int32, c_int64, c_int64, c_float, c_int64,
                                 c_void_p, c_void_p],
    "vn_noise_u32": [c_void_p, c_int32, c_int64, c_int64, c_int64, c_void_p, c_void_p],
    "vn_noise_f32": [c_void_p, c_int32, c_int64, c_int64, c_int64, c_void_p, c_void_p],
}

_RESTYPES = {"vn_status_string": ctypes.c_char_p, "vn_last_hip_error": ctypes.c_char_p}

_lib = None


class VNError(RuntimeError):
    """A vn_* call returned a non-OK status."""

    def __init__(self, fn: str, status: int, detail: str = ""):
        self.status = status
        msg = f"{fn} failed: {status_string(status)} (status {status})"
        if detail:
            msg += f": {detail}"
        super().__init__(msg)


def load(path: str = LIB_PATH):
    """Load libvn.so once; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m virtual_noise_perturbed_amd.build` "
            "(the HIP library is required; there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    for name, argtypes in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = _RESTYPES.get(name, c_int32)
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().vn_status_string(status).decode()


def check(fn_name: str, status: int):
    if status == VN_OK:
        return
    detail = ""
    if status == VN_ERR_HIP:
        detail = load().vn_last_hip_error().decode()
    if status in (VN_ERR_HIP,):
        raise VNError(fn_name, status, detail)
    err = VNError(fn_name, status, detail)
    raise ValueError(str(err)) from err
