"""ctypes loader for libepdc.so (the HIP library built from csrc/)."""

from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libepdc.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "epdc.h")

EP_OK = 0
EP_ERR_INVALID_ARG = -1
EP_ERR_UNSUPPORTED = -2
EP_ERR_WORKSPACE = -3
EP_ERR_LAUNCH = -4
EP_WS_WAIT_GAVE_UP = 1
NOALLOC_SCRATCH_BYTES = 4 << 20
EP_DTYPE_BF16 = 0
EP_DTYPE_FP8_E4M3 = 1
EP_SCALE_F32 = 0
EP_SCALE_POW2 = 1
EP_SCALE_UE8M0 = 2

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "ep_abi_version": (_I32, []),
    "ep_status_string": (ctypes.c_char_p, [_I32]),
    "ep_workspace_status": (_I32, [_P, _SZ, _P, _P]),
    "ep_counts_workspace_bytes": (_SZ, [_I64, _I32, _I32, _I32]),
    "ep_layout_workspace_bytes": (_SZ, [_I64, _I32]),
    "ep_batched_workspace_bytes": (_SZ, [_I64, _I32, _I64]),
    "ep_compute_send_counts": (
        _I32, [_P, _I64, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "ep_build_send_layout": (
        _I32, [_P, _P, _P, _P, _I64, _I32, _I32, _I32, _I64, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "ep_dispatch_layout_workspace_bytes": (_SZ, [_I64, _I32, _I32]),
    "ep_dispatch_layout": (
        _I32, [_P, _P, _I64, _I32, _I32, _I32, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
               _P, _SZ, _P]),
    "ep_dispatch_layout_noalloc": (
        _I32, [_P, _P, _I64, _I32, _I32, _I32, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "ep_dispatch_layout_chunked_workspace_bytes": (_SZ, [_I64, _I32, _I32]),
    "ep_dispatch_layout_chunked": (
        _I32, [_P, _P, _I64, _I32, _I32, _I32, _I32, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P,
               _P, _SZ, _P]),
    "ep_regroup_workspace_bytes": (_SZ, [_I64, _I32]),
    "ep_regroup_by_expert": (
        _I32, [_P, _P, _P, _P, _I32, _I64, _I32, _I32, _I32, _I32, _I64, _P, _P, _P, _P, _P,
               _P, _P, _SZ, _P]),
    "ep_dispatch_permute": (_I32, [_P, _I64, _I32, _P, _I32, _I64, _I32, _P, _P, _P]),
    "ep_batched_prepare": (
        _I32, [_P, _P, _I64, _I32, _I32, _I32, _I32, _I64, _P, _P, _P, _P, _SZ, _P]),
    "ep_batched_prepare_fp8": (
        _I32, [_P, _P, _I64, _I32, _I32, _I32, _I32, _I64, _I32, _I32, _P, _P, _P, _P, _P, _SZ,
               _P]),
    "ep_combine": (_I32, [_P, _I64, _P, _P, _I64, _I32, _I32, _P, _P, _P, _P]),
}

_lib = None


# EPDC_ABI_VERSION of include/epdc.h that the signatures above follow
ABI_VERSION = 6


def header_functions():
    """Names of the functions declared in include/epdc.h."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ep_[a-z0-9_]+)\s*\(", text)))


def lib():
    """The loaded library.  Raises ImportError if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m combine_ep_send_amd.build` "
                "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        # the version first: a library of another version may lack symbols
        # these bindings name
        try:
            ver = L.ep_abi_version
        except AttributeError:
            raise ImportError(f"{LIB_PATH} exports no ep_abi_version: not an epdc library")
        ver.restype, ver.argtypes = _I32, []
        if ver() != ABI_VERSION:
            raise ImportError(
                f"{LIB_PATH} reports ABI version {ver()}, these bindings are for "
                f"{ABI_VERSION}: rebuild it with `python -m combine_ep_send_amd.build`")
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class EpError(RuntimeError):
    pass


def check(status: int, what: str) -> None:
    if status == EP_OK:
        return
    msg = f"{what}: {lib().ep_status_string(status).decode()} (status {status})"
    if status in (EP_ERR_INVALID_ARG, EP_ERR_UNSUPPORTED, EP_ERR_WORKSPACE):
        raise ValueError(msg)
    raise EpError(msg)
