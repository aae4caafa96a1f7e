"""ctypes binding of liblla.so (declared in include/lla.h).

Argument marshalling only: every step of the forward pass runs in the HIP
library. PyTorch supplies device memory and the current stream. If the
library has not been built this module raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("LLA_LIBRARY", os.path.join(HERE, "liblla.so"))

LLA_OK = 0
LLA_ERR_INVALID_ARG = -1
LLA_ERR_UNSUPPORTED = -2
LLA_ERR_HIP = -3
LLA_ERR_WORKSPACE = -4

LLA_DTYPE_F32 = 0
LLA_DTYPE_BF16 = 1

LLA_KERNEL_AUTO = 0
LLA_KERNEL_VALU = 1
LLA_KERNEL_MFMA = 2

LLA_FLAG_SPLIT_U = 1
LLA_FLAG_PRECOND = 2
LLA_FLAG_NO_PRECOND = 4

# Every symbol include/lla.h declares.
EXPORTED_SYMBOLS = (
    "lla_forward_f32", "lla_forward_bf16", "lla_forward_ex", "lla_output_given_rho",
    "lla_workspace_bytes", "lla_decode_ex", "lla_decode_workspace_bytes",
    "lla_backward_ex", "lla_backward_workspace_bytes", "lla_status_string", "lla_last_error", "lla_version",
    "lla_source_hash", "lla_decode_noalloc", "lla_forward_naive", "lla_naive_workspace_bytes",
)

LLA_DECODE_NOALLOC_SCRATCH_BYTES = 64 << 20


class LlaFwdArgs(ctypes.Structure):
    """Mirror of ``lla_fwd_args``."""
    _fields_ = [
        ("dtype", ctypes.c_int),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("B", ctypes.c_int),
        ("H", ctypes.c_int),
        ("n", ctypes.c_int),
        ("d", ctypes.c_int),
        ("lambda_", ctypes.c_float),
        ("cg_max_iters", ctypes.c_int),
        ("cg_rel_tol", ctypes.c_float),
        ("omega", ctypes.c_void_p),
        ("rho", ctypes.c_void_p),
        ("rowmax", ctypes.c_void_p),
        ("cg_iters", ctypes.c_void_p),
        ("cg_resid", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("kernel", ctypes.c_int),
        ("flags", ctypes.c_int),
        ("ev_main_begin", ctypes.c_void_p),
        ("ev_main_end", ctypes.c_void_p),
        ("rho_c", ctypes.c_void_p),
    ]


class LlaDecodeArgs(ctypes.Structure):
    """Mirror of ``lla_decode_args``."""
    _fields_ = [
        ("dtype", ctypes.c_int),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("B", ctypes.c_int),
        ("H", ctypes.c_int),
        ("n", ctypes.c_int),
        ("d", ctypes.c_int),
        ("lambda_", ctypes.c_float),
        ("cg_max_iters", ctypes.c_int),
        ("cg_rel_tol", ctypes.c_float),
        ("omega", ctypes.c_void_p),
        ("rho", ctypes.c_void_p),
        ("rowmax", ctypes.c_void_p),
        ("cg_iters", ctypes.c_void_p),
        ("cg_resid", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("ev_main_begin", ctypes.c_void_p),
        ("ev_main_end", ctypes.c_void_p),
    ]


class LlaBwdArgs(ctypes.Structure):
    """Mirror of ``lla_bwd_args``."""
    _fields_ = [
        ("dtype", ctypes.c_int),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("dout", ctypes.c_void_p),
        ("rho_c", ctypes.c_void_p),
        ("dq", ctypes.c_void_p),
        ("dk", ctypes.c_void_p),
        ("dv", ctypes.c_void_p),
        ("B", ctypes.c_int),
        ("H", ctypes.c_int),
        ("n", ctypes.c_int),
        ("d", ctypes.c_int),
        ("lambda_", ctypes.c_float),
        ("cg_max_iters", ctypes.c_int),
        ("cg_rel_tol", ctypes.c_float),
        ("adj_iters", ctypes.c_void_p),
        ("adj_resid", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("ev_main_begin", ctypes.c_void_p),
        ("ev_main_end", ctypes.c_void_p),
        ("flags", ctypes.c_int),
        ("kernel", ctypes.c_int),
    ]


class LlaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{status_string(status)} ({status}): {detail}")
        self.status = status
        self.detail = detail


_lib: Optional[ctypes.CDLL] = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load liblla.so (once). Raises FileNotFoundError if it is not built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(
            f"{p} not found: build it with `python -m local_linear_attention_flashlla_amd.build`")
    lib = ctypes.CDLL(p)
    vp, ci, cf, cz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.lla_forward_f32.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, cf, ci, cf, vp]
    lib.lla_forward_f32.restype = ci
    lib.lla_forward_bf16.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, cf, ci, cf, vp]
    lib.lla_forward_bf16.restype = ci
    lib.lla_forward_ex.argtypes = [ctypes.POINTER(LlaFwdArgs), vp]
    lib.lla_forward_ex.restype = ci
    lib.lla_output_given_rho.argtypes = [ctypes.POINTER(LlaFwdArgs), vp, vp]
    lib.lla_output_given_rho.restype = ci
    lib.lla_forward_naive.argtypes = [ctypes.POINTER(LlaFwdArgs), vp]
    lib.lla_forward_naive.restype = ci
    lib.lla_naive_workspace_bytes.argtypes = [ci, ci, ci, ci, ci]
    lib.lla_naive_workspace_bytes.restype = cz
    lib.lla_decode_ex.argtypes = [ctypes.POINTER(LlaDecodeArgs), vp]
    lib.lla_decode_ex.restype = ci
    lib.lla_decode_noalloc.argtypes = [ctypes.POINTER(LlaDecodeArgs), vp]
    lib.lla_decode_noalloc.restype = ci
    lib.lla_decode_workspace_bytes.argtypes = [ci, ci, ci, ci, ci]
    lib.lla_decode_workspace_bytes.restype = cz
    lib.lla_backward_ex.argtypes = [ctypes.POINTER(LlaBwdArgs), vp]
    lib.lla_backward_ex.restype = ci
    lib.lla_backward_workspace_bytes.argtypes = [ci, ci, ci, ci, ci]
    lib.lla_backward_workspace_bytes.restype = cz
    lib.lla_workspace_bytes.argtypes = [ci, ci, ci, ci, ci, ci]
    lib.lla_workspace_bytes.restype = cz
    lib.lla_status_string.argtypes = [ci]
    lib.lla_status_string.restype = ctypes.c_char_p
    lib.lla_last_error.argtypes = []
    lib.lla_last_error.restype = ctypes.c_char_p
    lib.lla_version.argtypes = []
    lib.lla_version.restype = ci
    lib.lla_source_hash.argtypes = []
    lib.lla_source_hash.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def is_current(lib: Optional[ctypes.CDLL] = None) -> bool:
    """Whether the loaded library was built from the sources in this tree
    (its lla_source_hash() equals the build script's hash of them)."""
    from .build import source_hash
    lib = lib or load()
    return lib.lla_source_hash().decode() == source_hash()


def status_string(status: int) -> str:
    return load().lla_status_string(int(status)).decode()


def last_error() -> str:
    return load().lla_last_error().decode()


def check(status: int) -> None:
    if status != LLA_OK:
        raise LlaError(status, last_error())
