"""Causal Local Linear Attention (LLA) forward for AMD Instinct MI355X.

The computation runs in liblla.so (hand-written HIP kernels for gfx950
behind the C ABI of include/lla.h); this package is a thin binding over it.
``forward`` takes torch tensors on the GPU and calls the library on torch's
current stream. There is no CPU fallback: without the built library or a GPU
the call raises.
"""
from __future__ import annotations

from typing import Optional

from . import _lib
from ._lib import (LLA_DTYPE_BF16, LLA_DTYPE_F32, LLA_FLAG_NO_PRECOND, LLA_FLAG_PRECOND,
                   LLA_FLAG_SPLIT_U, LLA_KERNEL_AUTO,
                   LLA_KERNEL_MFMA, LLA_KERNEL_VALU, LlaError)

__all__ = ["forward", "decode", "decode_workspace_bytes", "workspace_bytes", "naive_workspace_bytes",
           "LlaError", "LLA_KERNEL_AUTO", "LLA_KERNEL_VALU",
           "LLA_KERNEL_MFMA", "LLA_FLAG_SPLIT_U", "LLA_FLAG_PRECOND", "LLA_FLAG_NO_PRECOND", "version"]


def version() -> int:
    return _lib.load().lla_version()


def workspace_bytes(B: int, H: int, n: int, d: int, dtype: str = "bf16",
                    kernel: int = LLA_KERNEL_AUTO) -> int:
    dt = LLA_DTYPE_BF16 if dtype == "bf16" else LLA_DTYPE_F32
    return int(_lib.load().lla_workspace_bytes(B, H, n, d, dt, kernel))


def naive_workspace_bytes(B: int, H: int, n: int, d: int, dtype: str = "bf16") -> int:
    """Workspace of the naive forward (``forward(..., naive=True)``): the
    pairwise differences and moment matrices it materialises."""
    dt = LLA_DTYPE_BF16 if dtype == "bf16" else LLA_DTYPE_F32
    return int(_lib.load().lla_naive_workspace_bytes(B, H, n, d, dt))


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def forward(q, k, v, lam: float, cg_max_iters: int, cg_rel_tol: float, *,
            out=None, omega=None, rho=None, rowmax=None, cg_iters=None, cg_resid=None, rho_c=None,
            workspace=None, kernel: int = LLA_KERNEL_AUTO, flags: int = 0, stream=None,
            events=None, rho_in=None, naive: bool = False):
    """Causal LLA forward on the GPU.

    q, k, v: contiguous [B, H, n, d] tensors on a HIP device, all float32 or all
    bfloat16. Returns ``out`` ([B, H, n, d] float32). Optional outputs are
    filled when given: omega/rowmax/cg_resid [B, H, n] float32, rho and rho_c
    [B, H, n, d] float32 (the pages' rho_i and the solution of the system
    centred at the weighted key mean, which ``backward`` takes), cg_iters
    [B, H, n] int32. ``workspace`` is an
    optional uint8 device tensor of at least ``workspace_bytes(...)`` bytes.
    The call is asynchronous on ``stream`` (default: torch's current stream).
    ``events``: optional (begin, end) pair of ``torch.cuda.Event`` that the
    library records around its main kernel.
    ``rho_in``: optional [B, H, n, d] float32 GPU tensor; when given, the CG
    solve is skipped and ``out`` is Eq. (8) with this rho_i
    (``lla_output_given_rho``); ``lam``, ``cg_max_iters`` and ``cg_rel_tol``
    are then passed through but do not change the result.
    ``naive``: run ``lla_forward_naive`` instead (pairwise differences and
    moment matrices materialised, exact Cholesky solves, fp32; CG settings
    ignored, ``workspace`` sized by ``naive_workspace_bytes``).
    """
    import torch

    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, n, d] shape")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one dtype")
    if q.dtype == torch.float32:
        dtype = LLA_DTYPE_F32
    elif q.dtype == torch.bfloat16:
        dtype = LLA_DTYPE_BF16
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    B, H, n, d = (int(s) for s in q.shape)
    if out is None:
        out = torch.empty((B, H, n, d), dtype=torch.float32, device=q.device)
    for name, t, dt, shape in (("out", out, torch.float32, (B, H, n, d)),
                               ("omega", omega, torch.float32, (B, H, n)),
                               ("rho", rho, torch.float32, (B, H, n, d)),
                               ("rowmax", rowmax, torch.float32, (B, H, n)),
                               ("cg_iters", cg_iters, torch.int32, (B, H, n)),
                               ("cg_resid", cg_resid, torch.float32, (B, H, n)),
                               ("rho_c", rho_c, torch.float32, (B, H, n, d))):
        if t is None:
            continue
        if t.dtype != dt or tuple(t.shape) != shape or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous {dt} GPU tensor of shape {shape}")
    a = _lib.LlaFwdArgs()
    a.rho_c = _ptr(rho_c)
    a.dtype = dtype
    a.q, a.k, a.v, a.out = _ptr(q), _ptr(k), _ptr(v), _ptr(out)
    a.B, a.H, a.n, a.d = B, H, n, d
    a.lambda_ = float(lam)
    a.cg_max_iters = int(cg_max_iters)
    a.cg_rel_tol = float(cg_rel_tol)
    a.omega, a.rho, a.rowmax = _ptr(omega), _ptr(rho), _ptr(rowmax)
    a.cg_iters, a.cg_resid = _ptr(cg_iters), _ptr(cg_resid)
    if workspace is not None:
        a.workspace = _ptr(workspace)
        a.workspace_bytes = int(workspace.numel() * workspace.element_size())
    a.kernel = int(kernel)
    a.flags = int(flags)
    if events is not None:
        ev0, ev1 = events
        ev0.record()  # makes torch create the underlying HIP events
        ev1.record()
        a.ev_main_begin, a.ev_main_end = int(ev0.cuda_event), int(ev1.cuda_event)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    import ctypes
    if naive:
        if rho_in is not None:
            raise ValueError("naive and rho_in do not combine")
        st = _lib.load().lla_forward_naive(ctypes.byref(a), ctypes.c_void_p(handle))
    elif rho_in is not None:
        if (rho_in.dtype != torch.float32 or tuple(rho_in.shape) != (B, H, n, d)
                or not rho_in.is_contiguous() or not rho_in.is_cuda):
            raise ValueError(f"rho_in must be a contiguous float32 GPU tensor of shape {(B, H, n, d)}")
        st = _lib.load().lla_output_given_rho(ctypes.byref(a), ctypes.c_void_p(_ptr(rho_in)),
                                             ctypes.c_void_p(handle))
    else:
        st = _lib.load().lla_forward_ex(ctypes.byref(a), ctypes.c_void_p(handle))
    _lib.check(st)
    return out


def decode_workspace_bytes(B: int, H: int, n: int, d: int, dtype: str = "bf16") -> int:
    dt = LLA_DTYPE_BF16 if dtype == "bf16" else LLA_DTYPE_F32
    return int(_lib.load().lla_decode_workspace_bytes(B, H, n, d, dt))


def decode(q, k, v, lam: float, cg_max_iters: int, cg_rel_tol: float, *, out=None, omega=None,
           rho=None, rowmax=None, cg_iters=None, cg_resid=None, workspace=None, stream=None,
           events=None, noalloc: bool = False):
    """Decode-shaped LLA forward on the GPU: one new query per (batch, head).

    q: [B, H, d]; k, v: [B, H, n, d] key and value caches (the new key and
    value included), contiguous GPU tensors, all float32 or all bfloat16.
    Returns ``out`` ([B, H, d] float32), the last row of the causal forward
    whose query is q. Optional outputs: omega/rowmax/cg_resid [B, H] float32,
    rho [B, H, d] float32, cg_iters [B, H] int32. ``events``: optional
    (begin, end) pair recorded around the Gram kernel. ``noalloc``: call
    lla_decode_noalloc (the library's static per-GPU scratch; no workspace,
    nothing allocated) instead of lla_decode_ex; pass ``out`` to allocate
    nothing on this side either.
    """
    import ctypes
    import torch

    if q.dim() != 3 or k.dim() != 4 or k.shape != v.shape or tuple(q.shape) != (
            k.shape[0], k.shape[1], k.shape[3]):
        raise ValueError("q must be [B, H, d] and k, v [B, H, n, d]")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one dtype")
    if q.dtype == torch.float32:
        dtype = LLA_DTYPE_F32
    elif q.dtype == torch.bfloat16:
        dtype = LLA_DTYPE_BF16
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    B, H, n, d = (int(s) for s in k.shape)
    if out is None:
        out = torch.empty((B, H, d), dtype=torch.float32, device=q.device)
    for name, t, dt, shape in (("out", out, torch.float32, (B, H, d)),
                               ("omega", omega, torch.float32, (B, H)),
                               ("rho", rho, torch.float32, (B, H, d)),
                               ("rowmax", rowmax, torch.float32, (B, H)),
                               ("cg_iters", cg_iters, torch.int32, (B, H)),
                               ("cg_resid", cg_resid, torch.float32, (B, H))):
        if t is None:
            continue
        if t.dtype != dt or tuple(t.shape) != shape or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous {dt} GPU tensor of shape {shape}")
    a = _lib.LlaDecodeArgs()
    a.dtype = dtype
    a.q, a.k, a.v, a.out = _ptr(q), _ptr(k), _ptr(v), _ptr(out)
    a.B, a.H, a.n, a.d = B, H, n, d
    a.lambda_ = float(lam)
    a.cg_max_iters = int(cg_max_iters)
    a.cg_rel_tol = float(cg_rel_tol)
    a.omega, a.rho, a.rowmax = _ptr(omega), _ptr(rho), _ptr(rowmax)
    a.cg_iters, a.cg_resid = _ptr(cg_iters), _ptr(cg_resid)
    if workspace is not None:
        a.workspace = _ptr(workspace)
        a.workspace_bytes = int(workspace.numel() * workspace.element_size())
    if events is not None:
        ev0, ev1 = events
        ev0.record()
        ev1.record()
        a.ev_main_begin, a.ev_main_end = int(ev0.cuda_event), int(ev1.cuda_event)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc decode takes no workspace")
        _lib.check(_lib.load().lla_decode_noalloc(ctypes.byref(a), ctypes.c_void_p(handle)))
    else:
        _lib.check(_lib.load().lla_decode_ex(ctypes.byref(a), ctypes.c_void_p(handle)))
    return out


def backward_workspace_bytes(B: int, H: int, n: int, d: int, dtype: str = "bf16") -> int:
    dt = LLA_DTYPE_BF16 if dtype == "bf16" else LLA_DTYPE_F32
    return int(_lib.load().lla_backward_workspace_bytes(B, H, n, d, dt))


def backward(q, k, v, out, dout, rho_c, lam: float, cg_max_iters: int, cg_rel_tol: float, *,
             dq=None, dk=None, dv=None, adj_iters=None, adj_resid=None, workspace=None,
             stream=None, events=None, flags=0, kernel=LLA_KERNEL_AUTO):
    """Gradient of sum(dout * out) for the causal LLA forward on the GPU.

    q, k, v: [B, H, n, d], the forward's inputs (float32 or bfloat16; the
    matrix-core path takes bfloat16 with d in {64, 128}, the vector path any
    d in {16, 32, 64, 128}; ``kernel`` as for ``forward``, the same choice);
    out, rho_c: the forward's output and its ``rho_c`` output ([B, H, n, d]
    float32, from ``forward(..., rho_c=...)`` with the same lam and CG
    policy);
    dout: [B, H, n, d] float32. Returns (dq, dk, dv), float32 [B, H, n, d].
    Optional: adj_iters [B, H, n] int32 and adj_resid [B, H, n] float32 (the
    adjoint CG's steps and final relative residual); ``events``: a (begin,
    end) pair recorded around the adjoint CG kernel.
    """
    import ctypes
    import torch

    if q.dtype not in (torch.bfloat16, torch.float32) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("backward: q, k, v must share one dtype, float32 or bfloat16")
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, n, d] shape")
    B, H, n, d = (int(s) for s in q.shape)
    shape = (B, H, n, d)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if dq is None:
        dq = torch.empty(shape, dtype=torch.float32, device=q.device)
    if dk is None:
        dk = torch.empty(shape, dtype=torch.float32, device=q.device)
    if dv is None:
        dv = torch.empty(shape, dtype=torch.float32, device=q.device)
    for name, t, dt, shp in (("out", out, torch.float32, shape), ("dout", dout, torch.float32, shape),
                             ("rho_c", rho_c, torch.float32, shape), ("dq", dq, torch.float32, shape),
                             ("dk", dk, torch.float32, shape), ("dv", dv, torch.float32, shape),
                             ("adj_iters", adj_iters, torch.int32, shape[:3]),
                             ("adj_resid", adj_resid, torch.float32, shape[:3])):
        if t is None:
            continue
        if t.dtype != dt or tuple(t.shape) != shp or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous {dt} GPU tensor of shape {shp}")
    a = _lib.LlaBwdArgs()
    a.dtype = LLA_DTYPE_BF16 if q.dtype == torch.bfloat16 else LLA_DTYPE_F32
    a.kernel = int(kernel)
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    a.out, a.dout, a.rho_c = _ptr(out), _ptr(dout), _ptr(rho_c)
    a.dq, a.dk, a.dv = _ptr(dq), _ptr(dk), _ptr(dv)
    a.B, a.H, a.n, a.d = B, H, n, d
    a.lambda_ = float(lam)
    a.cg_max_iters = int(cg_max_iters)
    a.cg_rel_tol = float(cg_rel_tol)
    a.adj_iters, a.adj_resid = _ptr(adj_iters), _ptr(adj_resid)
    a.flags = int(flags)
    if workspace is not None:
        a.workspace = _ptr(workspace)
        a.workspace_bytes = int(workspace.numel() * workspace.element_size())
    if events is not None:
        ev0, ev1 = events
        ev0.record()
        ev1.record()
        a.ev_main_begin, a.ev_main_end = int(ev0.cuda_event), int(ev1.cuda_event)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    _lib.check(_lib.load().lla_backward_ex(ctypes.byref(a), ctypes.c_void_p(handle)))
    return dq, dk, dv
