"""MI355X (gfx950) E2-TTT chunk update: Python binding of libe2ttt.so.

Argument marshalling only: every step of the chunk update runs in the HIP
kernels behind the C ABI (include/e2ttt.h).  PyTorch supplies device memory
and the current HIP stream.  There is no CPU fallback: without the built
library, or with tensors that are not on a GPU, every entry point raises.

Method: "Rethinking Expressivity and Efficiency in Test-Time Training"
(E2-TTT).  For each chunk, gradients of the fast-weight loss at the
chunk-start weights feed a closed-form transition that reproduces the
chunk-end weights W and momentum M of the per-token recurrence
M_t = beta_t M_{t-1} + eta_t g_t, W_t = alpha_t W_{t-1} - M_t, and the chunk
output comes from the chunk-start weights.  Variants: ``momentum=False``
(W_t = alpha_t W_{t-1} - eta_t g_t) and ``chunk_avg=True`` (the per-token
kernels replaced by their chunk means).  ``chunk_backward`` is the
vector-Jacobian product of ``chunk_forward`` (SwiGLU MFMA path).
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (E2TTTError, FLAG_CHUNK_AVG, FLAG_FORCE_GENERIC, FLAG_NO_MOMENTUM, FLAG_PRECISE, FLAG_SAVE_STATES,
                   make_desc)

__all__ = ["chunk_forward", "chunk_forward_noalloc", "chunk_backward", "chunk_update", "training_workspace", "logscan", "workspace_size", "param_count", "path", "validate", "E2TTTError",
           "library"]


def library():
    return _lib.load()


def _io_name(t: torch.Tensor) -> str:
    if t.dtype == torch.bfloat16:
        return "bf16"
    if t.dtype == torch.float32:
        return "f32"
    raise TypeError(f"q/k/v must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def param_count(kind: str, D: int, Hd: int = 0) -> int:
    return int(library().e2ttt_param_count(ctypes.byref(make_desc(kind, "mse", "f32", 1, 1, 0, D, Hd, 1))))


def workspace_size(kind, loss, io_dtype, B, H, T, D, Hd, chunk, flags=0) -> int:
    d = make_desc(kind, loss, io_dtype, B, H, T, D, Hd, chunk, flags)
    n = library().e2ttt_workspace_size(ctypes.byref(d))
    if n == ctypes.c_size_t(-1).value:
        raise E2TTTError("e2ttt_workspace_size", 1)
    return int(n)


def path(kind, loss, io_dtype, B, H, T, D, Hd, chunk, flags=0) -> int:
    return int(library().e2ttt_path(ctypes.byref(make_desc(kind, loss, io_dtype, B, H, T, D, Hd, chunk, flags))))


def validate(desc, ptrs) -> int:
    arr = (ctypes.c_void_p * 11)(*[ctypes.c_void_p(p) for p in ptrs])
    return int(library().e2ttt_validate(ctypes.byref(desc), arr))


def _stream_handle(stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def training_workspace(q, *, chunk: int, kind: str = "swiglu", loss: str = "negdot", Hd: int = 0,
                       momentum: bool = True, chunk_avg: bool = False, force_generic: bool = False):
    """A workspace shared by chunk_forward(save_states=True) and the
    chunk_backward(saved=True) that follows it (uint8 tensor on q's device)."""
    B, H, T, D = q.shape
    flags = FLAG_SAVE_STATES | (0 if momentum else FLAG_NO_MOMENTUM) | (FLAG_CHUNK_AVG if chunk_avg else 0) | \
        (FLAG_FORCE_GENERIC if force_generic else 0)
    d = make_desc(kind, loss, _io_name(q), B, H, T, D, Hd, chunk, flags)
    n = library().e2ttt_backward_workspace_size(ctypes.byref(d))
    if n == ctypes.c_size_t(-1).value:
        raise E2TTTError("e2ttt_backward_workspace_size", 1)
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=q.device)


def _forward_args(q, k, v, eta, alpha, beta, W0, M0, chunk, kind, loss, Hd, out, W_end, M_end, force_generic,
                  momentum, chunk_avg, save_states, precise=False):
    """Checks and descriptor shared by chunk_forward and chunk_forward_noalloc;
    returns (lib, desc, beta, M0, out, W_end, M_end)."""
    lib = library()
    if not momentum:
        beta = M0 = None
        M_end = None
    for name, t in (("q", q), ("k", k), ("v", v), ("eta", eta), ("alpha", alpha), ("beta", beta),
                    ("W0", W0), ("M0", M0)):
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    io = _io_name(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    for name, t in (("eta", eta), ("alpha", alpha), ("beta", beta), ("W0", W0), ("M0", M0)):
        if t is not None and t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    B, H, T, D = q.shape
    flags = (FLAG_FORCE_GENERIC if force_generic else 0) | (0 if momentum else FLAG_NO_MOMENTUM) | \
        (FLAG_CHUNK_AVG if chunk_avg else 0) | (FLAG_SAVE_STATES if save_states else 0) | \
        (FLAG_PRECISE if precise else 0)
    desc = make_desc(kind, loss, io, B, H, T, D, Hd, chunk, flags)
    P = int(lib.e2ttt_param_count(ctypes.byref(desc)))
    if tuple(W0.shape) != (B, H, P) or (M0 is not None and tuple(M0.shape) != (B, H, P)):
        raise ValueError(f"W0/M0 must have shape {(B, H, P)}")
    if tuple(eta.shape) != (B, H, T) or alpha.shape != eta.shape or (beta is not None and beta.shape != eta.shape):
        raise ValueError(f"eta/alpha/beta must have shape {(B, H, T)}")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one shape")
    if out is None:
        out = torch.empty_like(q)
    if W_end is None:
        W_end = torch.empty_like(W0)
    if M_end is None and momentum:
        M_end = torch.empty_like(M0)
    return lib, desc, beta, M0, out, W_end, M_end


def chunk_forward(q, k, v, eta, alpha, beta, W0, M0, *, chunk: int, kind: str, loss: str, Hd: int = 0,
                  out=None, W_end=None, M_end=None, workspace=None, force_generic: bool = False,
                  momentum: bool = True, chunk_avg: bool = False, save_states: bool = False, precise: bool = False,
                  stream=None):
    """Run the chunk update; returns (out, W_end, M_end).

    q, k, v: [B, H, T, D] float32 or bfloat16 (same dtype), contiguous, on GPU;
    eta, alpha, beta: [B, H, T] float32; W0, M0: [B, H, P] float32.
    ``W_end=W0`` / ``M_end=M0`` update the state in place.  With
    ``momentum=False`` beta and M0 are ignored (may be None) and M_end is None.
    ``save_states`` keeps in ``workspace`` (from training_workspace, required)
    what chunk_backward(saved=True) needs, so that it skips its recompute.
    ``precise`` (E2TTT_FLAG_PRECISE): hi/lo bf16 operands on the SwiGLU MFMA
    path, for states the bf16 operands cannot follow closely enough.
    """
    if save_states and workspace is None:
        raise ValueError("save_states needs the shared workspace from training_workspace()")
    lib, desc, beta, M0, out, W_end, M_end = _forward_args(
        q, k, v, eta, alpha, beta, W0, M0, chunk, kind, loss, Hd, out, W_end, M_end, force_generic, momentum,
        chunk_avg, save_states, precise)
    ws_bytes = int(lib.e2ttt_workspace_size(ctypes.byref(desc)))
    if ws_bytes == ctypes.c_size_t(-1).value:
        raise E2TTTError("e2ttt_workspace_size", 1)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    st = lib.e2ttt_chunk_forward(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(alpha),
                                 _ptr(beta), _ptr(W0), _ptr(M0), _ptr(out), _ptr(W_end), _ptr(M_end),
                                 _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream_handle(stream))
    if st != 0:
        raise E2TTTError("e2ttt_chunk_forward", st)
    return out, W_end, M_end


def chunk_forward_noalloc(q, k, v, eta, alpha, beta, W0, M0, *, chunk: int, kind: str, loss: str, Hd: int = 0,
                          out=None, W_end=None, M_end=None, force_generic: bool = False, momentum: bool = True,
                          chunk_avg: bool = False, precise: bool = False, stream=None):
    """chunk_forward through e2ttt_chunk_forward_noalloc: the library's own
    per-GPU scratch instead of a workspace (no device allocation by the
    library; pass ``out``, ``W_end`` and ``M_end`` to allocate nothing here
    either).  Calls that overlap in time on one GPU race on that scratch."""
    lib, desc, beta, M0, out, W_end, M_end = _forward_args(
        q, k, v, eta, alpha, beta, W0, M0, chunk, kind, loss, Hd, out, W_end, M_end, force_generic, momentum,
        chunk_avg, False, precise)
    st = lib.e2ttt_chunk_forward_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(alpha),
                                         _ptr(beta), _ptr(W0), _ptr(M0), _ptr(out), _ptr(W_end), _ptr(M_end),
                                         _stream_handle(stream))
    if st != 0:
        raise E2TTTError("e2ttt_chunk_forward_noalloc", st)
    return out, W_end, M_end


def chunk_backward(q, k, v, eta, alpha, beta, W0, M0, dout, dW_end, dM_end, *, chunk: int, Hd: int,
                   kind: str = "swiglu", loss: str = "negdot", momentum: bool = True, chunk_avg: bool = False,
                   force_generic: bool = False, precise: bool = False, workspace=None, saved: bool = False,
                   stream=None):
    """Gradients of <dout, out> + <dW_end, W_end> + <dM_end, M_end> through
    ``chunk_forward``; returns a dict with keys q, k, v (the I/O dtype), eta,
    alpha, beta, W0, M0 (float32).  Without momentum beta, M0 and dM_end are
    ignored and the beta / M0 gradients are None.  ``force_generic`` takes the
    portable fp32 backward where the SwiGLU MFMA one applies; so does
    ``precise`` (the backward of a precise forward).  ``saved``:
    ``workspace`` holds the states a chunk_forward(save_states=True) call on
    the same inputs left in it; the forward is then not recomputed."""
    if saved and workspace is None:
        raise ValueError("saved=True needs the workspace the forward call filled")
    lib = library()
    if not momentum:
        beta = M0 = dM_end = None
    named = (("q", q), ("k", k), ("v", v), ("eta", eta), ("alpha", alpha), ("beta", beta), ("W0", W0),
             ("M0", M0), ("dout", dout), ("dW_end", dW_end), ("dM_end", dM_end))
    for name, t in named:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    for name, t in named:
        want = q.dtype if name in ("q", "k", "v", "dout") else torch.float32
        if t is not None and t.dtype != want:
            raise TypeError(f"{name} must be {want}")
    B, H, T, D = q.shape
    flags = (0 if momentum else FLAG_NO_MOMENTUM) | (FLAG_CHUNK_AVG if chunk_avg else 0) | \
        (FLAG_FORCE_GENERIC if force_generic else 0) | (FLAG_SAVE_STATES if saved else 0) | \
        (FLAG_PRECISE if precise else 0)
    desc = make_desc(kind, loss, _io_name(q), B, H, T, D, Hd, chunk, flags)
    P = int(lib.e2ttt_param_count(ctypes.byref(desc)))
    for name, t, shp in (("k", k, q.shape), ("v", v, q.shape), ("dout", dout, q.shape),
                         ("eta", eta, (B, H, T)), ("alpha", alpha, (B, H, T)), ("beta", beta, (B, H, T)),
                         ("W0", W0, (B, H, P)), ("M0", M0, (B, H, P)), ("dW_end", dW_end, (B, H, P)),
                         ("dM_end", dM_end, (B, H, P))):
        if t is not None and tuple(t.shape) != tuple(shp):
            raise ValueError(f"{name} must have shape {tuple(shp)}")
    g = {"q": torch.empty_like(q), "k": torch.empty_like(k), "v": torch.empty_like(v),
         "eta": torch.empty_like(eta), "alpha": torch.empty_like(alpha),
         "beta": torch.empty_like(beta) if momentum else None, "W0": torch.empty_like(W0),
         "M0": torch.empty_like(M0) if momentum else None}
    ws_bytes = int(lib.e2ttt_backward_workspace_size(ctypes.byref(desc)))
    if ws_bytes == ctypes.c_size_t(-1).value:
        raise E2TTTError("e2ttt_backward_workspace_size", 1)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    st = lib.e2ttt_chunk_backward(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(alpha),
                                  _ptr(beta), _ptr(W0), _ptr(M0), _ptr(dout), _ptr(dW_end), _ptr(dM_end),
                                  _ptr(g["q"]), _ptr(g["k"]), _ptr(g["v"]), _ptr(g["eta"]), _ptr(g["alpha"]),
                                  _ptr(g["beta"]), _ptr(g["W0"]), _ptr(g["M0"]), _ptr(workspace),
                                  ctypes.c_size_t(workspace.numel()), _stream_handle(stream))
    if st != 0:
        raise E2TTTError("e2ttt_chunk_backward", st)
    return g


def logscan(eta, alpha, beta, *, chunk: int, momentum: bool = True, chunk_avg: bool = False, stream=None):
    """The scalar-kernel step alone: returns (cM, cW, scal[B, H, T/chunk, 4]).
    ``momentum=False`` takes beta = 0 (beta may be None); ``chunk_avg`` replaces
    the per-token kernels by their chunk means."""
    lib = library()
    if not momentum:
        beta = None
    for name, t in (("eta", eta), ("alpha", alpha), ("beta", beta)):
        if t is None:
            continue
        if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 GPU tensor")
    B, H, T = eta.shape
    if chunk < 1:
        raise ValueError("chunk must be positive")
    cM = torch.empty_like(eta)
    cW = torch.empty_like(eta)
    scal = torch.empty(B, H, (T + chunk - 1) // chunk, 4, dtype=torch.float32, device=eta.device)
    flags = (0 if momentum else FLAG_NO_MOMENTUM) | (FLAG_CHUNK_AVG if chunk_avg else 0)
    desc = make_desc("linear", "mse", "f32", B, H, T, 1, 0, chunk, flags)
    st = lib.e2ttt_logscan(ctypes.byref(desc), _ptr(eta), _ptr(alpha), _ptr(beta), _ptr(cM), _ptr(cW),
                           _ptr(scal), _stream_handle(stream))
    if st != 0:
        raise E2TTTError("e2ttt_logscan", st)
    return cM, cW, scal


class _ChunkUpdate(torch.autograd.Function):
    """chunk_forward with chunk_backward as its derivative (both through the C ABI)."""

    @staticmethod
    def forward(ctx, q, k, v, eta, alpha, beta, W0, M0, chunk, kind, loss, Hd, momentum, chunk_avg):
        ws = training_workspace(q, chunk=chunk, kind=kind, loss=loss, Hd=Hd, momentum=momentum,
                                chunk_avg=chunk_avg)
        out, W, M = chunk_forward(q, k, v, eta, alpha, beta, W0, M0, chunk=chunk, kind=kind, loss=loss, Hd=Hd,
                                  momentum=momentum, chunk_avg=chunk_avg, workspace=ws, save_states=True)
        ctx.save_for_backward(q, k, v, eta, alpha, beta, W0, M0)
        ctx.ws = ws  # the chunk-start states for the backward
        ctx.opts = (chunk, kind, loss, Hd, momentum, chunk_avg)
        if M is None:
            M = torch.zeros_like(W0)  # no momentum: a placeholder output with no gradient path
        return out, W, M

    @staticmethod
    def backward(ctx, dout, dW, dM):
        q, k, v, eta, alpha, beta, W0, M0 = ctx.saved_tensors
        chunk, kind, loss, Hd, momentum, chunk_avg = ctx.opts
        dout = torch.zeros_like(q) if dout is None else dout.to(q.dtype).contiguous()
        dW = torch.zeros_like(W0) if dW is None else dW.contiguous()
        dM = (torch.zeros_like(W0) if dM is None else dM.contiguous()) if momentum else None
        g = chunk_backward(q, k, v, eta, alpha, beta if momentum else None, W0, M0 if momentum else None, dout, dW, dM,
                           chunk=chunk, Hd=Hd, kind=kind, loss=loss, momentum=momentum, chunk_avg=chunk_avg,
                           workspace=ctx.ws, saved=True)
        ctx.ws = None
        return (g["q"], g["k"], g["v"], g["eta"], g["alpha"], g["beta"], g["W0"], g["M0"],
                None, None, None, None, None, None)


def chunk_update(q, k, v, eta, alpha, beta, W0, M0, *, chunk: int, kind: str = "swiglu", loss: str = "negdot",
                 Hd: int = 0, momentum: bool = True, chunk_avg: bool = False):
    """The chunk update as a differentiable PyTorch op: (out, W_end, M_end),
    with gradients for every input from ``chunk_backward``.  Without
    momentum, beta and M0 may be None and M_end is None."""
    if not momentum:
        beta = M0 = None
        dummy = torch.zeros((), device=q.device)  # keeps the argument list tensor-typed
        out, W, _ = _ChunkUpdate.apply(q, k, v, eta, alpha, dummy, W0, dummy, chunk, kind, loss, Hd, False,
                                       chunk_avg)
        return out, W, None
    return _ChunkUpdate.apply(q, k, v, eta, alpha, beta, W0, M0, chunk, kind, loss, Hd, True, chunk_avg)
