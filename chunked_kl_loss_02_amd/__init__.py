"""Fused chunked top-K KL distillation loss on AMD MI355X (gfx950).

Thin Python binding over the C ABI in include/kdkl.h (libkdkl.so, built in
this directory by chunked_kl_loss_02_amd.build).  This module only marshals
arguments: torch provides device memory and the current HIP stream; every
step of the loss runs in the library's HIP kernels.  If the library is not
built, importing works but every call raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["fwd_bwd", "workspace_size", "lse", "KdProblem", "library_path", "lib",
           "timing_enable", "timing_collect", "KERNEL_CLASSES", "KD_FLAG_VALIDATE"]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libkdkl.so")

KD_FLAG_VALIDATE = 1
KERNEL_CLASSES = ("teacher", "gather", "pass1", "lse", "loss", "pass2", "fixup", "bwd", "other")
_STATUS = {0: "KD_OK", 1: "KD_ERR_ARG", 2: "KD_ERR_UNSUPPORTED", 3: "KD_ERR_WORKSPACE",
           4: "KD_ERR_INDEX", 5: "KD_ERR_NONFINITE", 6: "KD_ERR_HIP"}


class KdProblem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int64), ("V", ctypes.c_int64),
                ("K", ctypes.c_int32), ("tau", ctypes.c_float), ("chunk_v", ctypes.c_int32),
                ("block_t", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class KdError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{_STATUS.get(code, code)}: {msg}")
        self.code = code


_lib = None


def lib():
    """The loaded libkdkl.so (ctypes.CDLL); raises if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise RuntimeError(f"{library_path} is missing: build it with "
                           "`python -m chunked_kl_loss_02_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(library_path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    P = ctypes.POINTER(KdProblem)
    L.kd_topk_kl_workspace_size.argtypes = [P, ctypes.POINTER(sz)]
    L.kd_topk_kl_workspace_size.restype = ctypes.c_int
    L.kd_topk_kl_fwd_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.kd_topk_kl_fwd_bwd.restype = ctypes.c_int
    L.kd_topk_kl_workspace_lse2.argtypes = [P, vp]
    L.kd_topk_kl_workspace_lse2.restype = vp
    L.kd_status_string.argtypes = [ctypes.c_int]
    L.kd_status_string.restype = ctypes.c_char_p
    L.kd_abi_version.argtypes = []
    L.kd_abi_version.restype = ctypes.c_int
    L.kd_timing_enable.argtypes = [ctypes.c_int]
    L.kd_timing_enable.restype = ctypes.c_int
    L.kd_timing_collect.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    L.kd_timing_collect.restype = ctypes.c_int
    _lib = L
    return L


def _raise(code):
    if code != 0:
        raise KdError(code, lib().kd_status_string(code).decode())


def problem(T, H, V, K, tau=1.0, chunk_v=0, block_t=0, validate=False) -> KdProblem:
    return KdProblem(int(T), int(H), int(V), int(K), float(tau), int(chunk_v), int(block_t),
                     KD_FLAG_VALIDATE if validate else 0)


def workspace_size(T, H, V, K, tau=1.0, chunk_v=0, block_t=0) -> int:
    n = ctypes.c_size_t(0)
    _raise(lib().kd_topk_kl_workspace_size(ctypes.byref(problem(T, H, V, K, tau, chunk_v, block_t)),
                                           ctypes.byref(n)))
    return n.value


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def fwd_bwd(h, W, teacher_idx, teacher_logit, mask=None, tau=1.0, *, chunk_v=0, block_t=0,
            grad_h=True, grad_w=True, row_loss=False, validate=False, workspace=None,
            return_workspace=False, out=None):
    """loss, dH, dW [, row_loss] [, workspace] of the fused chunked top-K KL loss.

    h [T,H] bf16, W [V,H] bf16, teacher_idx [T,K] int32, teacher_logit [T,K]
    fp32, mask [T] uint8/bool or None; all contiguous on the same GPU.  dH and
    dW are fp32 (None when not requested); loss is a 0-d fp32 tensor.  Runs on
    torch's current stream; returns without synchronising.  `out` may pass
    preallocated (loss, dH, dW[, row_loss]) tensors to be overwritten."""
    import torch
    T, H = h.shape
    V = W.shape[0]
    K = teacher_idx.shape[1] if teacher_idx.dim() == 2 else 0
    dev = h.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    if h.dtype != torch.bfloat16 or W.dtype != torch.bfloat16:
        raise TypeError("h and W must be bfloat16")
    if teacher_idx.dtype != torch.int32 or teacher_logit.dtype != torch.float32:
        raise TypeError("teacher_idx must be int32 and teacher_logit float32")
    for name, t in (("h", h), ("W", W), ("teacher_idx", teacher_idx), ("teacher_logit", teacher_logit)):
        if not t.is_contiguous() or t.device != dev:
            raise ValueError(f"{name} must be contiguous on {dev}")
    if W.shape[1] != H or teacher_idx.shape != (T, K) or teacher_logit.shape != (T, K):
        raise ValueError("shape mismatch")
    if mask is not None:
        if mask.dtype == torch.bool:
            mask = mask.view(torch.uint8)
        if mask.dtype != torch.uint8 or mask.shape != (T,) or not mask.is_contiguous() or mask.device != dev:
            raise ValueError("mask must be a contiguous uint8/bool [T] tensor on the same device")
    prob = problem(T, H, V, K, tau, chunk_v, block_t, validate)
    n = ctypes.c_size_t(0)
    _raise(lib().kd_topk_kl_workspace_size(ctypes.byref(prob), ctypes.byref(n)))
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(max(n.value, 256), dtype=torch.uint8, device=dev)
    if out is not None:
        loss, dH, dW = out[0], out[1], out[2]
        rl = out[3] if row_loss else None
        for t, shp in ((loss, ()), (dH, (T, H)), (dW, (V, H)), (rl, (T,))):
            if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != shp or not t.is_contiguous()
                                  or t.device != dev):
                raise ValueError("preallocated outputs must be contiguous fp32 of the right shapes")
        grad_h, grad_w = dH is not None, dW is not None
    else:
        loss = torch.empty((), dtype=torch.float32, device=dev)
        dH = torch.empty((T, H), dtype=torch.float32, device=dev) if grad_h else None
        dW = torch.empty((V, H), dtype=torch.float32, device=dev) if grad_w else None
        rl = torch.empty((T,), dtype=torch.float32, device=dev) if row_loss else None
    stream = torch.cuda.current_stream(dev).cuda_stream
    code = lib().kd_topk_kl_fwd_bwd(ctypes.byref(prob), _ptr(h), _ptr(W), _ptr(teacher_idx),
                                    _ptr(teacher_logit), _ptr(mask), _ptr(loss), _ptr(dH), _ptr(dW),
                                    _ptr(rl), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
                                    ctypes.c_void_p(stream))
    _raise(code)
    res = [loss, dH, dW]
    if row_loss:
        res.append(rl)
    if return_workspace:
        res.append(workspace)
    return tuple(res)


def lse(workspace, T, H, V, K, tau=1.0, chunk_v=0, block_t=0):
    """Per-token natural-log log-sum-exp of S/tau left in `workspace` by the
    last completed fwd_bwd call with the same problem (fp32 [T] view)."""
    import torch
    prob = problem(T, H, V, K, tau, chunk_v, block_t)
    addr = lib().kd_topk_kl_workspace_lse2(ctypes.byref(prob), _ptr(workspace))
    if not addr:
        raise KdError(1, "invalid problem")
    off = addr - workspace.data_ptr()
    return workspace[off:off + 4 * T].view(torch.float32) * 0.6931471805599453


def timing_enable(on=True):
    _raise(lib().kd_timing_enable(1 if on else 0))


def timing_collect():
    """{class: (total_ms, launches)} for the launches recorded since enabling."""
    ms = (ctypes.c_double * 9)()
    cnt = (ctypes.c_int64 * 9)()
    _raise(lib().kd_timing_collect(ms, cnt))
    return {KERNEL_CLASSES[i]: (ms[i], cnt[i]) for i in range(9)}
