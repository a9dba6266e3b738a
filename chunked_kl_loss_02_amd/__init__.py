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

__all__ = ["fwd_bwd", "fwd_bwd_noalloc", "tiling", "NOALLOC_SCRATCH_BYTES", "fwd", "bwd", "topk_kl_loss", "kl_logits", "logits_workspace_size", "KdLogitsProblem",
           "topk_select", "KdTopkProblem", "TopKKLLoss", "workspace_size", "fwd_workspace_size",
           "saved_size", "lse", "saved_lse", "KdProblem", "library_path", "lib", "timing_enable",
           "timing_collect", "KERNEL_CLASSES", "KD_FLAG_VALIDATE", "KD_FLAG_ACCUMULATE_DH",
           "KD_FLAG_ACCUMULATE_DW", "KD_FLAG_GRAD_BF16", "KD_FLAG_SEQ_CHUNK"]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libkdkl.so")

KD_FLAG_VALIDATE = 1
KD_FLAG_ACCUMULATE_DH = 2
KD_FLAG_ACCUMULATE_DW = 4
KD_FLAG_GRAD_BF16 = 8
KD_FLAG_SEQ_CHUNK = 16
ABI_VERSION = 5
KD_FLAG_LOGITS_F32 = 32
NOALLOC_SCRATCH_BYTES = 128 << 20  # KD_NOALLOC_SCRATCH_BYTES
KERNEL_CLASSES = ("teacher", "gather", "pass1", "lse", "loss", "pass2", "buckets", "bwd", "other", "logits", "topk",
                  "bwd_pass2")
_STATUS = {0: "KD_OK", 1: "KD_ERR_ARG", 2: "KD_ERR_UNSUPPORTED", 3: "KD_ERR_WORKSPACE",
           4: "KD_ERR_INDEX", 5: "KD_ERR_NONFINITE", 6: "KD_ERR_HIP"}


class KdProblem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int64), ("V", ctypes.c_int64),
                ("K", ctypes.c_int32), ("tau", ctypes.c_float), ("chunk_v", ctypes.c_int32),
                ("block_t", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class KdLogitsProblem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("V", ctypes.c_int64), ("K", ctypes.c_int32), ("tau", ctypes.c_float),
                ("flags", ctypes.c_uint32)]


class KdTopkProblem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("V", ctypes.c_int64), ("K", ctypes.c_int32), ("flags", ctypes.c_uint32)]


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
    # torch first: its HIP runtime must be the one the library binds to (a
    # second runtime loaded ahead of torch's sees no device in this process)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(library_path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    P = ctypes.POINTER(KdProblem)
    L.kd_topk_kl_workspace_size.argtypes = [P, ctypes.POINTER(sz)]
    L.kd_topk_kl_workspace_size.restype = ctypes.c_int
    L.kd_topk_kl_tiling.argtypes = [P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                                    ctypes.POINTER(ctypes.c_int32)]
    L.kd_topk_kl_tiling.restype = ctypes.c_int
    L.kd_topk_kl_fwd_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.kd_topk_kl_fwd_bwd.restype = ctypes.c_int
    L.kd_topk_kl_fwd_bwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.kd_topk_kl_fwd_bwd_noalloc.restype = ctypes.c_int
    for name in ("kd_topk_kl_saved_size", "kd_topk_kl_fwd_workspace_size"):
        getattr(L, name).argtypes = [P, ctypes.POINTER(sz)]
        getattr(L, name).restype = ctypes.c_int
    L.kd_topk_kl_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.kd_topk_kl_fwd.restype = ctypes.c_int
    L.kd_topk_kl_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.kd_topk_kl_bwd.restype = ctypes.c_int
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
    L.kd_timing_classes.argtypes = [ctypes.c_uint32]
    L.kd_timing_classes.restype = ctypes.c_int
    LP = ctypes.POINTER(KdLogitsProblem)
    L.kd_topk_kl_logits_workspace_size.argtypes = [LP, ctypes.POINTER(sz)]
    L.kd_topk_kl_logits_workspace_size.restype = ctypes.c_int
    L.kd_topk_kl_logits.argtypes = [LP, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.kd_topk_kl_logits.restype = ctypes.c_int
    L.kd_topk_select.argtypes = [ctypes.POINTER(KdTopkProblem), vp, vp, vp, vp]
    L.kd_topk_select.restype = ctypes.c_int
    if L.kd_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{library_path} has ABI {L.kd_abi_version()}, this binding expects {ABI_VERSION}: rebuild it")
    _lib = L
    return L


def _raise(code):
    if code != 0:
        raise KdError(code, lib().kd_status_string(code).decode())


def problem(T, H, V, K, tau=1.0, chunk_v=0, block_t=0, validate=False, flags=0) -> KdProblem:
    return KdProblem(int(T), int(H), int(V), int(K), float(tau), int(chunk_v), int(block_t),
                     (KD_FLAG_VALIDATE if validate else 0) | int(flags))


def _size(fn, prob):
    n = ctypes.c_size_t(0)
    _raise(fn(ctypes.byref(prob), ctypes.byref(n)))
    return n.value


def workspace_size(T, H, V, K, tau=1.0, chunk_v=0, block_t=0, flags=0, seq_chunk=False) -> int:
    """Workspace bytes of fwd_bwd / bwd."""
    flags |= KD_FLAG_SEQ_CHUNK if seq_chunk else 0
    return _size(lib().kd_topk_kl_workspace_size, problem(T, H, V, K, tau, chunk_v, block_t, flags=flags))


def tiling(T, H, V, K, tau=1.0, chunk_v=0, block_t=0, flags=0, seq_chunk=False):
    """(tokens per block, vocabulary rows per chunk, gradient buffers) that
    fwd_bwd / bwd use for this problem."""
    flags |= KD_FLAG_SEQ_CHUNK if seq_chunk else 0
    bt, cv, nb = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int32(0)
    prob = problem(T, H, V, K, tau, chunk_v, block_t, flags=flags)
    _raise(lib().kd_topk_kl_tiling(ctypes.byref(prob), ctypes.byref(bt), ctypes.byref(cv), ctypes.byref(nb)))
    return bt.value, cv.value, nb.value


def fwd_workspace_size(T, H, V, K, tau=1.0, chunk_v=0, block_t=0) -> int:
    """Workspace bytes of fwd (no gradient buffer)."""
    return _size(lib().kd_topk_kl_fwd_workspace_size, problem(T, H, V, K, tau, chunk_v, block_t))


def saved_size(T, H, V, K, tau=1.0, chunk_v=0, block_t=0) -> int:
    """Bytes of the state fwd leaves for bwd."""
    return _size(lib().kd_topk_kl_saved_size, problem(T, H, V, K, tau, chunk_v, block_t))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _check_inputs(h, W, teacher_idx, teacher_logit, mask):
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
    return T, H, V, K, dev, mask


def _grad_flags(grad_dtype, accumulate_dh, accumulate_dw):
    import torch
    if grad_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("gradient outputs are float32 or bfloat16")
    return ((KD_FLAG_GRAD_BF16 if grad_dtype == torch.bfloat16 else 0)
            | (KD_FLAG_ACCUMULATE_DH if accumulate_dh else 0) | (KD_FLAG_ACCUMULATE_DW if accumulate_dw else 0))


def _check_out(t, shape, dtype, dev, what):
    if t is not None and (t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous()
                          or t.device != dev):
        raise ValueError(f"{what} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {dev}")


def _workspace(workspace, nbytes, dev):
    """The caller's workspace (a contiguous uint8 tensor on the inputs'
    device) if it is large enough, else a new one."""
    import torch
    if workspace is not None and (workspace.dtype != torch.uint8 or workspace.device != dev
                                  or not workspace.is_contiguous()):
        raise ValueError(f"workspace must be a contiguous uint8 tensor on {dev}")
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    return workspace


def fwd_bwd(h, W, teacher_idx, teacher_logit, mask=None, tau=1.0, *, chunk_v=0, block_t=0,
            grad_h=True, grad_w=True, row_loss=False, validate=False, workspace=None,
            return_workspace=False, out=None, grad_dtype=None, accumulate_dh=False, accumulate_dw=False,
            seq_chunk=False):
    """loss, dH, dW [, row_loss] [, workspace] of the fused chunked top-K KL loss.

    h [T,H] bf16, W [V,H] bf16, teacher_idx [T,K] int32, teacher_logit [T,K]
    fp32, mask [T] uint8/bool or None; all contiguous on the same GPU.  dH and
    dW are fp32, or bf16 with grad_dtype=torch.bfloat16 (None when not
    requested); loss is a 0-d fp32 tensor.  Runs on torch's current stream;
    returns without synchronising.  `out` may pass preallocated
    (loss, dH, dW[, row_loss]) tensors, which are overwritten (dH / dW are
    added to with accumulate_dh / accumulate_dw).  seq_chunk=True selects the
    sequence-chunk schedule (stored block logits, no recompute; block_t
    tokens x V fp32 of workspace)."""
    import torch
    T, H, V, K, dev, mask = _check_inputs(h, W, teacher_idx, teacher_logit, mask)
    gdt = grad_dtype or (out[1].dtype if out is not None and out[1] is not None else
                         out[2].dtype if out is not None and out[2] is not None else torch.float32)
    flags = _grad_flags(gdt, accumulate_dh, accumulate_dw) | (KD_FLAG_SEQ_CHUNK if seq_chunk else 0)
    prob = problem(T, H, V, K, tau, chunk_v, block_t, validate, flags)
    workspace = _workspace(workspace, _size(lib().kd_topk_kl_workspace_size, prob), dev)
    if out is not None:
        loss, dH, dW = out[0], out[1], out[2]
        rl = out[3] if row_loss else None
        _check_out(loss, (), torch.float32, dev, "loss")
        _check_out(dH, (T, H), gdt, dev, "dH")
        _check_out(dW, (V, H), gdt, dev, "dW")
        _check_out(rl, (T,), torch.float32, dev, "row_loss")
    else:
        if accumulate_dh or accumulate_dw:
            raise ValueError("accumulation needs preallocated outputs (out=...)")
        loss = torch.empty((), dtype=torch.float32, device=dev)
        dH = torch.empty((T, H), dtype=gdt, device=dev) if grad_h else None
        dW = torch.empty((V, H), dtype=gdt, device=dev) if grad_w else None
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


def fwd_bwd_noalloc(h, W, teacher_idx, teacher_logit, mask=None, tau=1.0, *, out, chunk_v=0, block_t=0,
                    row_loss=False, validate=False, accumulate_dh=False, accumulate_dw=False, seq_chunk=False):
    """fwd_bwd through kd_topk_kl_fwd_bwd_noalloc: no workspace and no device
    allocation (the library's static per-GPU scratch of NOALLOC_SCRATCH_BYTES
    takes its place).  `out` = preallocated (loss, dH, dW[, row_loss]), dH /
    dW may be None; they are overwritten (added to with accumulate_*).
    Returns `out`'s tensors."""
    import torch
    T, H, V, K, dev, mask = _check_inputs(h, W, teacher_idx, teacher_logit, mask)
    loss, dH, dW = out[0], out[1], out[2]
    rl = out[3] if row_loss else None
    gdt = dH.dtype if dH is not None else dW.dtype if dW is not None else torch.float32
    flags = _grad_flags(gdt, accumulate_dh, accumulate_dw) | (KD_FLAG_SEQ_CHUNK if seq_chunk else 0)
    prob = problem(T, H, V, K, tau, chunk_v, block_t, validate, flags)
    _check_out(loss, (), torch.float32, dev, "loss")
    _check_out(dH, (T, H), gdt, dev, "dH")
    _check_out(dW, (V, H), gdt, dev, "dW")
    _check_out(rl, (T,), torch.float32, dev, "row_loss")
    stream = torch.cuda.current_stream(dev).cuda_stream
    _raise(lib().kd_topk_kl_fwd_bwd_noalloc(ctypes.byref(prob), _ptr(h), _ptr(W), _ptr(teacher_idx),
                                            _ptr(teacher_logit), _ptr(mask), _ptr(loss), _ptr(dH), _ptr(dW),
                                            _ptr(rl), ctypes.c_void_p(stream)))
    return (loss, dH, dW, rl) if row_loss else (loss, dH, dW)


def fwd(h, W, teacher_idx, teacher_logit, mask=None, tau=1.0, *, chunk_v=0, block_t=0, row_loss=False,
        validate=False, workspace=None):
    """Loss pass only: (loss, saved[, row_loss]).  `saved` (uint8 device
    tensor) holds the per-token state bwd needs."""
    import torch
    T, H, V, K, dev, mask = _check_inputs(h, W, teacher_idx, teacher_logit, mask)
    prob = problem(T, H, V, K, tau, chunk_v, block_t, validate)
    workspace = _workspace(workspace, _size(lib().kd_topk_kl_fwd_workspace_size, prob), dev)
    saved = torch.empty(_size(lib().kd_topk_kl_saved_size, prob), dtype=torch.uint8, device=dev)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    rl = torch.empty((T,), dtype=torch.float32, device=dev) if row_loss else None
    stream = torch.cuda.current_stream(dev).cuda_stream
    _raise(lib().kd_topk_kl_fwd(ctypes.byref(prob), _ptr(h), _ptr(W), _ptr(teacher_idx), _ptr(teacher_logit),
                                _ptr(mask), _ptr(loss), _ptr(rl), _ptr(saved), _ptr(workspace),
                                ctypes.c_size_t(workspace.numel()), ctypes.c_void_p(stream)))
    return (loss, saved, rl) if row_loss else (loss, saved)


def bwd(saved, h, W, teacher_idx, teacher_logit, mask=None, tau=1.0, *, grad_loss=None, chunk_v=0, block_t=0,
        grad_h=True, grad_w=True, grad_dtype=None, dH=None, dW=None, accumulate_dh=False, accumulate_dw=False,
        validate=False, workspace=None):
    """Gradient pass: (dH, dW) = grad_loss * d(loss)/d(h, W), from the
    `saved` state of fwd on the same inputs.  grad_loss: 0-d fp32 device
    tensor or None (= 1).  dH / dW may be preallocated (required to
    accumulate); their dtype (fp32 or bf16) selects the output type."""
    import torch
    T, H, V, K, dev, mask = _check_inputs(h, W, teacher_idx, teacher_logit, mask)
    gdt = grad_dtype or (dH.dtype if dH is not None else dW.dtype if dW is not None else torch.float32)
    flags = _grad_flags(gdt, accumulate_dh, accumulate_dw)
    prob = problem(T, H, V, K, tau, chunk_v, block_t, validate, flags)
    if saved.dtype != torch.uint8 or saved.device != dev or saved.numel() < _size(lib().kd_topk_kl_saved_size, prob):
        raise ValueError("saved must be the uint8 state returned by fwd for this problem")
    if grad_loss is not None:
        if grad_loss.numel() != 1 or grad_loss.device != dev:
            raise ValueError("grad_loss must be a one-element tensor on the inputs' device")
        grad_loss = grad_loss.reshape(()).to(torch.float32).contiguous()
    if (accumulate_dh and dH is None) or (accumulate_dw and dW is None):
        raise ValueError("accumulation needs preallocated dH / dW")
    if dH is None and grad_h:
        dH = torch.empty((T, H), dtype=gdt, device=dev)
    if dW is None and grad_w:
        dW = torch.empty((V, H), dtype=gdt, device=dev)
    _check_out(dH, (T, H), gdt, dev, "dH")
    _check_out(dW, (V, H), gdt, dev, "dW")
    workspace = _workspace(workspace, _size(lib().kd_topk_kl_workspace_size, prob), dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    _raise(lib().kd_topk_kl_bwd(ctypes.byref(prob), _ptr(h), _ptr(W), _ptr(teacher_idx), _ptr(teacher_logit),
                                _ptr(mask), _ptr(saved), _ptr(grad_loss), _ptr(dH), _ptr(dW), _ptr(workspace),
                                ctypes.c_size_t(workspace.numel()), ctypes.c_void_p(stream)))
    return dH, dW


def saved_lse(saved, T):
    """Natural-log per-token log-sum-exp of S/tau from fwd's saved state."""
    import torch
    return saved[:4 * T].view(torch.float32) * 0.6931471805599453


def _make_autograd():
    import torch

    class TopKKLLoss(torch.autograd.Function):
        """Autograd wrapper: forward = fwd, backward = bwd with the incoming
        gradient as grad_loss; gradients come back in the inputs' dtype
        (bf16) straight from the library."""

        @staticmethod
        def forward(ctx, h, W, teacher_idx, teacher_logit, mask, tau, chunk_v, block_t):
            loss, saved = fwd(h, W, teacher_idx, teacher_logit, mask, tau, chunk_v=chunk_v, block_t=block_t)
            ctx.save_for_backward(h, W, teacher_idx, teacher_logit, saved,
                                  mask if mask is not None else torch.empty(0, device=h.device))
            ctx.has_mask = mask is not None
            ctx.args = (tau, chunk_v, block_t)
            return loss

        @staticmethod
        def backward(ctx, grad):
            h, W, idx, logit, saved, mask = ctx.saved_tensors
            tau, chunk_v, block_t = ctx.args
            need_h, need_w = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
            dH = dW = None
            if need_h or need_w:
                dH, dW = bwd(saved, h, W, idx, logit, mask if ctx.has_mask else None, tau, grad_loss=grad,
                             chunk_v=chunk_v, block_t=block_t, grad_h=need_h, grad_w=need_w,
                             grad_dtype=h.dtype)
            return dH, dW, None, None, None, None, None, None

    return TopKKLLoss


TopKKLLoss = None


def topk_kl_loss(h, W, teacher_idx, teacher_logit, mask=None, tau=1.0, *, chunk_v=0, block_t=0):
    """Differentiable fused chunked top-K KL loss (mean over kept tokens);
    d/dh and d/dW flow back through the library's gradient pass."""
    global TopKKLLoss
    if TopKKLLoss is None:
        TopKKLLoss = _make_autograd()
    return TopKKLLoss.apply(h, W, teacher_idx, teacher_logit, mask, float(tau), int(chunk_v), int(block_t))


def lse(workspace, T, H, V, K, tau=1.0, chunk_v=0, block_t=0, flags=0):
    """Per-token natural-log log-sum-exp of S/tau left in `workspace` by the
    last completed fwd_bwd call with the same problem (fp32 [T] view)."""
    import torch
    prob = problem(T, H, V, K, tau, chunk_v, block_t, flags=flags)
    addr = lib().kd_topk_kl_workspace_lse2(ctypes.byref(prob), _ptr(workspace))
    if not addr:
        raise KdError(1, "invalid problem")
    off = addr - workspace.data_ptr()
    return workspace[off:off + 4 * T].view(torch.float32) * 0.6931471805599453


def timing_enable(on=True, classes=None):
    """Per-kernel HIP-event timing on or off; classes: names from
    KERNEL_CLASSES to time (None: all), the others record no events."""
    mask = 0xFFFFFFFF
    if classes is not None:
        mask = 0
        for c in classes:
            mask |= 1 << KERNEL_CLASSES.index(c)
    _raise(lib().kd_timing_classes(mask))
    _raise(lib().kd_timing_enable(1 if on else 0))


def timing_collect():
    """{class: (total_ms, launches)} for the launches recorded since enabling."""
    n = len(KERNEL_CLASSES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _raise(lib().kd_timing_collect(ms, cnt))
    return {KERNEL_CLASSES[i]: (ms[i], cnt[i]) for i in range(n)}


def logits_workspace_size(T, V, K, tau=1.0, f32=False) -> int:
    p = KdLogitsProblem(int(T), int(V), int(K), float(tau), KD_FLAG_LOGITS_F32 if f32 else 0)
    n = ctypes.c_size_t(0)
    _raise(lib().kd_topk_kl_logits_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def kl_logits(Z, teacher_idx, teacher_logit, mask=None, tau=1.0, *, grad=True, row_loss=False, validate=False,
              workspace=None, out=None):
    """Forward-chunked KL on materialised student logits Z [T,V] (bf16 or
    fp32): (loss, dZ[, row_loss]); dZ has Z's dtype (None with grad=False).
    `out` may pass preallocated (loss, dZ[, row_loss])."""
    import torch
    if Z.dim() != 2 or Z.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("Z must be a 2-D bfloat16 or float32 tensor")
    T, V = Z.shape
    K = teacher_idx.shape[1] if teacher_idx.dim() == 2 else 0
    dev = Z.device
    if dev.type != "cuda" or not Z.is_contiguous():
        raise ValueError("Z must be a contiguous GPU tensor")
    if teacher_idx.dtype != torch.int32 or teacher_logit.dtype != torch.float32:
        raise TypeError("teacher_idx must be int32 and teacher_logit float32")
    for name, t in (("teacher_idx", teacher_idx), ("teacher_logit", teacher_logit)):
        if not t.is_contiguous() or t.device != dev or tuple(t.shape) != (T, K):
            raise ValueError(f"{name} must be a contiguous [T, K] tensor on {dev}")
    if mask is not None:
        if mask.dtype == torch.bool:
            mask = mask.view(torch.uint8)
        if mask.dtype != torch.uint8 or mask.shape != (T,) or not mask.is_contiguous() or mask.device != dev:
            raise ValueError("mask must be a contiguous uint8/bool [T] tensor on the same device")
    f32 = Z.dtype == torch.float32
    p = KdLogitsProblem(int(T), int(V), int(K), float(tau),
                        (KD_FLAG_LOGITS_F32 if f32 else 0) | (KD_FLAG_VALIDATE if validate else 0))
    n = ctypes.c_size_t(0)
    _raise(lib().kd_topk_kl_logits_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    workspace = _workspace(workspace, n.value, dev)
    if out is not None:
        loss, dZ = out[0], out[1]
        rl = out[2] if row_loss else None
        _check_out(loss, (), torch.float32, dev, "loss")
        _check_out(dZ, (T, V), Z.dtype, dev, "dZ")
        _check_out(rl, (T,), torch.float32, dev, "row_loss")
    else:
        loss = torch.empty((), dtype=torch.float32, device=dev)
        dZ = torch.empty((T, V), dtype=Z.dtype, device=dev) if grad else None
        rl = torch.empty((T,), dtype=torch.float32, device=dev) if row_loss else None
    stream = torch.cuda.current_stream(dev).cuda_stream
    _raise(lib().kd_topk_kl_logits(ctypes.byref(p), _ptr(Z), _ptr(teacher_idx), _ptr(teacher_logit), _ptr(mask),
                                   _ptr(loss), _ptr(dZ), _ptr(rl), _ptr(workspace),
                                   ctypes.c_size_t(workspace.numel()), ctypes.c_void_p(stream)))
    return (loss, dZ, rl) if row_loss else (loss, dZ)


def topk_select(X, K, *, out=None):
    """The K largest values of every row of X [T,V] (bf16, on the GPU): ids
    (int32 [T,K], descending value, equal values by ascending id) and values
    (fp32 [T,K]) -- the content of the teacher's top-K cache."""
    import torch
    if X.dim() != 2 or X.dtype != torch.bfloat16 or X.device.type != "cuda" or not X.is_contiguous():
        raise TypeError("X must be a contiguous 2-D bfloat16 GPU tensor")
    T, V = X.shape
    dev = X.device
    if out is not None:
        idx, val = out
        _check_out(idx, (T, K), torch.int32, dev, "idx")
        _check_out(val, (T, K), torch.float32, dev, "values")
    else:
        idx = torch.empty((T, K), dtype=torch.int32, device=dev)
        val = torch.empty((T, K), dtype=torch.float32, device=dev)
    p = KdTopkProblem(int(T), int(V), int(K), 0)
    stream = torch.cuda.current_stream(dev).cuda_stream
    _raise(lib().kd_topk_select(ctypes.byref(p), _ptr(X), _ptr(idx), _ptr(val), ctypes.c_void_p(stream)))
    return idx, val
