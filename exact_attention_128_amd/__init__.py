"""Fused exact attention for AMD MI355X (gfx950): thin Python binding.

Every step of the computation runs in the HIP kernels of ``libattn.so``
(built from ``csrc/`` by ``build.py``); this module only checks tensors,
allocates outputs with PyTorch and passes raw device pointers and the current
stream through the C ABI declared in ``include/attn.h``.  There is no CPU or
PyTorch fallback: if the library is missing, every call raises.

    o, lse = fwd(q, k, v, causal=False, scale=None)
    dq, dk, dv = bwd(q, k, v, o, lse, do, causal=False, scale=None)

q, k, v, do: torch.bfloat16 CUDA tensors, contiguous [B, H, S, D], D in {64, 128}.
"""
from __future__ import annotations

import math

from . import _lib
from ._lib import AttnError, load, library_path  # noqa: F401

__all__ = ["fwd", "bwd", "fwd_out", "fwd_rescale_events", "bwd_out", "bwd_workspace_size",
           "bwd_noalloc_out", "default_policy", "fwd_fp8", "fwd_fp8_out", "AttnError", "load",
           "library_path"]


def _check(t, name, shape=None, device=None):
    """bf16, contiguous, 4-D, on a GPU -- and on `device` (q's) when given."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != torch.bfloat16:
        raise TypeError("%s must be torch.bfloat16, got %s" % (name, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU device" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, q on %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous [B,H,S,D]" % name)
    if t.dim() != 4:
        raise ValueError("%s must be 4-D [B,H,S,D]" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s shape %s != %s" % (name, tuple(t.shape), tuple(shape)))


def _check_lse(lse, B, H, S, device):
    """fp32, contiguous [B,H,S], on q's device (the kernels write or read it)."""
    import torch
    if not isinstance(lse, torch.Tensor):
        raise TypeError("lse must be a torch.Tensor")
    if lse.device != device:
        raise ValueError("lse is on %s, q on %s" % (lse.device, device))
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, S) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B,H,S]")


def _stream(device):
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def fwd_out(q, k, v, o, lse, causal: bool = False, scale: float | None = None,
            rescale_log2: float | None = None, exp_poly_every: int | None = None) -> None:
    """Forward into caller-provided o (bf16 [B,H,S,D]) and lse (fp32 [B,H,S]).

    rescale_log2 / exp_poly_every override the per-shape softmax policy
    (attn_fwd_ex / attn_fwd_policy); None keeps the library's choice."""
    _check(q, "q")
    B, H, S, D = q.shape
    _check(k, "k", q.shape, q.device)
    _check(v, "v", q.shape, q.device)
    _check(o, "o", q.shape, q.device)
    _check_lse(lse, B, H, S, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = _stream(q.device)
    if exp_poly_every is not None:
        if rescale_log2 is None:
            rescale_log2 = default_policy(D, causal, S)[0]
        rc = _lib.load().attn_fwd_policy(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                         lse.data_ptr(), B, H, S, D, float(scale),
                                         int(bool(causal)), float(rescale_log2),
                                         int(exp_poly_every), st)
    elif rescale_log2 is None:
        rc = _lib.load().attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  lse.data_ptr(), B, H, S, D, float(scale), int(bool(causal)), st)
    else:
        rc = _lib.load().attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                     lse.data_ptr(), B, H, S, D, float(scale), int(bool(causal)),
                                     float(rescale_log2), st)
    _lib.raise_for(rc, "attn_fwd")


def fwd(q, k, v, causal: bool = False, scale: float | None = None,
        rescale_log2: float | None = None, exp_poly_every: int | None = None):
    """Returns (O bf16 [B,H,S,D], LSE fp32 [B,H,S])."""
    import torch
    _check(q, "q")
    B, H, S, D = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    fwd_out(q, k, v, o, lse, causal=causal, scale=scale, rescale_log2=rescale_log2,
            exp_poly_every=exp_poly_every)
    return o, lse


def _check_u8(t, name, shape=None, device=None):
    """E4M3 codes: uint8, contiguous, 4-D, on q's GPU."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != torch.uint8:
        raise TypeError("%s must hold E4M3 codes as torch.uint8, got %s" % (name, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU device" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, q on %s" % (name, t.device, device))
    if not t.is_contiguous() or t.dim() != 4:
        raise ValueError("%s must be contiguous 4-D [B,H,S,D]" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s shape %s != %s" % (name, tuple(t.shape), tuple(shape)))


def fwd_fp8_out(q, k, v, q_descale, k_descale, v_descale, o, lse, causal: bool = False,
                scale: float | None = None) -> None:
    """FP8 forward (attn_fwd_fp8) into caller-provided o (bf16) and lse (fp32);
    q, k, v are E4M3 codes (uint8 [B,H,S,D]) with one descale factor each."""
    import torch
    _check_u8(q, "q")
    B, H, S, D = q.shape
    _check_u8(k, "k", q.shape, q.device)
    _check_u8(v, "v", q.shape, q.device)
    if o.dtype != torch.bfloat16 or o.device != q.device or not o.is_contiguous() or \
            tuple(o.shape) != tuple(q.shape):
        raise ValueError("o must be contiguous bf16 [B,H,S,D] on q's device")
    _check_lse(lse, B, H, S, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rc = _lib.load().attn_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  lse.data_ptr(), B, H, S, D, float(scale), int(bool(causal)),
                                  float(q_descale), float(k_descale), float(v_descale),
                                  _stream(q.device))
    _lib.raise_for(rc, "attn_fwd_fp8")


def fwd_fp8(q, k, v, q_descale, k_descale, v_descale, causal: bool = False,
            scale: float | None = None):
    """Returns (O bf16 [B,H,S,D], LSE fp32 [B,H,S]) of the FP8 forward."""
    import torch
    _check_u8(q, "q")
    B, H, S, D = q.shape
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    fwd_fp8_out(q, k, v, q_descale, k_descale, v_descale, o, lse, causal=causal, scale=scale)
    return o, lse


def default_policy(D: int, causal: bool, S: int):
    """(rescale_log2, exp_poly_every) that attn_fwd picks for this shape."""
    import ctypes
    tau, poly = ctypes.c_float(), ctypes.c_int()
    rc = _lib.load().attn_fwd_default_policy(int(D), int(bool(causal)), int(S), ctypes.byref(tau),
                                             ctypes.byref(poly))
    _lib.raise_for(rc, "attn_fwd_default_policy")
    return float(tau.value), int(poly.value)


def fwd_rescale_events(q, k, v, causal: bool = False, scale: float | None = None,
                       rescale_log2: float = 32.0):
    """Diagnostic forward (attn_fwd_rescale_events): returns (O, LSE, tests,
    rescales), the counts of conditional-rescale tests (one per wave of 32
    query rows and 128-key step after the first) and of those that fired.
    Synchronises the current stream to read the counters."""
    import torch
    _check(q, "q")
    B, H, S, D = q.shape
    _check(k, "k", q.shape, q.device)
    _check(v, "v", q.shape, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    ev = torch.zeros(2, dtype=torch.int64, device=q.device)
    rc = _lib.load().attn_fwd_rescale_events(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                             o.data_ptr(), lse.data_ptr(), B, H, S, D,
                                             float(scale), int(bool(causal)),
                                             float(rescale_log2), ev.data_ptr(),
                                             _stream(q.device))
    _lib.raise_for(rc, "attn_fwd_rescale_events")
    tests, rescales = (int(x) for x in ev.cpu().tolist())
    return o, lse, tests, rescales


def bwd_workspace_size(B: int, H: int, S: int, D: int) -> int:
    return int(_lib.load().attn_bwd_workspace_size(B, H, S, D))


BWD_PRE, BWD_MAIN, BWD_DQ, BWD_ALL = 1, 2, 4, 7


def bwd_out(q, k, v, o, lse, do, dq, dk, dv, workspace, causal: bool = False,
            scale: float | None = None, phases: int = BWD_ALL) -> None:
    """Backward into caller-provided dq, dk, dv and a uint8 workspace tensor.

    `phases` selects a subset of the three launches (see attn_bwd_phases)."""
    _check(q, "q")
    B, H, S, D = q.shape
    for name, t in (("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check(t, name, q.shape, q.device)
    _check_lse(lse, B, H, S, q.device)
    if workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    nbytes = workspace.numel() * workspace.element_size()
    rc = _lib.load().attn_bwd_phases(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                     lse.data_ptr(), do.data_ptr(), dq.data_ptr(),
                                     dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), nbytes,
                                     B, H, S, D, float(scale), int(bool(causal)), int(phases),
                                     _stream(q.device))
    _lib.raise_for(rc, "attn_bwd")


def bwd_noalloc_out(q, k, v, o, lse, do, dq, dk, dv, causal: bool = False,
                    scale: float | None = None) -> None:
    """Backward into caller-provided dq, dk, dv with no workspace argument
    (attn_bwd_noalloc: the library's static per-GPU scratch array).  Calls
    that overlap on one GPU race on that array."""
    _check(q, "q")
    B, H, S, D = q.shape
    for name, t in (("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check(t, name, q.shape, q.device)
    _check_lse(lse, B, H, S, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rc = _lib.load().attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                      lse.data_ptr(), do.data_ptr(), dq.data_ptr(),
                                      dk.data_ptr(), dv.data_ptr(), B, H, S, D, float(scale),
                                      int(bool(causal)), _stream(q.device))
    _lib.raise_for(rc, "attn_bwd_noalloc")


def bwd(q, k, v, o, lse, do, causal: bool = False, scale: float | None = None):
    """Returns (dQ, dK, dV), bf16 [B,H,S,D]."""
    import torch
    _check(q, "q")
    B, H, S, D = q.shape
    ws = torch.empty(max(1, bwd_workspace_size(B, H, S, D)), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    bwd_out(q, k, v, o, lse, do, dq, dk, dv, ws, causal=causal, scale=scale)
    return dq, dk, dv
