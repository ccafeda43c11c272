"""Python binding of libfattn (fused exact attention for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libfattn.so``; PyTorch supplies device memory and the current
stream. There is no fallback: if the library is not built, or a call fails,
an exception is raised.

    o, lse = fwd(q, k, v, causal=False, scale=None, exp_mode="auto")
    dq, dk, dv = bwd(q, k, v, o, lse, do, causal=False, scale=None)
    o, lse = fwd_fp8(q, k, v, causal=False, scale=None, rotate=True, seed=0)
    o, lse = fwd_varlen(q, k, v, cu_seqlens, max_seqlen, causal=False)
    dq, dk, dv = bwd_varlen(q, k, v, o, lse, do, cu_seqlens, max_seqlen, causal=False)
    o, lse = fwd_blocksparse(q, k, v, block_mask, causal=False)
    dq, dk, dv = bwd_blocksparse(q, k, v, o, lse, do, block_mask, causal=False)

Tensors are contiguous CUDA (HIP) bfloat16 [B, H, N, d], d ∈ {64, 128};
``scale`` defaults to 1/√d.
"""
import ctypes
import os

from ._lib import FattnError, lib, lib_path  # noqa: F401

__all__ = ["fwd", "bwd", "fwd_varlen", "bwd_varlen", "fwd_blocksparse", "bwd_blocksparse", "fwd_fp8", "fwd_fp8_attend", "fp8_workspace_views", "bwd_workspace_bytes",
           "fp8_workspace_bytes", "FattnError", "lib", "lib_path",
           "EXP_AUTO", "EXP_HW", "EXP_POLY", "EXP_SPLIT"]

EXP_AUTO, EXP_HW, EXP_POLY, EXP_SPLIT = 0, 1, 2, 3
_EXP = {"auto": EXP_AUTO, "hw": EXP_HW, "poly": EXP_POLY, "split": EXP_SPLIT,
        EXP_AUTO: EXP_AUTO, EXP_HW: EXP_HW, EXP_POLY: EXP_POLY, EXP_SPLIT: EXP_SPLIT}


def _torch():
    import torch
    return torch


def _check(t, name, dtype=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shape(q):
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    return tuple(int(x) for x in q.shape)


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _call(status):
    if status != 0:
        raise FattnError(status)


def fwd(q, k, v, causal=False, scale=None, exp_mode="auto", out=None, lse=None):
    """Forward. Returns (O bf16 [B,H,N,d], LSE fp32 [B,H,N])."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, torch.bfloat16)
    B, H, N, d = _shape(q)
    if _shape(k) != (B, H, N, d) or _shape(v) != (B, H, N, d):
        raise ValueError("q, k, v must have the same shape")
    scale = float(d ** -0.5 if scale is None else scale)
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check(o, "out", torch.bfloat16)
    _check(lse_t, "lse", torch.float32)
    with torch.cuda.device(q.device):
        _call(lib().fattn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H, N, d,
                              int(bool(causal)), ctypes.c_float(scale), _EXP[exp_mode],
                              _stream(q)))
    return o, lse_t


def _cu(cu_seqlens, q):
    torch = _torch()
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dtype != torch.int32 \
            or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous() \
            or cu_seqlens.device != q.device or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 tensor of nseq+1 >= 2 "
                         "offsets on the device of q")
    return cu_seqlens.numel() - 1


def fwd_varlen(q, k, v, cu_seqlens, max_seqlen, causal=False, scale=None, exp_mode="auto",
               out=None, lse=None):
    """Forward over packed variable-length sequences: rows [cu[s], cu[s+1]) of
    every head are segment s. Returns (O, LSE) like fwd."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, torch.bfloat16)
    B, H, N, d = _shape(q)
    if _shape(k) != (B, H, N, d) or _shape(v) != (B, H, N, d):
        raise ValueError("q, k, v must have the same shape")
    nseq = _cu(cu_seqlens, q)
    scale = float(d ** -0.5 if scale is None else scale)
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check(o, "out", torch.bfloat16)
    _check(lse_t, "lse", torch.float32)
    with torch.cuda.device(q.device):
        _call(lib().fattn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t),
                                     _ptr(cu_seqlens), nseq, int(max_seqlen), B, H, N, d,
                                     int(bool(causal)), ctypes.c_float(scale), _EXP[exp_mode],
                                     _stream(q)))
    return o, lse_t


def _bmask(block_mask, q):
    torch = _torch()
    B, H, N, _ = _shape(q)
    nb = (N + 127) // 128
    if not isinstance(block_mask, torch.Tensor) or block_mask.dtype != torch.uint8 \
            or not block_mask.is_contiguous() or block_mask.device != q.device \
            or tuple(block_mask.shape) not in ((nb, nb), (B * H, nb, nb)):
        raise ValueError(f"block_mask must be a contiguous uint8 tensor of shape ({nb}, {nb}) "
                         f"or ({B * H}, {nb}, {nb}) on the device of q")
    return int(block_mask.dim() == 3)


def fwd_blocksparse(q, k, v, block_mask, causal=False, scale=None, exp_mode="auto", out=None,
                    lse=None):
    """Block-sparse forward: block_mask is a uint8 tensor on the device of q,
    [nb, nb] for every head or [B*H, nb, nb], nb = ceil(N/128); entry (i, j)
    non-zero makes key block j visible to query block i. Returns (O, LSE)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, torch.bfloat16)
    B, H, N, d = _shape(q)
    if _shape(k) != (B, H, N, d) or _shape(v) != (B, H, N, d):
        raise ValueError("q, k, v must have the same shape")
    per_head = _bmask(block_mask, q)
    scale = float(d ** -0.5 if scale is None else scale)
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check(o, "out", torch.bfloat16)
    _check(lse_t, "lse", torch.float32)
    with torch.cuda.device(q.device):
        _call(lib().fattn_fwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t),
                                          _ptr(block_mask), per_head, B, H, N, d,
                                          int(bool(causal)), ctypes.c_float(scale),
                                          _EXP[exp_mode], _stream(q)))
    return o, lse_t


def fwd_fp8_attend(workspace, B, H, N, d, causal=False, scale=None, want_lse=True, out=None,
                   device=None, exp_mode="auto"):
    """The attention step of fwd_fp8 alone, on a workspace a previous fwd_fp8
    call of the same (B, H, N, d) filled. Returns (O, LSE or None)."""
    torch = _torch()
    scale = float(d ** -0.5 if scale is None else scale)
    dev = workspace.device if device is None else device
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev) if out is None else out
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=dev) if want_lse else None
    with torch.cuda.device(dev):
        _call(lib().fattn_fwd_fp8_attend(_ptr(o), _ptr(lse_t), B, H, N, d, int(bool(causal)),
                                         ctypes.c_float(scale), _EXP[exp_mode], _ptr(workspace),
                                         ctypes.c_size_t(workspace.numel()), _stream(o)))
    return o, lse_t


def bwd_workspace_bytes(B, H, N, d):
    return int(lib().fattn_bwd_workspace_bytes(B, H, N, d))


def bwd(q, k, v, o, lse, do, causal=False, scale=None, workspace=None, out=None):
    """Backward from the forward's O and LSE. Returns (dQ, dK, dV) bf16."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _check(t, n, torch.bfloat16)
    _check(lse, "lse", torch.float32)
    B, H, N, d = _shape(q)
    scale = float(d ** -0.5 if scale is None else scale)
    if out is None:
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    else:
        dq, dk, dv = out
    need = bwd_workspace_bytes(B, H, N, d)
    ws = torch.empty(need, dtype=torch.uint8, device=q.device) if workspace is None else workspace
    with torch.cuda.device(q.device):
        _call(lib().fattn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq),
                              _ptr(dk), _ptr(dv), B, H, N, d, int(bool(causal)),
                              ctypes.c_float(scale), _ptr(ws), ctypes.c_size_t(ws.numel()),
                              _stream(q)))
    return dq, dk, dv


def bwd_varlen(q, k, v, o, lse, do, cu_seqlens, max_seqlen, causal=False, scale=None,
               workspace=None, out=None):
    """Backward of fwd_varlen from its O and LSE. Returns (dQ, dK, dV) bf16."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _check(t, n, torch.bfloat16)
    _check(lse, "lse", torch.float32)
    B, H, N, d = _shape(q)
    nseq = _cu(cu_seqlens, q)
    scale = float(d ** -0.5 if scale is None else scale)
    if out is None:
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    else:
        dq, dk, dv = out
    need = bwd_workspace_bytes(B, H, N, d)
    ws = torch.empty(need, dtype=torch.uint8, device=q.device) if workspace is None else workspace
    with torch.cuda.device(q.device):
        _call(lib().fattn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                                     _ptr(dq), _ptr(dk), _ptr(dv), _ptr(cu_seqlens), nseq,
                                     int(max_seqlen), B, H, N, d, int(bool(causal)),
                                     ctypes.c_float(scale), _ptr(ws), ctypes.c_size_t(ws.numel()),
                                     _stream(q)))
    return dq, dk, dv


def bwd_blocksparse(q, k, v, o, lse, do, block_mask, causal=False, scale=None, workspace=None,
                    out=None):
    """Backward of fwd_blocksparse from its O and LSE. Returns (dQ, dK, dV) bf16."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _check(t, n, torch.bfloat16)
    _check(lse, "lse", torch.float32)
    B, H, N, d = _shape(q)
    per_head = _bmask(block_mask, q)
    scale = float(d ** -0.5 if scale is None else scale)
    if out is None:
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    else:
        dq, dk, dv = out
    need = bwd_workspace_bytes(B, H, N, d)
    ws = torch.empty(need, dtype=torch.uint8, device=q.device) if workspace is None else workspace
    with torch.cuda.device(q.device):
        _call(lib().fattn_bwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                                          _ptr(dq), _ptr(dk), _ptr(dv), _ptr(block_mask), per_head,
                                          B, H, N, d, int(bool(causal)), ctypes.c_float(scale),
                                          _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(q)))
    return dq, dk, dv


def fp8_workspace_bytes(B, H, N, d):
    return int(lib().fattn_fwd_fp8_workspace_bytes(B, H, N, d))


def fp8_workspace_views(ws, B, H, N, d):
    """Views (q8, q8lo, k8, v8t, scales) into an fp8 workspace (uint8 tensor).

    q8, q8lo, k8: uint8 [B,H,N,d] e4m3 codes (q8lo: residual of Q'); v8t: uint8
    [B,H,d,Npad] (V transposed, zero padded to Npad = N rounded up to 64, keys
    permuted inside each 64-key block); scales: fp32 [3, B, H].
    """
    torch = _torch()
    offs = [ctypes.c_size_t() for _ in range(5)]
    _call(lib().fattn_fwd_fp8_workspace_layout(B, H, N, d, *[ctypes.byref(x) for x in offs]))
    oq, oql, ok, ov, osc = (x.value for x in offs)
    npad = (N + 63) // 64 * 64
    n = B * H * N * d
    q8 = ws[oq:oq + n].view(B, H, N, d)
    q8lo = ws[oql:oql + n].view(B, H, N, d)
    k8 = ws[ok:ok + n].view(B, H, N, d)
    v8t = ws[ov:ov + B * H * d * npad].view(B, H, d, npad)
    sc = ws[osc:osc + 12 * B * H].view(torch.float32).view(3, B, H)
    return q8, q8lo, k8, v8t, sc


def fwd_fp8(q, k, v, causal=False, scale=None, rotate=True, seed=0, want_lse=True,
            workspace=None, out=None, exp_mode="auto"):
    """fp8 (e4m3) forward with optional Hadamard rotation. Returns (O, LSE or None)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, torch.bfloat16)
    B, H, N, d = _shape(q)
    scale = float(d ** -0.5 if scale is None else scale)
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if want_lse else None
    need = fp8_workspace_bytes(B, H, N, d)
    ws = torch.empty(need, dtype=torch.uint8, device=q.device) if workspace is None else workspace
    with torch.cuda.device(q.device):
        _call(lib().fattn_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H, N, d,
                                  int(bool(causal)), ctypes.c_float(scale), _EXP[exp_mode],
                                  int(bool(rotate)),
                                  ctypes.c_uint64(seed & (2 ** 64 - 1)), _ptr(ws),
                                  ctypes.c_size_t(ws.numel()), _stream(q)))
    return o, lse_t
