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
    o, lse = fwd_fp8_blocksparse(q, k, v, block_mask, causal=False, rotate=True, seed=0)
    o, lse = fwd_fp8_varlen(q, k, v, cu_seqlens, max_seqlen, causal=False, rotate=True, seed=0)
    dq, dk, dv = bwd_blocksparse(q, k, v, o, lse, do, block_mask, causal=False)

Tensors are contiguous CUDA (HIP) bfloat16 [B, H, N, d], d ∈ {64, 128};
``scale`` defaults to 1/√d.
"""
import ctypes
import os

from ._lib import FattnError, lib, lib_path  # noqa: F401

__all__ = ["fwd", "bwd", "bwd_noalloc", "NOALLOC_WORKSPACE_BYTES", "fwd_varlen", "bwd_varlen", "fwd_blocksparse", "bwd_blocksparse", "fwd_fp8", "fwd_fp8_blocksparse", "fwd_fp8_varlen", "fwd_fp8_attend", "fp8_workspace_views", "bwd_workspace_bytes",
           "fp8_workspace_bytes", "fp8_varlen_workspace_bytes", "FattnError", "lib", "lib_path",
           "EXP_AUTO", "EXP_HW", "EXP_POLY", "EXP_SPLIT"]

EXP_AUTO, EXP_HW, EXP_POLY, EXP_SPLIT = 0, 1, 2, 3
_EXP = {"auto": EXP_AUTO, "hw": EXP_HW, "poly": EXP_POLY, "split": EXP_SPLIT,
        EXP_AUTO: EXP_AUTO, EXP_HW: EXP_HW, EXP_POLY: EXP_POLY, EXP_SPLIT: EXP_SPLIT}


def _torch():
    import torch
    return torch


def _check(t, name, dtype=None, shape=None):
    """Validate one tensor argument before anything reaches the C ABI, which
    sees raw pointers only: a tensor of the wrong shape, dtype or layout would
    otherwise become an out-of-bounds device access. Devices are checked
    afterwards, once for all arguments (`_on_device`), so every shape, dtype
    and layout check runs (and is tested) without a GPU."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_device(ref, named, ref_name="q"):
    """`ref` on a GPU and every (tensor, name) pair on its device (None
    entries skipped)."""
    if ref.device.type != "cuda":
        raise ValueError(f"{ref_name} must be on a GPU device, got {ref.device}")
    for t, n in named:
        if t is not None and t.device != ref.device:
            raise ValueError(f"{n} must be on {ref.device} (the device of {ref_name}), "
                             f"got {t.device}")


def _check_qkv(q, k, v, extra=()):
    """q, k, v (and the tensors in `extra`, (tensor, name) pairs) as bf16
    [B, H, N, d] on q's device; returns (B, H, N, d)."""
    torch = _torch()
    if not isinstance(q, torch.Tensor):
        raise TypeError("q must be a torch.Tensor")
    B, H, N, d = _shape(q)
    _check(q, "q", torch.bfloat16)
    for t, n in ((k, "k"), (v, "v"), *extra):
        _check(t, n, torch.bfloat16, (B, H, N, d))
    return B, H, N, d


def _outputs(q, out, lse, want_lse=True):
    """The caller's (or new) O [B,H,N,d] bf16 and LSE [B,H,N] fp32 buffers."""
    torch = _torch()
    B, H, N, d = _shape(q)
    o = torch.empty_like(q) if out is None else out
    _check(o, "out", torch.bfloat16, (B, H, N, d))
    if not want_lse:
        return o, None
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check(lse_t, "lse", torch.float32, (B, H, N))
    return o, lse_t


def _grads(q, out):
    """The caller's (or new) dQ, dK, dV buffers, bf16 of q's shape."""
    torch = _torch()
    if out is None:
        return tuple(torch.empty_like(q) for _ in range(3))
    if len(out) != 3:
        raise ValueError("out must be a (dq, dk, dv) triple")
    for t, n in zip(out, ("dq", "dk", "dv")):
        _check(t, n, torch.bfloat16, tuple(q.shape))
    return tuple(out)


def _workspace(ws, need, q):
    """The caller's (or a new) uint8 workspace of at least `need` bytes."""
    torch = _torch()
    if ws is None:
        return torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(ws, "workspace", torch.uint8)
    if ws.dim() != 1 or ws.numel() < need:
        raise ValueError(f"workspace must be a 1-D uint8 tensor of at least {need} bytes, "
                         f"got shape {tuple(ws.shape)}")
    return ws


def _shape(q):
    if q.dim() != 4:
        raise ValueError(f"expected a [B, H, N, d] tensor, got shape {tuple(q.shape)}")
    return tuple(int(x) for x in q.shape)


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _call(status):
    if status != 0:
        raise FattnError(status)


def _scale(scale, d):
    return float(d ** -0.5 if scale is None else scale)


def fwd(q, k, v, causal=False, scale=None, exp_mode="auto", out=None, lse=None):
    """Forward. Returns (O bf16 [B,H,N,d], LSE fp32 [B,H,N])."""
    B, H, N, d = _check_qkv(q, k, v)
    o, lse_t = _outputs(q, out, lse)
    _on_device(q, ((k, "k"), (v, "v"), (o, "out"), (lse_t, "lse")))
    with _torch().cuda.device(q.device):
        _call(lib().fattn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H, N, d,
                              int(bool(causal)), ctypes.c_float(_scale(scale, d)),
                              _EXP[exp_mode], _stream(q)))
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
    B, H, N, d = _check_qkv(q, k, v)
    nseq = _cu(cu_seqlens, q)
    o, lse_t = _outputs(q, out, lse)
    _on_device(q, ((k, "k"), (v, "v"), (o, "out"), (lse_t, "lse")))
    with _torch().cuda.device(q.device):
        _call(lib().fattn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t),
                                     _ptr(cu_seqlens), nseq, int(max_seqlen), B, H, N, d,
                                     int(bool(causal)), ctypes.c_float(_scale(scale, d)),
                                     _EXP[exp_mode], _stream(q)))
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
    B, H, N, d = _check_qkv(q, k, v)
    per_head = _bmask(block_mask, q)
    o, lse_t = _outputs(q, out, lse)
    _on_device(q, ((k, "k"), (v, "v"), (o, "out"), (lse_t, "lse")))
    with _torch().cuda.device(q.device):
        _call(lib().fattn_fwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t),
                                          _ptr(block_mask), per_head, B, H, N, d,
                                          int(bool(causal)), ctypes.c_float(_scale(scale, d)),
                                          _EXP[exp_mode], _stream(q)))
    return o, lse_t


def bwd_workspace_bytes(B, H, N, d):
    return int(lib().fattn_bwd_workspace_bytes(B, H, N, d))


def _bwd_args(q, k, v, o, lse, do, out):
    """Validated backward operands: (B, H, N, d, (dq, dk, dv))."""
    torch = _torch()
    B, H, N, d = _check_qkv(q, k, v, extra=((o, "o"), (do, "do")))
    _check(lse, "lse", torch.float32, (B, H, N))
    return B, H, N, d, _grads(q, out)


def bwd(q, k, v, o, lse, do, causal=False, scale=None, workspace=None, out=None):
    """Backward from the forward's O and LSE. Returns (dQ, dK, dV) bf16."""
    B, H, N, d, (dq, dk, dv) = _bwd_args(q, k, v, o, lse, do, out)
    ws = _workspace(workspace, bwd_workspace_bytes(B, H, N, d), q)
    _on_device(q, ((k, "k"), (v, "v"), (o, "o"), (lse, "lse"), (do, "do"), (dq, "dq"),
                   (dk, "dk"), (dv, "dv"), (ws, "workspace")))
    with _torch().cuda.device(q.device):
        _call(lib().fattn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq),
                              _ptr(dk), _ptr(dv), B, H, N, d, int(bool(causal)),
                              ctypes.c_float(_scale(scale, d)), _ptr(ws),
                              ctypes.c_size_t(ws.numel()), _stream(q)))
    return dq, dk, dv


NOALLOC_WORKSPACE_BYTES = 16 << 20  # FATTN_NOALLOC_WORKSPACE_BYTES


def bwd_noalloc(q, k, v, o, lse, do, causal=False, scale=None, out=None):
    """Backward like bwd, through fattn_bwd_noalloc: the row statistics use the
    library's static per-GPU buffer (no workspace argument, nothing allocated
    by the library; with `out` given, nothing allocated at all). Calls that
    overlap on one GPU race. Returns (dQ, dK, dV) bf16."""
    B, H, N, d, (dq, dk, dv) = _bwd_args(q, k, v, o, lse, do, out)
    _on_device(q, ((k, "k"), (v, "v"), (o, "o"), (lse, "lse"), (do, "do"), (dq, "dq"),
                   (dk, "dk"), (dv, "dv")))
    with _torch().cuda.device(q.device):
        _call(lib().fattn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                                      _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d,
                                      int(bool(causal)), ctypes.c_float(_scale(scale, d)),
                                      _stream(q)))
    return dq, dk, dv


def bwd_varlen(q, k, v, o, lse, do, cu_seqlens, max_seqlen, causal=False, scale=None,
               workspace=None, out=None):
    """Backward of fwd_varlen from its O and LSE. Returns (dQ, dK, dV) bf16."""
    B, H, N, d, (dq, dk, dv) = _bwd_args(q, k, v, o, lse, do, out)
    nseq = _cu(cu_seqlens, q)
    ws = _workspace(workspace, bwd_workspace_bytes(B, H, N, d), q)
    _on_device(q, ((k, "k"), (v, "v"), (o, "o"), (lse, "lse"), (do, "do"), (dq, "dq"),
                   (dk, "dk"), (dv, "dv"), (ws, "workspace")))
    with _torch().cuda.device(q.device):
        _call(lib().fattn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                                     _ptr(dq), _ptr(dk), _ptr(dv), _ptr(cu_seqlens), nseq,
                                     int(max_seqlen), B, H, N, d, int(bool(causal)),
                                     ctypes.c_float(_scale(scale, d)), _ptr(ws),
                                     ctypes.c_size_t(ws.numel()), _stream(q)))
    return dq, dk, dv


def bwd_blocksparse(q, k, v, o, lse, do, block_mask, causal=False, scale=None, workspace=None,
                    out=None):
    """Backward of fwd_blocksparse from its O and LSE. Returns (dQ, dK, dV) bf16."""
    B, H, N, d, (dq, dk, dv) = _bwd_args(q, k, v, o, lse, do, out)
    per_head = _bmask(block_mask, q)
    ws = _workspace(workspace, bwd_workspace_bytes(B, H, N, d), q)
    _on_device(q, ((k, "k"), (v, "v"), (o, "o"), (lse, "lse"), (do, "do"), (dq, "dq"),
                   (dk, "dk"), (dv, "dv"), (ws, "workspace")))
    with _torch().cuda.device(q.device):
        _call(lib().fattn_bwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                                          _ptr(dq), _ptr(dk), _ptr(dv), _ptr(block_mask), per_head,
                                          B, H, N, d, int(bool(causal)),
                                          ctypes.c_float(_scale(scale, d)), _ptr(ws),
                                          ctypes.c_size_t(ws.numel()), _stream(q)))
    return dq, dk, dv


def fp8_workspace_bytes(B, H, N, d):
    return int(lib().fattn_fwd_fp8_workspace_bytes(B, H, N, d))


def fp8_workspace_views(ws, B, H, N, d):
    """Views (k8, v8t, scales) into an fp8 workspace (uint8 tensor).

    k8: uint8 [B,H,N,d] e4m3 codes of K'; v8t: uint8 [B,H,d,Npad] (V
    transposed, zero padded to Npad = N rounded up to 64, keys permuted inside
    each 64-key block); scales: fp32 [B, H, ceil(N/128), 2], the (K', V) pair
    of each chunk of 128 keys. Q' is quantised inside the attention kernel and
    not stored.
    """
    torch = _torch()
    offs = [ctypes.c_size_t() for _ in range(3)]
    _call(lib().fattn_fwd_fp8_workspace_layout(B, H, N, d, *[ctypes.byref(x) for x in offs]))
    ok, ov, osc = (x.value for x in offs)
    npad = (N + 63) // 64 * 64
    nch = (N + 127) // 128
    n = B * H * N * d
    k8 = ws[ok:ok + n].view(B, H, N, d)
    v8t = ws[ov:ov + B * H * d * npad].view(B, H, d, npad)
    sc = ws[osc:osc + 8 * B * H * nch].view(torch.float32).view(B, H, nch, 2)
    return k8, v8t, sc


def fwd_fp8(q, k, v, causal=False, scale=None, rotate=True, seed=0, want_lse=True,
            workspace=None, out=None, exp_mode="auto"):
    """fp8 (e4m3) forward with optional Hadamard rotation. Returns (O, LSE or None)."""
    B, H, N, d = _check_qkv(q, k, v)
    o, lse_t = _outputs(q, out, None, want_lse)
    ws = _workspace(workspace, fp8_workspace_bytes(B, H, N, d), q)
    _on_device(q, ((k, "k"), (v, "v"), (o, "out"), (ws, "workspace")))
    with _torch().cuda.device(q.device):
        _call(lib().fattn_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H, N, d,
                                  int(bool(causal)), ctypes.c_float(_scale(scale, d)),
                                  _EXP[exp_mode], int(bool(rotate)),
                                  ctypes.c_uint64(seed & (2 ** 64 - 1)), _ptr(ws),
                                  ctypes.c_size_t(ws.numel()), _stream(q)))
    return o, lse_t


def fwd_fp8_blocksparse(q, k, v, block_mask, causal=False, scale=None, rotate=True, seed=0,
                        want_lse=True, workspace=None, out=None, exp_mode="auto"):
    """fwd_fp8 restricted by a block mask (as for fwd_blocksparse): the same
    quantisation, attention over the visible key blocks only. Returns
    (O, LSE or None)."""
    B, H, N, d = _check_qkv(q, k, v)
    per_head = _bmask(block_mask, q)
    o, lse_t = _outputs(q, out, None, want_lse)
    ws = _workspace(workspace, fp8_workspace_bytes(B, H, N, d), q)
    _on_device(q, ((k, "k"), (v, "v"), (o, "out"), (ws, "workspace")))
    with _torch().cuda.device(q.device):
        _call(lib().fattn_fwd_fp8_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t),
                                              _ptr(block_mask), per_head, B, H, N, d,
                                              int(bool(causal)), ctypes.c_float(_scale(scale, d)),
                                              _EXP[exp_mode], int(bool(rotate)),
                                              ctypes.c_uint64(seed & (2 ** 64 - 1)), _ptr(ws),
                                              ctypes.c_size_t(ws.numel()), _stream(q)))
    return o, lse_t


def fp8_varlen_workspace_bytes(B, H, N, d, nseq, max_seqlen):
    return int(lib().fattn_fwd_fp8_varlen_workspace_bytes(B, H, N, d, nseq, max_seqlen))


def fwd_fp8_varlen(q, k, v, cu_seqlens, max_seqlen, causal=False, scale=None, rotate=True, seed=0,
                   want_lse=True, workspace=None, out=None, exp_mode="auto"):
    """fwd_fp8 over packed variable-length sequences (cu_seqlens, max_seqlen
    as for fwd_varlen); each segment is quantised and attended as a sequence
    of its own. Returns (O, LSE or None)."""
    B, H, N, d = _check_qkv(q, k, v)
    nseq = _cu(cu_seqlens, q)
    o, lse_t = _outputs(q, out, None, want_lse)
    need = fp8_varlen_workspace_bytes(B, H, N, d, nseq, max(1, int(max_seqlen)))
    ws = _workspace(workspace, need, q)
    _on_device(q, ((k, "k"), (v, "v"), (o, "out"), (ws, "workspace")))
    with _torch().cuda.device(q.device):
        _call(lib().fattn_fwd_fp8_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t),
                                         _ptr(cu_seqlens), nseq, int(max_seqlen), B, H, N, d,
                                         int(bool(causal)), ctypes.c_float(_scale(scale, d)),
                                         _EXP[exp_mode], int(bool(rotate)),
                                         ctypes.c_uint64(seed & (2 ** 64 - 1)), _ptr(ws),
                                         ctypes.c_size_t(ws.numel()), _stream(q)))
    return o, lse_t


def fwd_fp8_attend(q, workspace, causal=False, scale=None, rotate=True, seed=0, want_lse=True,
                   out=None, exp_mode="auto"):
    """The attention step of fwd_fp8 alone: q (bf16 [B,H,N,d]) against the K/V
    operands a previous fwd_fp8 call of the same shape, rotate and seed left
    in `workspace`. Returns (O, LSE or None)."""
    torch = _torch()
    _check(q, "q", torch.bfloat16)
    B, H, N, d = _shape(q)
    _check(workspace, "workspace", torch.uint8)
    ws = _workspace(workspace, fp8_workspace_bytes(B, H, N, d), q)
    o, lse_t = _outputs(q, out, None, want_lse)
    _on_device(q, ((ws, "workspace"), (o, "out"), (lse_t, "lse")))
    with torch.cuda.device(q.device):
        _call(lib().fattn_fwd_fp8_attend(_ptr(q), _ptr(o), _ptr(lse_t), B, H, N, d,
                                         int(bool(causal)), ctypes.c_float(_scale(scale, d)),
                                         _EXP[exp_mode], int(bool(rotate)),
                                         ctypes.c_uint64(seed & (2 ** 64 - 1)), _ptr(ws),
                                         ctypes.c_size_t(ws.numel()), _stream(q)))
    return o, lse_t
