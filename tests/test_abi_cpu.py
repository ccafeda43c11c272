"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/fattn.h, and rejects bad arguments on the host before any
HIP call (fake, aligned, non-null device addresses are never dereferenced)."""
import ctypes
import os
import re

import pytest

import tiled_attention_fattn_amd as fa
from tiled_attention_fattn_amd._lib import PROTOTYPES

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "fattn.h")

OK, EINVAL, ENOTSUP, EWORKSPACE = 0, 1, 2, 3
P = ctypes.c_void_p(0x10000)           # aligned fake device address
MIS = ctypes.c_void_p(0x10008)         # 8-byte aligned only
NUL = ctypes.c_void_p(0)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(fattn_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = fa.lib()
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), f"{n} missing from libfattn.so"
        assert n in PROTOTYPES, f"{n} has no ctypes prototype"
    assert lib.fattn_version() >= 100


def test_strerror_covers_codes():
    lib = fa.lib()
    for s in range(6):
        assert lib.fattn_strerror(s)
    assert b"unknown" in lib.fattn_strerror(99)


def fwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=16, d=128, causal=0, scale=0.1, exp=0)
    a.update(kw)
    return fa.lib().fattn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"],
                              a["d"], a["causal"], ctypes.c_float(a["scale"]), a["exp"], NUL)


@pytest.mark.parametrize("kw,code", [
    (dict(q=NUL), EINVAL), (dict(k=NUL), EINVAL), (dict(v=NUL), EINVAL), (dict(o=NUL), EINVAL),
    (dict(lse=NUL), EINVAL), (dict(q=MIS), EINVAL), (dict(B=0), EINVAL), (dict(H=-1), EINVAL),
    (dict(N=0), EINVAL), (dict(d=96), ENOTSUP), (dict(d=256), ENOTSUP), (dict(causal=2), EINVAL),
    (dict(scale=0.0), EINVAL), (dict(scale=-1.0), EINVAL), (dict(scale=float("inf")), EINVAL),
    (dict(scale=float("nan")), EINVAL), (dict(exp=4), EINVAL), (dict(exp=-1), EINVAL),
    (dict(B=4096, H=64, N=8192, d=128), ENOTSUP),
])
def test_fwd_rejects_bad_arguments(kw, code):
    assert fwd(**kw) == code
    assert fa.lib().fattn_last_error()


def test_bwd_workspace_checks():
    lib = fa.lib()
    need = lib.fattn_bwd_workspace_bytes(2, 3, 100, 64)
    assert need >= 2 * 4 * 2 * 3 * 128
    assert need % 256 == 0
    assert lib.fattn_bwd_workspace_bytes(0, 1, 1, 64) == 0

    def call(ws, nbytes, **kw):
        a = dict(B=2, H=3, N=100, d=64, causal=1, scale=0.125)
        a.update(kw)
        return lib.fattn_bwd(P, P, P, P, P, P, P, P, P, a["B"], a["H"], a["N"], a["d"],
                             a["causal"], ctypes.c_float(a["scale"]), ws, nbytes, NUL)
    assert call(NUL, need) == EWORKSPACE
    assert call(ctypes.c_void_p(0x10010), need) == EWORKSPACE      # not 256-aligned
    assert call(P, need - 1) == EWORKSPACE
    assert call(P, need, d=32) == ENOTSUP
    assert call(P, need, N=0) == EINVAL


def test_fp8_workspace_layout_and_checks():
    lib = fa.lib()
    B, H, N, d = 2, 3, 100, 128
    need = lib.fattn_fwd_fp8_workspace_bytes(B, H, N, d)
    offs = [ctypes.c_size_t() for _ in range(3)]
    assert lib.fattn_fwd_fp8_workspace_layout(B, H, N, d, *[ctypes.byref(x) for x in offs]) == OK
    ok, ov, osc = (x.value for x in offs)
    npad = 128
    n = B * H * N * d
    assert ok == 0 and ov >= ok + n
    # then the scales: a (K', V) fp32 pair per (b, h) and chunk of 128 keys
    assert osc >= ov + B * H * d * npad
    assert need == (osc + 8 * B * H * ((N + 127) // 128) + 255) // 256 * 256
    assert all(x % 256 == 0 for x in (ok, ov, osc))

    def call(ws, nbytes, **kw):
        a = dict(rotate=1, lse=P, d=d, exp=0)
        a.update(kw)
        return lib.fattn_fwd_fp8(P, P, P, P, a["lse"], B, H, N, a["d"], 0, ctypes.c_float(0.1),
                                 a["exp"], a["rotate"], ctypes.c_uint64(7), ws, nbytes, NUL)
    assert call(P, need - 1) == EWORKSPACE
    assert call(NUL, need) == EWORKSPACE
    assert call(P, need, rotate=2) == EINVAL
    assert call(P, need, exp=4) == EINVAL
    assert call(P, need, exp=-1) == EINVAL
    assert call(P, need, lse=MIS) == EINVAL
    assert call(P, need, d=80) == ENOTSUP


def test_fp8_attend_checks():
    lib = fa.lib()
    B, H, N, d = 2, 3, 100, 128
    need = lib.fattn_fwd_fp8_workspace_bytes(B, H, N, d)

    def call(ws, nbytes, **kw):
        a = dict(q=P, o=P, lse=NUL, B=B, H=H, N=N, d=d, causal=0, scale=0.1, exp=0, rotate=1)
        a.update(kw)
        return lib.fattn_fwd_fp8_attend(a["q"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                                        a["causal"], ctypes.c_float(a["scale"]), a["exp"],
                                        a["rotate"], ctypes.c_uint64(7), ws, nbytes, NUL)
    assert call(NUL, need) == EWORKSPACE
    assert call(P, need, q=NUL) == EINVAL
    assert call(P, need, q=MIS) == EINVAL
    assert call(P, need, rotate=2) == EINVAL
    assert call(P, need - 1) == EWORKSPACE
    assert call(MIS, need) in (EINVAL, EWORKSPACE)
    assert call(P, need, o=NUL) == EINVAL
    assert call(P, need, lse=MIS) == EINVAL
    assert call(P, need, d=96) == ENOTSUP
    assert call(P, need, N=0) == EINVAL
    assert call(P, need, scale=float("nan")) == EINVAL
    assert call(P, need, causal=3) == EINVAL
    assert call(P, need, exp=5) == EINVAL


def fwd_varlen(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, cu=P, nseq=3, maxl=16, B=1, H=2, N=40, d=128, causal=1,
             scale=0.1, exp=0)
    a.update(kw)
    return fa.lib().fattn_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"],
                                     a["nseq"], a["maxl"], a["B"], a["H"], a["N"], a["d"],
                                     a["causal"], ctypes.c_float(a["scale"]), a["exp"], NUL)


@pytest.mark.parametrize("kw,code", [
    (dict(cu=NUL), EINVAL), (dict(cu=ctypes.c_void_p(0x10002)), EINVAL), (dict(nseq=0), EINVAL),
    (dict(maxl=0), EINVAL), (dict(maxl=41), EINVAL), (dict(q=NUL), EINVAL), (dict(d=80), ENOTSUP),
    (dict(causal=2), EINVAL), (dict(exp=7), EINVAL), (dict(N=0), EINVAL),
    (dict(B=1, H=1, N=16384, d=64, nseq=1 << 24, maxl=16384), ENOTSUP),  # grid size
])
def test_fwd_varlen_rejects_bad_arguments(kw, code):
    assert fwd_varlen(**kw) == code
    assert fa.lib().fattn_last_error()


def test_bwd_varlen_checks():
    lib = fa.lib()
    B, H, N, d = 1, 2, 40, 64
    need = lib.fattn_bwd_workspace_bytes(B, H, N, d)

    def call(ws, nbytes, **kw):
        a = dict(cu=P, nseq=2, maxl=30, dq=P)
        a.update(kw)
        return lib.fattn_bwd_varlen(P, P, P, P, P, P, a["dq"], P, P, a["cu"], a["nseq"], a["maxl"],
                                    B, H, N, d, 0, ctypes.c_float(0.125), ws, nbytes, NUL)
    assert call(P, need - 1) == EWORKSPACE
    assert call(NUL, need) == EWORKSPACE
    assert call(MIS, need) == EWORKSPACE
    assert call(P, need, cu=NUL) == EINVAL
    assert call(P, need, nseq=-1) == EINVAL
    assert call(P, need, maxl=N + 1) == EINVAL
    assert call(P, need, dq=MIS) == EINVAL


def test_fwd_blocksparse_checks():
    lib = fa.lib()

    def call(**kw):
        a = dict(q=P, mask=P, per_head=0, N=300, d=128, causal=0, scale=0.1, exp=0)
        a.update(kw)
        return lib.fattn_fwd_blocksparse(a["q"], P, P, P, P, a["mask"], a["per_head"], 1, 2, a["N"],
                                         a["d"], a["causal"], ctypes.c_float(a["scale"]), a["exp"],
                                         NUL)
    assert call(mask=NUL) == EINVAL
    assert call(per_head=2) == EINVAL
    assert call(q=MIS) == EINVAL
    assert call(d=32) == ENOTSUP
    assert call(N=40000) == ENOTSUP
    assert call(causal=5) == EINVAL
    assert call(exp=9) == EINVAL
    assert call(scale=-2.0) == EINVAL
    assert fa.lib().fattn_last_error()


def test_fp8_blocksparse_checks():
    lib = fa.lib()
    B, H, N, d = 1, 2, 300, 128
    need = lib.fattn_fwd_fp8_workspace_bytes(B, H, N, d)

    def call(ws, nbytes, **kw):
        a = dict(q=P, mask=P, per_head=0, N=N, d=d, causal=0, exp=0, rotate=1, lse=NUL)
        a.update(kw)
        return lib.fattn_fwd_fp8_blocksparse(a["q"], P, P, P, a["lse"], a["mask"], a["per_head"],
                                             B, H, a["N"], a["d"], a["causal"],
                                             ctypes.c_float(0.1), a["exp"], a["rotate"],
                                             ctypes.c_uint64(7), ws, nbytes, NUL)
    assert call(P, need, mask=NUL) == EINVAL
    assert call(P, need, per_head=2) == EINVAL
    assert call(P, need, q=MIS) == EINVAL
    assert call(P, need, lse=MIS) == EINVAL
    assert call(P, need, d=80) == ENOTSUP
    assert call(P, need, causal=3) == EINVAL
    assert call(P, need, exp=7) == EINVAL
    assert call(P, need, rotate=-1) == EINVAL
    assert call(P, need - 1) == EWORKSPACE
    assert call(NUL, need) == EWORKSPACE
    assert call(P, lib.fattn_fwd_fp8_workspace_bytes(B, H, 40000, d), N=40000) == ENOTSUP
    assert fa.lib().fattn_last_error()


def test_fp8_varlen_workspace_and_checks():
    lib = fa.lib()
    B, H, N, d, nseq, maxl = 1, 2, 300, 128, 3, 200
    need = lib.fattn_fwd_fp8_varlen_workspace_bytes(B, H, N, d, nseq, maxl)
    # K8, V8ᵀ with 64 more columns per segment, a scale pair per (head,
    # segment) and chunk of 128 keys of the longest segment, each region
    # 256-byte aligned.
    npad = (N + 63) // 64 * 64 + 64 * nseq
    r = lambda x: (x + 255) // 256 * 256
    assert need == r(r(r(B * H * N * d) + B * H * d * npad) + 8 * B * H * nseq * ((maxl + 127) // 128))
    assert need > lib.fattn_fwd_fp8_workspace_bytes(B, H, N, d)
    assert lib.fattn_fwd_fp8_varlen_workspace_bytes(B, H, N, d, 0, maxl) == 0

    def call(ws, nbytes, **kw):
        a = dict(q=P, cu=P, nseq=nseq, maxl=maxl, N=N, d=d, causal=0, exp=0, rotate=1, lse=NUL)
        a.update(kw)
        return lib.fattn_fwd_fp8_varlen(a["q"], P, P, P, a["lse"], a["cu"], a["nseq"], a["maxl"],
                                        B, H, a["N"], a["d"], a["causal"], ctypes.c_float(0.1),
                                        a["exp"], a["rotate"], ctypes.c_uint64(7), ws, nbytes,
                                        NUL)
    assert call(P, need, cu=NUL) == EINVAL
    assert call(P, need, nseq=0) == EINVAL
    assert call(P, need, maxl=0) == EINVAL
    assert call(P, need, maxl=N + 1) == EINVAL
    assert call(P, need, q=MIS) == EINVAL
    assert call(P, need, lse=MIS) == EINVAL
    assert call(P, need, d=80) == ENOTSUP
    assert call(P, need, rotate=3) == EINVAL
    assert call(P, need, exp=5) == EINVAL
    assert call(P, need - 1) == EWORKSPACE
    assert call(NUL, need) == EWORKSPACE
    # V8ᵀ rows of d·(N + 64·nseq) bytes must stay addressable with 32 bits.
    big = 2 ** 24
    assert call(P, need, nseq=big // 64, maxl=1) == ENOTSUP
    assert fa.lib().fattn_last_error()


def test_bwd_blocksparse_checks():
    lib = fa.lib()
    B, H, N, d = 1, 2, 300, 128
    need = lib.fattn_bwd_workspace_bytes(B, H, N, d)

    def call(ws, nbytes, **kw):
        a = dict(mask=P, per_head=0, N=N, dk=P)
        a.update(kw)
        return lib.fattn_bwd_blocksparse(P, P, P, P, P, P, P, a["dk"], P, a["mask"], a["per_head"],
                                         B, H, a["N"], d, 0, ctypes.c_float(0.1), ws, nbytes, NUL)
    assert call(P, need - 1) == EWORKSPACE
    assert call(NUL, need) == EWORKSPACE
    assert call(P, need, mask=NUL) == EINVAL
    assert call(P, need, per_head=-1) == EINVAL
    assert call(P, need, dk=MIS) == EINVAL
    assert call(P, lib.fattn_bwd_workspace_bytes(B, H, 40000, d), N=40000) == ENOTSUP


def test_bwd_noalloc_checks():
    # Rejections only (a call that passes every check would launch on fake
    # pointers): sizes past the static workspace, and the fattn_bwd checks.
    lib = fa.lib()
    cap = 16 << 20
    assert lib.fattn_bwd_workspace_bytes(1, 32, 65536, 64) == cap   # exactly at the limit

    def call(**kw):
        a = dict(q=P, dv=P, B=1, H=2, N=100, d=128, causal=1, scale=0.1)
        a.update(kw)
        return lib.fattn_bwd_noalloc(a["q"], P, P, P, P, P, P, P, a["dv"], a["B"], a["H"],
                                     a["N"], a["d"], a["causal"], ctypes.c_float(a["scale"]), NUL)
    assert call(B=1, H=32, N=65537, d=64) == EWORKSPACE     # one 64-row block past the limit
    assert b"static workspace" in lib.fattn_last_error()
    assert call(B=16, H=16, N=32768, d=64) == EWORKSPACE
    assert call(q=NUL) == EINVAL
    assert call(dv=MIS) == EINVAL
    assert call(d=96) == ENOTSUP
    assert call(N=0) == EINVAL
    assert call(causal=2) == EINVAL
    assert call(scale=0.0) == EINVAL
    assert call(B=4096, H=64, N=8192, d=128) == ENOTSUP
