"""The Python binding rejects malformed tensor arguments before any library
call: wrong shapes, dtypes, layouts, output buffers and workspaces raise
(the C ABI sees raw pointers only, so any of them would otherwise become an
out-of-bounds device access). Runs without a GPU: every layout check comes
before the device check, and CPU tensors of the right layout reach the
device check and fail there."""
import pytest
import torch

import tiled_attention_fattn_amd as fa

B, H, N, D = 1, 2, 16, 64
bf = torch.bfloat16


def t(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


q = t(B, H, N, D)
lse = t(B, H, N, dtype=torch.float32)


@pytest.mark.parametrize("call,msg", [
    (lambda: fa.fwd(q, t(B, H, N + 1, D), q), "k must have shape"),
    (lambda: fa.fwd(q, q, t(B, H, N, D, dtype=torch.float16)), "v must be"),
    (lambda: fa.fwd(t(H, N, D), q, q), r"\[B, H, N, d\]"),
    (lambda: fa.fwd(q.float(), q, q), "q must be"),
    (lambda: fa.fwd(q, q.transpose(2, 3).contiguous().transpose(2, 3), q), "k must be contiguous"),
    (lambda: fa.fwd(q, q, q, out=t(B, H, N, D - 1)), "out must have shape"),
    (lambda: fa.fwd(q, q, q, out=t(B, H, N, D, dtype=torch.float32)), "out must be"),
    (lambda: fa.fwd(q, q, q, lse=t(B, H, N + 1, dtype=torch.float32)), "lse must have shape"),
    (lambda: fa.fwd(q, q, q, lse=t(B, H, N)), "lse must be"),
    (lambda: fa.bwd(q, q, q, t(B, H, N, 2 * D), lse, q), "o must have shape"),
    (lambda: fa.bwd(q, q, q, q, lse, t(B, H, 1, D)), "do must have shape"),
    (lambda: fa.bwd(q, q, q, q, t(B, H, N - 1, dtype=torch.float32), q), "lse must have shape"),
    (lambda: fa.bwd(q, q, q, q, t(B, H, N), q), "lse must be"),
    (lambda: fa.bwd(q, q, q, q, lse, q, out=(q, q)), "triple"),
    (lambda: fa.bwd(q, q, q, q, lse, q, out=(q, q, t(B, H, N, D, dtype=torch.float32))),
     "dv must be"),
    (lambda: fa.bwd(q, q, q, q, lse, q, out=(q, t(1, 1, N, D), q)), "dk must have shape"),
    (lambda: fa.bwd(q, q, q, q, lse, q, workspace=t(8, dtype=torch.uint8)), "at least"),
    (lambda: fa.bwd(q, q, q, q, lse, q, workspace=t(10 ** 6, dtype=torch.float32)),
     "workspace must be"),
    (lambda: fa.bwd_varlen(q, q, q, q, lse, t(B, H, N, D + 64), torch.tensor([0, N], dtype=torch.int32), N),
     "do must have shape"),
    (lambda: fa.bwd_blocksparse(q, q, q, q, lse, q, t(1, 1, dtype=torch.uint8), out=(q, q, q[:, :1])),
     "dv must have shape"),
    (lambda: fa.fwd_fp8(q, q, t(B, H, N, D, dtype=torch.float32)), "v must be"),
    (lambda: fa.fwd_fp8(q, q, q, out=t(B, H, N, D, dtype=torch.float16)), "out must be"),
    (lambda: fa.fwd_fp8(q, q, q, workspace=t(64, dtype=torch.uint8)), "at least"),
    (lambda: fa.fwd_fp8_blocksparse(q, q, q, t(2, 2, dtype=torch.uint8)), "block_mask must be"),
    (lambda: fa.fwd_fp8_blocksparse(q, q, q, t(1, 1, dtype=torch.float32)), "block_mask must be"),
    (lambda: fa.fwd_fp8_blocksparse(q, q, q, t(1, 1, dtype=torch.uint8),
                                    workspace=t(64, dtype=torch.uint8)), "at least"),
    (lambda: fa.fwd_fp8_varlen(q, q, q, t(3, dtype=torch.int64), N), "cu_seqlens must be"),
    (lambda: fa.fwd_fp8_varlen(q, q, q, t(1, dtype=torch.int32), N), "cu_seqlens must be"),
    (lambda: fa.fwd_fp8_varlen(q, q, q, t(3, dtype=torch.int32), N,
                               workspace=t(64, dtype=torch.uint8)), "at least"),
    (lambda: fa.fwd_fp8_attend(q, t(64, dtype=torch.uint8)), "at least"),
    (lambda: fa.fwd_fp8_attend(q, None), "workspace must be"),
    (lambda: fa.fwd_fp8_attend(t(B, H, N, D, dtype=torch.float32), t(10 ** 6, dtype=torch.uint8)),
     "q must be"),
    (lambda: fa.fwd_fp8_attend(q, t(10 ** 6, dtype=torch.uint8), out=t(B, H, N, D + 1)),
     "out must have shape"),
])
def test_malformed_arguments_raise_before_any_call(call, msg):
    with pytest.raises((ValueError, TypeError), match=msg):
        call()


@pytest.mark.parametrize("call", [
    lambda: fa.fwd(q, q, q),
    lambda: fa.bwd(q, q, q, q, lse, q),
    lambda: fa.fwd_fp8(q, q, q),
    lambda: fa.fwd_fp8_attend(q, t(10 ** 6, dtype=torch.uint8)),
    lambda: fa.fwd_fp8_blocksparse(q, q, q, t(1, 1, dtype=torch.uint8)),
    lambda: fa.fwd_fp8_varlen(q, q, q, t(3, dtype=torch.int32), N),
])
def test_well_formed_cpu_tensors_reach_the_device_check(call):
    with pytest.raises(ValueError, match="must be on a GPU device"):
        call()
