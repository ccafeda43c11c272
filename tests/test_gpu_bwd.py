"""GPU parity of the bf16 backward (libfattn fattn_bwd) against the float64 oracle.

O and LSE come from the GPU forward, as in training. Small shapes are compared
element by element with the full oracle (several 128-key and 64-query tiles,
ragged tails, N = 1, both head dimensions, causal and not). The backward
workload (causal B=4 H=16 N=4096 d=128) runs at full size in the launch
configuration the bench times and is compared on whole sampled heads.
"""
import numpy as np
import pytest

from oracle.attention import attention_backward
from tests.parity import assert_bf16_close, to_np
from tiled_attention_fattn_amd.inputs import WORKLOADS, gen_workload, to_device_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _run(k, shape, causal, poison=False):
    import tiled_attention_fattn_amd as fa
    inp = gen_workload(k, names=("q", "k", "v", "do"), shape=shape)
    q, kk, v, do = (to_device_bf16(inp[n][1]) for n in ("q", "k", "v", "do"))
    scale = shape[-1] ** -0.5
    print(f"[bwd] seed={k} shape={shape} causal={causal}", flush=True)
    o, lse = fa.fwd(q, kk, v, causal=causal, scale=scale)
    # poison: outputs prefilled with NaN, so an element no workgroup writes shows
    out = tuple(torch.full_like(q, float("nan")) for _ in range(3)) if poison else None
    dq, dk, dv = fa.bwd(q, kk, v, o, lse, do, causal=causal, scale=scale, out=out)
    torch.cuda.synchronize()
    return inp, (dq, dk, dv), scale


SMALL = [
    (31, (1, 1, 1, 128), False),
    (32, (1, 2, 7, 64), True),
    (33, (1, 2, 64, 128), True),
    (34, (2, 2, 200, 128), False),
    (35, (2, 2, 200, 128), True),
    (36, (1, 3, 300, 64), True),
    (37, (1, 1, 513, 128), True),
    (38, (1, 2, 384, 128), False),
    (39, (2, 1, 129, 64), False),
]


@pytest.mark.parametrize("k,shape,causal", SMALL)
def test_bwd_matches_oracle(k, shape, causal):
    inp, grads, scale = _run(k, shape, causal)
    ref = attention_backward(inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], causal, scale)
    for name, got, r in zip(("dQ", "dK", "dV"), grads, ref[:3]):
        assert_bf16_close(to_np(got), r, f"{name} {shape} causal={causal}")


def test_bwd_full_size_sampled_heads():
    w = WORKLOADS[4]
    shape = (w["B"], w["H"], w["N"], w["d"])
    inp, grads, scale = _run(4, shape, w["causal"], poison=True)
    # Every element of every gradient written (the whole grid of the bench's launch).
    for name, g in zip(("dQ", "dK", "dV"), grads):
        assert not torch.isnan(g).any().item(), f"{name}: elements left unwritten"
    for (b, h) in [(0, 0), (w["B"] - 1, w["H"] - 1), (2, 7)]:
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = attention_backward(inp["q"][0][sl], inp["k"][0][sl], inp["v"][0][sl],
                                 inp["do"][0][sl], w["causal"], scale)
        for name, got, r in zip(("dQ", "dK", "dV"), grads, ref[:3]):
            assert_bf16_close(to_np(got[b:b + 1, h:h + 1]), r, f"{name} {w['name']} b={b} h={h}")


def test_bwd_invariants_on_gpu_outputs():
    # Σ_j dK_j = 0 and Σ_j dV_j = Σ_i dO_i hold for the exact gradients; the GPU
    # sums must match them to the bf16 tolerance scaled by √N.
    shape = (1, 2, 512, 128)
    inp, (dq, dk, dv), _ = _run(40, shape, True)
    n = shape[2]
    dk_sum = to_np(dk).sum(axis=2)
    assert np.max(np.abs(dk_sum)) < 2e-2 * np.sqrt(n)
    dv_sum = to_np(dv).sum(axis=2)
    do_sum = inp["do"][0].sum(axis=2)
    assert np.max(np.abs(dv_sum - do_sum)) < 2e-2 * np.sqrt(n)


def test_bwd_single_token_and_writes_everything():
    import tiled_attention_fattn_amd as fa
    shape = (2, 3, 1, 64)
    inp = gen_workload(41, names=("q", "k", "v", "do"), shape=shape)
    q, k, v, do = (to_device_bf16(inp[n][1]) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v)
    outs = tuple(torch.full_like(q, float("nan")) for _ in range(3))
    fa.bwd(q, k, v, o, lse, do, out=outs)
    torch.cuda.synchronize()
    dq, dk, dv = (to_np(t) for t in outs)
    # exact gradients: dQ = dK = 0 and dV = dO; the kernel's dS = P·(dP − D) is
    # a difference of two fp32 sums of the same products, so it is zero only up
    # to rounding.
    assert np.all(np.isfinite(dq)) and np.all(np.isfinite(dk))
    assert np.max(np.abs(dq)) <= 1e-5 and np.max(np.abs(dk)) <= 1e-5
    assert_bf16_close(dv, inp["do"][0], "dV at N=1")


def test_bwd_bitwise_reproducible():
    # No global atomics anywhere in the backward: two calls give identical bits.
    import tiled_attention_fattn_amd as fa
    shape = (2, 2, 777, 128)
    inp = gen_workload(42, names=("q", "k", "v", "do"), shape=shape)
    q, k, v, do = (to_device_bf16(inp[n][1]) for n in ("q", "k", "v", "do"))
    print(f"[bwd] reproducible shape={shape}", flush=True)
    o, lse = fa.fwd(q, k, v, causal=True)
    g1 = fa.bwd(q, k, v, o, lse, do, causal=True)
    g2 = fa.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
