"""GPU parity of the bf16 forward (libfattn fattn_fwd) against the float64 oracle.

Small shapes are compared element by element with the full oracle; they span
several 128-row query tiles and 64-key tiles, ragged tails, N = 1, both head
dimensions, and a ragged N above 4096 where the non-causal d=128 launch uses
256-query workgroups. The two throughput workloads (causal B=8 H=16 N=2048 and
non-causal B=2 H=16 N=8192, d=128) run at full size in the launch
configuration the bench times and are compared on sampled heads and rows.
"""
import numpy as np
import pytest

from oracle.attention import attention_forward, attention_forward_rows
from tests.parity import assert_bf16_close, assert_lse_close, to_np
from tiled_attention_fattn_amd.inputs import WORKLOADS, gen_workload, to_device_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _run(k, shape, causal, exp_mode, scale=None, poison=False):
    import tiled_attention_fattn_amd as fa
    inp = gen_workload(k, shape=shape)
    q, kk, v = (to_device_bf16(inp[n][1]) for n in ("q", "k", "v"))
    d = shape[-1]
    scale = d ** -0.5 if scale is None else scale
    print(f"[fwd] seed={k} shape={shape} causal={causal} exp={exp_mode}", flush=True)
    # poison: outputs prefilled with NaN, so an element no workgroup writes shows
    o = torch.full_like(q, float("nan")) if poison else None
    lse = torch.full(shape[:3], float("nan"), device=q.device) if poison else None
    o, lse = fa.fwd(q, kk, v, causal=causal, scale=scale, exp_mode=exp_mode, out=o, lse=lse)
    torch.cuda.synchronize()
    return inp, o, lse, scale


SMALL = [
    (1, (1, 2, 256, 64), False),     # the d=64 correctness workload
    (11, (1, 1, 1, 64), False),
    (12, (1, 1, 1, 128), True),
    (13, (1, 2, 7, 128), True),
    (14, (2, 3, 200, 128), False),
    (15, (2, 3, 200, 128), True),
    (16, (1, 2, 300, 64), True),
    (17, (1, 1, 513, 128), False),
    (18, (1, 2, 1024, 128), True),
    (19, (2, 1, 129, 64), False),
    (20, (1, 1, 4100, 128), False),  # 256-query workgroups (non-causal, d=128, N >= 4096), ragged
]


@pytest.mark.parametrize("exp_mode", ["hw", "poly", "split"])
@pytest.mark.parametrize("k,shape,causal", SMALL)
def test_fwd_matches_oracle(k, shape, causal, exp_mode):
    inp, o, lse, scale = _run(k, shape, causal, exp_mode)
    ref_o, ref_lse = attention_forward(inp["q"][0], inp["k"][0], inp["v"][0], causal, scale)
    assert_bf16_close(to_np(o), ref_o, f"O {shape} causal={causal} {exp_mode}")
    assert_lse_close(to_np(lse), ref_lse, f"LSE {shape}")


@pytest.mark.parametrize("wk", [2, 3])
def test_fwd_full_size_sampled(wk):
    w = WORKLOADS[wk]
    shape = (w["B"], w["H"], w["N"], w["d"])
    for exp_mode in (["hw", "poly", "split"] if wk == 3 else ["auto"]):
        inp, o, lse, scale = _run(wk, shape, w["causal"], exp_mode, poison=True)
        # Every output element written (the whole grid of the bench's launch).
        assert not torch.isnan(o).any().item(), f"O: elements left unwritten ({exp_mode})"
        assert not torch.isnan(lse).any().item(), f"LSE: rows left unwritten ({exp_mode})"
        o_np = o.view(-1, w["N"], w["d"])
        lse_np = lse.view(-1, w["N"])
        rng = np.random.default_rng(wk)
        N = w["N"]
        rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, N - 129, N - 1],
                                         rng.integers(0, N, 56)]))
        for (b, h) in [(0, 0), (w["B"] - 1, w["H"] - 1), (w["B"] // 2, 3)]:
            ref_o, ref_lse = attention_forward_rows(inp["q"][0], inp["k"][0], inp["v"][0],
                                                    w["causal"], scale, b, h, rows)
            bh = b * w["H"] + h
            got_o = to_np(o_np[bh][torch.as_tensor(rows, device=o.device)])
            got_l = to_np(lse_np[bh][torch.as_tensor(rows, device=o.device)])
            assert_bf16_close(got_o, ref_o, f"O rows {w['name']} b={b} h={h} {exp_mode}")
            assert_lse_close(got_l, ref_lse, f"LSE rows {w['name']} b={b} h={h}")


def test_fwd_identical_keys_and_causal_row0():
    # Closed forms re-applied to GPU outputs: identical keys give O_i = mean of the
    # visible V rows; under the causal mask row 0 equals V[0].
    import tiled_attention_fattn_amd as fa
    from tiled_attention_fattn_amd.inputs import bf16_round
    B, H, N, d = 1, 2, 300, 128
    inp = gen_workload(21, shape=(B, H, N, d))
    kv = np.broadcast_to(inp["k"][0][:, :, :1], (B, H, N, d)).copy()
    kbits = bf16_round(kv)[1]
    q = to_device_bf16(inp["q"][1])
    k = to_device_bf16(kbits)
    v = to_device_bf16(inp["v"][1])
    vv = inp["v"][0]
    for causal in (False, True):
        o, _ = fa.fwd(q, k, v, causal=causal)
        o = to_np(o)
        cnt = np.arange(1, N + 1)[:, None] if causal else N
        mean = (np.cumsum(vv, axis=2) / cnt) if causal else np.broadcast_to(vv.mean(axis=2, keepdims=True), vv.shape)
        assert_bf16_close(o, mean, f"identical keys causal={causal}")
        if causal:
            np.testing.assert_array_equal(o[:, :, 0], vv[:, :, 0])


def test_fwd_bitwise_reproducible_and_writes_everything():
    import tiled_attention_fattn_amd as fa
    shape = (2, 3, 333, 128)
    inp = gen_workload(22, shape=shape)
    q, k, v = (to_device_bf16(inp[n][1]) for n in ("q", "k", "v"))
    o1 = torch.full_like(q, float("nan"))
    l1 = torch.full(shape[:3], float("nan"), device=q.device)
    fa.fwd(q, k, v, causal=True, out=o1, lse=l1)
    o2, l2 = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert not torch.isnan(o1).any() and not torch.isnan(l1).any()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fwd_exp_modes_agree():
    import tiled_attention_fattn_amd as fa
    inp = gen_workload(23, shape=(1, 4, 512, 128))
    q, k, v = (to_device_bf16(inp[n][1]) for n in ("q", "k", "v"))
    o_hw, l_hw = fa.fwd(q, k, v, exp_mode="hw")
    o_p, l_p = fa.fwd(q, k, v, exp_mode="poly")
    o_s, l_s = fa.fwd(q, k, v, exp_mode="split")
    o_a, l_a = fa.fwd(q, k, v, exp_mode="auto")
    assert torch.equal(o_a, o_hw)
    for other in (o_p, o_s):
        diff = (o_hw.float() - other.float()).abs().max().item()
        assert diff < 1e-2, diff


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_offset_moves(causal):
    # Inputs whose scores keep rising along the keys, so the exponent offset
    # has to move inside the loop: head 0 has key rows whose norm grows 16x
    # over the sequence; in head 1 every third query row is 3.0 and key 100
    # (an inner tile) and key 690 (the last, ragged tile) are 3.0 and 3.5, so
    # those queries meet score jumps far past 2^τ, the first one large
    # enough (≈147 in log2 units) that 2^(s − m) overflows fp32 before the
    # offset moves.
    import tiled_attention_fattn_amd as fa
    from tiled_attention_fattn_amd.inputs import bf16_round
    B, H, N, d = 1, 2, 700, 128
    inp = gen_workload(24, shape=(B, H, N, d))
    q = inp["q"][0].copy()
    k = inp["k"][0].copy()
    k[:, 0] *= np.linspace(0.25, 4.0, N)[None, :, None]
    q[:, 1, ::3] = 3.0
    k[:, 1, 100] = 3.0
    k[:, 1, 690] = 3.5
    qv, qb = bf16_round(q)
    kv, kb = bf16_round(k)
    scale = d ** -0.5
    print(f"[fwd] offset moves causal={causal}", flush=True)
    o, lse = fa.fwd(to_device_bf16(qb), to_device_bf16(kb), to_device_bf16(inp["v"][1]),
                    causal=causal, scale=scale)
    torch.cuda.synchronize()
    ref_o, ref_lse = attention_forward(qv, kv, inp["v"][0], causal, scale)
    assert_bf16_close(to_np(o), ref_o, f"O offset moves causal={causal}")
    assert_lse_close(to_np(lse), ref_lse, f"LSE offset moves causal={causal}")
