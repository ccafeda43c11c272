"""GPU parity of the packed variable-length forward and backward
(fattn_fwd_varlen, fattn_bwd_varlen) against the float64 oracle with segment
offsets.

Small packings mix segment lengths of 1, a few rows, exact tile multiples and
ragged tails, both head dimensions, causal and not, up to 70 segments; they are compared element
by element with the full oracle. Each segment must also come out bit for bit
as the plain kernels compute it on that segment alone (the same tiles and the
same accumulation order). A larger packing (B=1, H=8, N=16384, lengths drawn
from a seeded mix between 1 and 4096 rows) is checked on sampled rows for the
forward and against the oracle gradients of whole segments for the backward.
"""
import numpy as np
import pytest

from oracle.attention import attention_backward, attention_forward, attention_forward_rows
from tests.parity import assert_bf16_close, assert_lse_close, to_np
from tiled_attention_fattn_amd.inputs import gen_workload, to_device_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = [
    # (seed, H, d, lengths, causal)
    (80, 2, 128, [1, 7, 64, 100, 129, 300], False),
    (81, 2, 128, [1, 7, 64, 100, 129, 300], True),
    (82, 1, 64, [200, 1, 1, 333, 128], False),
    (83, 3, 64, [5, 250, 64, 64, 17], True),
    (84, 1, 128, [513], True),
    # 64 segments (the most the forward's longest-first order ranks), 70 (more:
    # segment order kept), both with many equal lengths
    (85, 1, 64, [(i * 13) % 29 + 1 for i in range(64)], False),
    (86, 1, 128, [(i * 37) % 41 + 1 for i in range(70)], False),
    # one segment of 4100 rows: the plain forward it is compared with bit for
    # bit runs 256-query workgroups (non-causal, d=128, N >= 4096), the packed
    # one 128-query workgroups
    (87, 1, 128, [4100], False),
]


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def _setup(seed, H, d, lengths, names=("q", "k", "v")):
    cu = _cu(lengths)
    N = int(cu[-1])
    inp = gen_workload(seed, shape=(1, H, N, d), names=names)
    dev = {n: to_device_bf16(inp[n][1]) for n in names}
    cu_t = torch.as_tensor(cu, device="cuda")
    return inp, dev, cu, cu_t, N


@pytest.mark.parametrize("exp_mode", ["hw", "split"])
@pytest.mark.parametrize("seed,H,d,lengths,causal", CASES)
def test_fwd_varlen_matches_oracle(seed, H, d, lengths, causal, exp_mode):
    import tiled_attention_fattn_amd as fa
    inp, t, cu, cu_t, N = _setup(seed, H, d, lengths)
    scale = d ** -0.5
    print(f"[varlen fwd] seed={seed} lengths={lengths} d={d} causal={causal} exp={exp_mode}",
          flush=True)
    o, lse = fa.fwd_varlen(t["q"], t["k"], t["v"], cu_t, max(lengths), causal=causal,
                           scale=scale, exp_mode=exp_mode)
    torch.cuda.synchronize()
    ref_o, ref_lse = attention_forward(inp["q"][0], inp["k"][0], inp["v"][0], causal, scale,
                                       cu_seqlens=cu)
    assert_bf16_close(to_np(o), ref_o, f"O varlen {lengths} causal={causal}")
    assert_lse_close(to_np(lse), ref_lse, f"LSE varlen {lengths}")
    # every segment bit for bit as the plain forward of that segment alone
    for a, b in zip(cu[:-1], cu[1:]):
        if b == a:
            continue
        so, sl = fa.fwd(t["q"][:, :, a:b].clone(), t["k"][:, :, a:b].clone(),
                        t["v"][:, :, a:b].clone(), causal=causal, scale=scale,
                        exp_mode=exp_mode)
        assert torch.equal(o[:, :, a:b], so), f"segment [{a}, {b}) differs from fwd"
        assert torch.equal(lse[:, :, a:b], sl)


@pytest.mark.parametrize("seed,H,d,lengths,causal", CASES)
def test_bwd_varlen_matches_oracle(seed, H, d, lengths, causal):
    import tiled_attention_fattn_amd as fa
    inp, t, cu, cu_t, N = _setup(seed + 10, H, d, lengths, names=("q", "k", "v", "do"))
    scale = d ** -0.5
    print(f"[varlen bwd] seed={seed + 10} lengths={lengths} d={d} causal={causal}", flush=True)
    o, lse = fa.fwd_varlen(t["q"], t["k"], t["v"], cu_t, max(lengths), causal=causal,
                           scale=scale)
    grads = fa.bwd_varlen(t["q"], t["k"], t["v"], o, lse, t["do"], cu_t, max(lengths),
                          causal=causal, scale=scale)
    torch.cuda.synchronize()
    ref = attention_backward(inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], causal, scale,
                             cu_seqlens=cu)
    for name, got, r in zip(("dQ", "dK", "dV"), grads, ref[:3]):
        assert_bf16_close(to_np(got), r, f"{name} varlen {lengths} causal={causal}")
    for a, b in zip(cu[:-1], cu[1:]):
        if b == a:
            continue
        sl = [x[:, :, a:b].clone() for x in (t["q"], t["k"], t["v"], o, lse, t["do"])]
        seg = fa.bwd(*sl, causal=causal, scale=scale)
        for name, got, g in zip(("dQ", "dK", "dV"), grads, seg):
            assert torch.equal(got[:, :, a:b], g), f"{name} segment [{a}, {b}) differs from bwd"


@pytest.mark.parametrize("causal", [True, False])
def test_varlen_single_segment_equals_plain_and_empty_segments(causal):
    import tiled_attention_fattn_amd as fa
    inp, t, cu, cu_t, N = _setup(90, 2, 128, [300], names=("q", "k", "v", "do"))
    o1, l1 = fa.fwd(t["q"], t["k"], t["v"], causal=causal)
    # empty segments at the start, middle and end change nothing (without the
    # mask the forward ranks segments by length: the empty ones tie at 0)
    cu2 = torch.as_tensor(np.array([0, 0, 300, 300], dtype=np.int32), device="cuda")
    o2, l2 = fa.fwd_varlen(t["q"], t["k"], t["v"], cu2, 300, causal=causal)
    g1 = fa.bwd(t["q"], t["k"], t["v"], o1, l1, t["do"], causal=causal)
    g2 = fa.bwd_varlen(t["q"], t["k"], t["v"], o2, l2, t["do"], cu2, 300, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def _mix_lengths(total, seed):
    rng = np.random.default_rng(seed)
    lengths = []
    while sum(lengths) < total:
        lengths.append(int(min(rng.integers(1, 4097), total - sum(lengths))))
    return lengths


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_length_mix_large(causal):
    import tiled_attention_fattn_amd as fa
    lengths = _mix_lengths(16384, 95)
    inp, t, cu, cu_t, N = _setup(95, 8, 128, lengths, names=("q", "k", "v", "do"))
    scale = 128 ** -0.5
    print(f"[varlen mix] {len(lengths)} segments, max {max(lengths)}, causal={causal}", flush=True)
    o, lse = fa.fwd_varlen(t["q"], t["k"], t["v"], cu_t, max(lengths), causal=causal, scale=scale)
    grads = fa.bwd_varlen(t["q"], t["k"], t["v"], o, lse, t["do"], cu_t, max(lengths),
                          causal=causal, scale=scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(96)
    rows = np.unique(np.concatenate([cu[:-1], cu[1:] - 1, rng.integers(0, N, 64)]))
    idx = torch.as_tensor(rows, device="cuda")
    for h in (0, 7):
        ref_o, ref_l = attention_forward_rows(inp["q"][0], inp["k"][0], inp["v"][0], causal,
                                              scale, 0, h, rows, cu_seqlens=cu)
        assert_bf16_close(to_np(o[0, h][idx]), ref_o, f"O mix h={h}")
        assert_lse_close(to_np(lse[0, h][idx]), ref_l, f"LSE mix h={h}")
    # gradients of two whole segments (the longest and the first) of head 3
    for s in sorted({int(np.argmax(lengths)), 0}):
        a, b = int(cu[s]), int(cu[s + 1])
        sl = (slice(0, 1), slice(3, 4), slice(a, b))
        ref = attention_backward(inp["q"][0][sl], inp["k"][0][sl], inp["v"][0][sl],
                                 inp["do"][0][sl], causal, scale)
        for name, got, r in zip(("dQ", "dK", "dV"), grads, ref[:3]):
            assert_bf16_close(to_np(got[0:1, 3:4, a:b]), r, f"{name} mix segment {s}")
