"""GPU parity of the block-sparse forward and backward (fattn_fwd_blocksparse,
fattn_bwd_blocksparse) against the float64 oracle with the same block mask
(blocks of 128 queries x 128 keys).

Masks are seeded random 0/1 patterns (shared by all heads or one per head)
with some block rows left empty, on shapes with ragged tails, both head
dimensions, causal and not, hardware and split exp2; rows that see no key
must come out as O = 0 and LSE = -inf, and the gradients as the oracle's
(zero for rows and key blocks that see nothing). An all-ones mask must
reproduce the dense forward and backward bit for bit. At full size (B=2, H=16, N=8192, d=128, a local
band plus random blocks) the output is checked on sampled rows.
"""
import numpy as np
import pytest

from oracle.attention import attention_backward, attention_forward, attention_forward_rows
from tests.parity import assert_bf16_close, assert_lse_close, to_np
from tiled_attention_fattn_amd.inputs import gen_workload, to_device_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = [
    # (seed, B, H, N, d, causal, per_head)
    (100, 1, 2, 300, 128, False, False),
    (101, 1, 2, 513, 128, True, False),
    (102, 2, 1, 640, 64, False, True),
    (103, 1, 3, 1000, 64, True, True),
    (104, 1, 1, 129, 128, False, False),
]


def _mask(seed, heads, nb, density=0.5):
    rng = np.random.default_rng(seed)
    m = (rng.random((heads, nb, nb)) < density).astype(np.uint8)
    m[:, nb // 2, :] = 0  # an empty block row in every head
    m[:, 0, 0] = 1        # and the first block row never empty
    return m


def _compare(o, lse, ref_o, ref_lse, what):
    got_o, got_l = to_np(o), to_np(lse)
    empty = np.isneginf(ref_lse)
    assert np.all(got_o[empty] == 0), f"{what}: rows with no visible key are not zero"
    assert np.all(np.isneginf(got_l[empty])), f"{what}: LSE of empty rows is not -inf"
    keep = ~empty
    assert_bf16_close(got_o[keep], ref_o[keep], what)
    assert_lse_close(got_l[keep], ref_lse[keep], what)


@pytest.mark.parametrize("exp_mode", ["hw", "split"])
@pytest.mark.parametrize("seed,B,H,N,d,causal,per_head", CASES)
def test_blocksparse_matches_oracle(seed, B, H, N, d, causal, per_head, exp_mode):
    import tiled_attention_fattn_amd as fa
    inp = gen_workload(seed, shape=(B, H, N, d))
    q, k, v = (to_device_bf16(inp[n][1]) for n in ("q", "k", "v"))
    nb = (N + 127) // 128
    m = _mask(seed, B * H if per_head else 1, nb)
    mask = m if per_head else m[0]
    scale = d ** -0.5
    print(f"[sparse] seed={seed} shape={(B, H, N, d)} causal={causal} per_head={per_head} "
          f"exp={exp_mode}", flush=True)
    o, lse = fa.fwd_blocksparse(q, k, v, torch.as_tensor(mask, device="cuda"), causal=causal,
                                scale=scale, exp_mode=exp_mode)
    torch.cuda.synchronize()
    ref_o, ref_lse = attention_forward(inp["q"][0], inp["k"][0], inp["v"][0], causal, scale,
                                       block_mask=mask)
    _compare(o, lse, ref_o, ref_lse, f"sparse {(B, H, N, d)} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_blocksparse_all_ones_equals_dense(causal):
    import tiled_attention_fattn_amd as fa
    inp = gen_workload(105, shape=(1, 2, 700, 128))
    q, k, v = (to_device_bf16(inp[n][1]) for n in ("q", "k", "v"))
    ones = torch.ones((6, 6), dtype=torch.uint8, device="cuda")
    o1, l1 = fa.fwd_blocksparse(q, k, v, ones, causal=causal)
    o2, l2 = fa.fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def _band_mask(nb, seed):
    rng = np.random.default_rng(seed)
    m = (rng.random((nb, nb)) < 0.25).astype(np.uint8)
    for i in range(nb):
        m[i, max(0, i - 2):i + 1] = 1  # local band of three blocks
    return m


def test_blocksparse_full_size_sampled():
    import tiled_attention_fattn_amd as fa
    B, H, N, d = 2, 16, 8192, 128
    inp = gen_workload(106, shape=(B, H, N, d))
    q, k, v = (to_device_bf16(inp[n][1]) for n in ("q", "k", "v"))
    m = _band_mask(N // 128, 106)
    print(f"[sparse full] density {m.mean():.3f}", flush=True)
    o, lse = fa.fwd_blocksparse(q, k, v, torch.as_tensor(m, device="cuda"))
    torch.cuda.synchronize()
    rng = np.random.default_rng(107)
    rows = np.unique(np.concatenate([[0, 127, 128, 4095, N - 1], rng.integers(0, N, 40)]))
    idx = torch.as_tensor(rows, device="cuda")
    for (b, h) in [(0, 0), (1, 15)]:
        ref_o, ref_l = attention_forward_rows(inp["q"][0], inp["k"][0], inp["v"][0], False,
                                              d ** -0.5, b, h, rows, block_mask=m)
        assert_bf16_close(to_np(o[b, h][idx]), ref_o, f"O sparse full b={b} h={h}")
        assert_lse_close(to_np(lse[b, h][idx]), ref_l, f"LSE sparse full b={b} h={h}")


@pytest.mark.parametrize("seed,B,H,N,d,causal,per_head", CASES)
def test_blocksparse_backward_matches_oracle(seed, B, H, N, d, causal, per_head):
    import tiled_attention_fattn_amd as fa
    inp = gen_workload(seed + 20, shape=(B, H, N, d), names=("q", "k", "v", "do"))
    q, k, v, do = (to_device_bf16(inp[n][1]) for n in ("q", "k", "v", "do"))
    nb = (N + 127) // 128
    m = _mask(seed + 20, B * H if per_head else 1, nb)
    mask = m if per_head else m[0]
    mt = torch.as_tensor(mask, device="cuda")
    scale = d ** -0.5
    print(f"[sparse bwd] seed={seed + 20} shape={(B, H, N, d)} causal={causal} "
          f"per_head={per_head}", flush=True)
    o, lse = fa.fwd_blocksparse(q, k, v, mt, causal=causal, scale=scale)
    grads = fa.bwd_blocksparse(q, k, v, o, lse, do, mt, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ref = attention_backward(inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], causal, scale,
                             block_mask=mask)
    for name, got, r in zip(("dQ", "dK", "dV"), grads, ref[:3]):
        g = to_np(got)
        assert np.all(np.isfinite(g)), f"{name}: non-finite"
        assert_bf16_close(g, r, f"{name} sparse {(B, H, N, d)} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_blocksparse_backward_all_ones_equals_dense(causal):
    import tiled_attention_fattn_amd as fa
    inp = gen_workload(108, shape=(1, 2, 700, 128), names=("q", "k", "v", "do"))
    q, k, v, do = (to_device_bf16(inp[n][1]) for n in ("q", "k", "v", "do"))
    ones = torch.ones((6, 6), dtype=torch.uint8, device="cuda")
    o, lse = fa.fwd(q, k, v, causal=causal)
    g1 = fa.bwd_blocksparse(q, k, v, o, lse, do, ones, causal=causal)
    g2 = fa.bwd(q, k, v, o, lse, do, causal=causal)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
