"""GPU parity of the fp8 forward (libfattn fattn_fwd_fp8).

The output is compared with the float64 attention on the unrotated bf16
inputs (the rotation cannot change the exact result): relative RMS ≤ 6e-2
with the rotation (the configuration the bound is stated for); without it
the error is reported and only held to a loose sanity bound. The
quantisation is checked separately against the oracle's E4M3 model: the K'
codes in the workspace must equal the model's codes except for rare
one-step differences where the float32 rotation and the float64 one round on
opposite sides of a tie, the V codes (a power-of-two scaling) exactly, and
the per-chunk scales the model's. Q' is quantised (one scale per row, two terms)
inside the attention kernel and never stored; the LSE, compared with the
model's LSE, checks its scores (it isolates the kernel's own error from the
quantisation error), and scaling one query row by a power of two must leave
every other row's output bit for bit unchanged.
"""
import json
import os

import numpy as np
import pytest

from oracle.attention import attention_forward
from oracle.e4m3 import e4m3_decode
from oracle.fp8_model import fp8_attention_model
from tests.parity import FP8_REL_RMS, max_abs, rel_rms, to_np
from tiled_attention_fattn_amd.inputs import WORKLOADS, gen_workload, to_device_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _inputs(k, shape, outliers=True):
    w = WORKLOADS[5]
    kw = dict(outlier_frac=w["outlier_frac"], outlier_factor=w["outlier_factor"]) if outliers else {}
    return gen_workload(k, shape=shape, **kw)


def _run(inp, causal, rotate, seed):
    import tiled_attention_fattn_amd as fa
    q, k, v = (to_device_bf16(inp[n][1]) for n in ("q", "k", "v"))
    B, H, N, d = q.shape
    ws = torch.empty(fa.fp8_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=q.device)
    print(f"[fp8] shape={tuple(q.shape)} causal={causal} rotate={rotate} seed={seed}", flush=True)
    o, lse = fa.fwd_fp8(q, k, v, causal=causal, rotate=rotate, seed=seed, workspace=ws)
    torch.cuda.synchronize()
    return o, lse, ws


def _unpermute_v8t(v8t, N):
    """[B,H,d,Npad] codes in kernel key order → [B,H,N,d] codes (N=None: all Npad)."""
    B, H, d, npad = v8t.shape
    pos = np.arange(64)
    a, s = pos // 32, pos % 32
    key_of_pos = 32 * (s // 16) + 8 * ((s % 16) // 4) + 4 * a + s % 4
    out = np.empty((B, H, npad, d), dtype=v8t.dtype)
    for blk in range(npad // 64):
        out[:, :, blk * 64 + key_of_pos, :] = np.swapaxes(v8t[:, :, :, blk * 64:(blk + 1) * 64], 2, 3)
    return out if N is None else out[:, :, :N]


def _code_steps(a, b):
    """Distance in representable steps between two e4m3 code arrays."""
    va, vb = e4m3_decode(a), e4m3_decode(b)
    mag = np.sort(np.unique(np.abs(e4m3_decode(np.arange(0x7F)))))
    ia = np.searchsorted(mag, np.abs(va)) * np.sign(va)
    ib = np.searchsorted(mag, np.abs(vb)) * np.sign(vb)
    return np.abs(ia - ib)


CASES = [
    ((1, 2, 256, 128), False),
    ((1, 2, 200, 128), True),
    ((2, 2, 129, 64), False),
    ((1, 1, 1, 128), False),
    ((1, 3, 300, 64), True),
    ((1, 2, 1000, 128), False),
    ((1, 1, 4100, 128), False),  # many key tiles, ragged
    ((1, 2, 2085, 128), True),   # causal over many tiles, ragged
]


@pytest.mark.parametrize("rotate", [True, False])
@pytest.mark.parametrize("shape,causal", CASES)
def test_fp8_matches_exact_attention(shape, causal, rotate):
    import tiled_attention_fattn_amd as fa
    inp = _inputs(50 + shape[2], shape)
    o, lse, ws = _run(inp, causal, rotate, seed=5)
    scale = shape[-1] ** -0.5
    ref_o, ref_lse = attention_forward(inp["q"][0], inp["k"][0], inp["v"][0], causal, scale)
    got = to_np(o)
    assert np.all(np.isfinite(got))
    rr = rel_rms(got, ref_o)
    print(f"[fp8] rel-RMS {rr:.4e}", flush=True)
    assert rr <= (FP8_REL_RMS if rotate else 0.15), f"fp8 O rel-RMS {rr:.3e} (rotate={rotate})"

    # quantisation step against the E4M3 model
    model = fp8_attention_model(inp["q"][0], inp["k"][0], inp["v"][0], causal, scale,
                                rotate=rotate, seed=5)
    # The fp8 MFMA's sums agree with float64 sums of the same products to about
    # 1e-4 relative, so the LSE tolerance scales with |LSE|.
    lse_err = np.abs(to_np(lse) - model["lse"])
    assert np.all(lse_err <= 2e-3 + 1e-3 * np.abs(model["lse"])), lse_err.max()
    B, H, N, d = shape
    k8, v8t, sc = (t.cpu().numpy() for t in fa.fp8_workspace_views(ws, B, H, N, d))
    v8 = _unpermute_v8t(v8t, N)
    steps = _code_steps(k8, model["k8"])
    assert steps.max() <= 1, f"K8: codes differ by {steps.max()} steps"
    assert np.mean(steps == 0) >= 0.999, f"K8: {np.mean(steps != 0):.2e} codes differ"
    # V is not rotated and its scale is a power of two: every code has the
    # model's value (a negative value that rounds to zero may come out as
    # the code of −0, which decodes equal to +0)
    assert np.array_equal(e4m3_decode(v8), e4m3_decode(model["v8"])), "V8 differs from the model"
    # one (K', V) scale pair per chunk of 128 keys; the model holds the
    # scale of every row
    np.testing.assert_allclose(sc[..., 0], model["sk"][..., ::128], rtol=1e-5)
    np.testing.assert_array_equal(sc[..., 1], model["sv"][..., ::128])
    # padding keys of V8ᵀ are zero
    if v8t.shape[-1] > N:
        assert np.all(_unpermute_v8t(v8t, None)[:, :, N:] == 0)


def test_fp8_whole_tensor_error_and_rotation_ratio():
    # The fp8 workload at full size (B=4 H=16 N=4096 d=128, outliers), relative
    # RMS over the whole O tensor (all 64 heads) against the float64 exact
    # attention on the unrotated bf16 inputs, with and without the rotation.
    # Outputs are prefilled with NaN: every element must be written.
    import tiled_attention_fattn_amd as fa
    w = WORKLOADS[5]
    shape = (w["B"], w["H"], w["N"], w["d"])
    inp = _inputs(5, shape)
    scale = w["d"] ** -0.5
    q, k, v = (to_device_bf16(inp[n][1]) for n in ("q", "k", "v"))
    B, H, N, d = shape
    ws = torch.empty(fa.fp8_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=q.device)
    got = {}
    for rotate in (True, False):
        print(f"[fp8] whole tensor {w['name']} rotate={rotate}", flush=True)
        o = torch.full_like(q, float("nan"))
        fa.fwd_fp8(q, k, v, scale=scale, rotate=rotate, seed=5, want_lse=False, workspace=ws,
                   out=o)
        torch.cuda.synchronize()
        assert not torch.isnan(o).any().item(), f"rotate={rotate}: elements left unwritten"
        got[rotate] = to_np(o)
    ref, _ = attention_forward(inp["q"][0], inp["k"][0], inp["v"][0], False, scale)
    err = {rot: rel_rms(g, ref) for rot, g in got.items()}
    ratio = err[False] / err[True]
    print(f"[fp8] whole tensor rel-RMS with rotation {err[True]:.4e}, without "
          f"{err[False]:.4e}, ratio {ratio:.3f}", flush=True)
    out = os.environ.get("FATTN_REPORT_DIR")
    if out:
        with open(os.path.join(out, "fp8_rotation_error.json"), "w") as fh:
            json.dump({"rel_rms_rotate": err[True], "rel_rms_no_rotate": err[False],
                       "ratio": ratio, "workload": w["name"], "scope": "whole O tensor"}, fh)
    assert err[True] <= FP8_REL_RMS, f"rotate=True: rel-RMS {err[True]:.3e}"
    assert err[False] <= 0.2, f"rotate=False: rel-RMS {err[False]:.3e}"


@pytest.mark.parametrize("rotate", [True, False])
def test_fp8_query_rows_are_quantised_independently(rotate):
    # One scale per query row: multiplying row r of Q by 2^3 leaves every
    # other row's O and LSE bit for bit unchanged (a per-head scale would
    # move them all), and row r's codes too (only its scale changes).
    import tiled_attention_fattn_amd as fa
    shape = (1, 2, 300, 128)
    inp = _inputs(62, shape)
    q, k, v = (to_device_bf16(inp[n][1]) for n in ("q", "k", "v"))
    B, H, N, d = shape
    ws = torch.empty(fa.fp8_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=q.device)
    print(f"[fp8] per-row Q scale, shape={shape} rotate={rotate}", flush=True)
    o1, l1 = fa.fwd_fp8(q, k, v, rotate=rotate, seed=4, workspace=ws)
    q2 = q.clone()
    q2[0, 1, 77] *= 8.0
    o2, l2 = fa.fwd_fp8(q2, k, v, rotate=rotate, seed=4, workspace=ws)
    torch.cuda.synchronize()
    keep = torch.ones(N, dtype=torch.bool, device=q.device)
    keep[77] = False
    assert torch.equal(o1[0, 0], o2[0, 0]) and torch.equal(l1[0, 0], l2[0, 0])
    assert torch.equal(o1[0, 1][keep], o2[0, 1][keep])
    assert torch.equal(l1[0, 1][keep], l2[0, 1][keep])
    assert not torch.equal(o1[0, 1, 77], o2[0, 1, 77])


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_attend_reuses_workspace(causal):
    # The attention step alone on the operands a full call left in the
    # workspace reproduces that call's O and LSE bit for bit.
    import tiled_attention_fattn_amd as fa
    shape = (2, 3, 300, 128)
    inp = _inputs(61, shape)
    q, k, v = (to_device_bf16(inp[n][1]) for n in ("q", "k", "v"))
    B, H, N, d = shape
    ws = torch.empty(fa.fp8_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=q.device)
    print(f"[fp8] attend on workspace shape={shape} causal={causal}", flush=True)
    o1, l1 = fa.fwd_fp8(q, k, v, causal=causal, rotate=True, seed=3, workspace=ws)
    o2, l2 = fa.fwd_fp8_attend(q, ws, causal=causal, rotate=True, seed=3)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("exp_mode", ["poly", "split"])
@pytest.mark.parametrize("shape,causal", [((1, 2, 256, 128), False), ((1, 3, 300, 64), True),
                                          ((1, 2, 1000, 128), False)])
def test_fp8_exp_modes(shape, causal, exp_mode):
    # The polynomial exp2 (all elements, or one in four) feeds P̃ to the same
    # e4m3 rounding; the output stays within the fp8 bound of exact attention,
    # within 2e-2 (relative RMS) of the hardware-exp2 output, and the LSE
    # within the model's tolerance.
    import tiled_attention_fattn_amd as fa
    inp = _inputs(70 + shape[2], shape)
    q, k, v = (to_device_bf16(inp[n][1]) for n in ("q", "k", "v"))
    B, H, N, d = shape
    scale = d ** -0.5
    ws = torch.empty(fa.fp8_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=q.device)
    print(f"[fp8] exp={exp_mode} shape={shape} causal={causal}", flush=True)
    o_hw, _ = fa.fwd_fp8(q, k, v, causal=causal, rotate=True, seed=5, workspace=ws,
                         exp_mode="hw")
    o_x, l_x = fa.fwd_fp8(q, k, v, causal=causal, rotate=True, seed=5, workspace=ws,
                          exp_mode=exp_mode)
    o_a, l_a = fa.fwd_fp8_attend(q, ws, causal=causal, scale=scale, rotate=True, seed=5,
                                 exp_mode=exp_mode)
    torch.cuda.synchronize()
    assert torch.equal(o_x, o_a) and torch.equal(l_x, l_a)
    ref_o, _ = attention_forward(inp["q"][0], inp["k"][0], inp["v"][0], causal, scale)
    got = to_np(o_x)
    assert np.all(np.isfinite(got))
    assert rel_rms(got, ref_o) <= FP8_REL_RMS
    assert rel_rms(got, to_np(o_hw)) <= 2e-2
    model = fp8_attention_model(inp["q"][0], inp["k"][0], inp["v"][0], causal, scale,
                                rotate=True, seed=5)
    lse_err = np.abs(to_np(l_x) - model["lse"])
    assert np.all(lse_err <= 2e-3 + 1e-3 * np.abs(model["lse"])), lse_err.max()


@pytest.mark.parametrize("shape,causal", [((1, 2, 300, 128), False), ((1, 3, 500, 64), True),
                                          ((2, 2, 4100, 128), False)])
def test_fp8_output_does_not_depend_on_the_lse_request(shape, causal):
    # The kernel without the LSE output (the one the bench times) and the one
    # with it form O by the same arithmetic: bit for bit the same O.
    import tiled_attention_fattn_amd as fa
    inp = _inputs(90 + shape[2], shape)
    q, k, v = (to_device_bf16(inp[n][1]) for n in ("q", "k", "v"))
    B, H, N, d = shape
    ws = torch.empty(fa.fp8_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=q.device)
    print(f"[fp8] lse / no lse shape={shape} causal={causal}", flush=True)
    o1, l1 = fa.fwd_fp8(q, k, v, causal=causal, rotate=True, seed=8, workspace=ws)
    o2, l2 = fa.fwd_fp8(q, k, v, causal=causal, rotate=True, seed=8, workspace=ws,
                        want_lse=False)
    torch.cuda.synchronize()
    assert l2 is None
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("d,causal", [(128, False), (128, True), (64, False)])
def test_fp8_row_max_growing_past_the_exponent_cap(d, causal):
    # Every 128 keys the row max rises by 3.8 to 6.4 log2 units (key rows
    # t·e₀ with t growing chunk by chunk, query rows with 3 ≤ q₀ ≤ 5), 57 to
    # 96 units over the row: the P operand's block-scale exponent grows and
    # passes its cap of 32 once or twice per row, at different tiles for
    # different rows of a wave, which moves the offset and rescales O. The
    # keys of a 128-key chunk are identical (their e4m3 codes exact: every
    # rotated element has the chunk's amax), so the fp8 softmax weights are
    # nearly exact: O against exact attention within the fp8 bound, the LSE
    # within the dense tests' tolerance of the model.
    import tiled_attention_fattn_amd as fa
    from tiled_attention_fattn_amd.inputs import bf16_round
    N = 2000
    rng = np.random.default_rng(95 + d)
    q = rng.standard_normal((1, 2, N, d))
    q[..., 0] = 3.0 + 0.5 * rng.integers(0, 5, size=(1, 2, N))
    k = np.zeros((1, 2, N, d))
    step = 10.0 if d == 128 else 7.0
    k[..., 0] = step * (np.arange(N) // 128)
    v = rng.standard_normal((1, 2, N, d))
    (qf, qb), (kf, kb), (vf, vb) = bf16_round(q), bf16_round(k), bf16_round(v)
    scale = d ** -0.5
    print(f"[fp8] growing row max d={d} causal={causal}", flush=True)
    o, lse = fa.fwd_fp8(to_device_bf16(qb), to_device_bf16(kb), to_device_bf16(vb),
                        causal=causal, scale=scale, rotate=True, seed=2)
    torch.cuda.synchronize()
    ref_o, _ = attention_forward(qf, kf, vf, causal, scale)
    got = to_np(o)
    assert np.all(np.isfinite(got))
    rr = rel_rms(got, ref_o)
    print(f"[fp8] growing row max rel-RMS {rr:.3e}", flush=True)
    assert rr <= FP8_REL_RMS
    model = fp8_attention_model(qf, kf, vf, causal, scale, rotate=True, seed=2)
    lse_err = np.abs(to_np(lse) - model["lse"])
    assert np.all(lse_err <= 2e-3 + 1e-3 * np.abs(model["lse"])), lse_err.max()


def test_fp8_tiny_value_chunks():
    # Chunks of 128 keys whose V (and K) values lie far below the usual range
    # (|v| ≤ 2^-120, so 448·2^e would need e < −126): V keeps the scale
    # 2^-126 and its codes (many of them bf16 subnormals), K its exact
    # ratio; every code and scale as the model's, nothing overflows, and O
    # stays within the fp8 bound of exact attention (the tiny K chunk's keys
    # score about 0 and take a visible share of every row's weight).
    import tiled_attention_fattn_amd as fa
    from tiled_attention_fattn_amd.inputs import bf16_round
    B, H, N, d = 1, 2, 512, 128
    rng = np.random.default_rng(97)
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    v[:, :, 128:256] *= 2.0 ** -122           # a whole chunk of tiny V
    k[:, :, 256:384] *= 2.0 ** -122           # a whole chunk of tiny K
    (qf, qb), (kf, kb), (vf, vb) = bf16_round(q), bf16_round(k), bf16_round(v)
    scale = d ** -0.5
    ws = torch.zeros(fa.fp8_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    print("[fp8] tiny-value chunks", flush=True)
    o, lse = fa.fwd_fp8(to_device_bf16(qb), to_device_bf16(kb), to_device_bf16(vb),
                        scale=scale, rotate=True, seed=7, workspace=ws)
    torch.cuda.synchronize()
    model = fp8_attention_model(qf, kf, vf, False, scale, rotate=True, seed=7)
    k8, v8t, sc = (t.cpu().numpy() for t in fa.fp8_workspace_views(ws, B, H, N, d))
    assert np.all(sc[:, :, 1, 1] == 2.0 ** -126)
    np.testing.assert_array_equal(sc[..., 1], model["sv"][..., ::128])
    np.testing.assert_allclose(sc[..., 0], model["sk"][..., ::128], rtol=1e-5)
    v8 = _unpermute_v8t(v8t, N)
    assert np.array_equal(e4m3_decode(v8), e4m3_decode(model["v8"]))
    steps = _code_steps(k8, model["k8"])
    assert steps.max() <= 1 and np.mean(steps == 0) >= 0.999
    ref_o, _ = attention_forward(qf, kf, vf, False, scale)
    got = to_np(o)
    assert np.all(np.isfinite(got))
    assert rel_rms(got, ref_o) <= FP8_REL_RMS
    lse_err = np.abs(to_np(lse) - model["lse"])
    assert np.all(lse_err <= 2e-3 + 1e-3 * np.abs(model["lse"])), lse_err.max()


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_bitwise_reproducible(causal):
    # No atomics and a fixed reduction order: two calls on the same inputs
    # give the same O, LSE and workspace bit for bit (dense, and packed
    # segments with a length mix).
    import tiled_attention_fattn_amd as fa
    shape = (2, 4, 1100, 128)
    inp = _inputs(40, shape)
    q, k, v = (to_device_bf16(inp[n][1]) for n in ("q", "k", "v"))
    B, H, N, d = shape
    print(f"[fp8] reproducibility causal={causal}", flush=True)
    ws1 = torch.zeros(fa.fp8_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    ws2 = torch.ones_like(ws1)
    o1, l1 = fa.fwd_fp8(q, k, v, causal=causal, rotate=True, seed=9, workspace=ws1)
    o2, l2 = fa.fwd_fp8(q, k, v, causal=causal, rotate=True, seed=9, workspace=ws2)
    cu = torch.tensor([0, 1, 300, 301, 777, 1100], dtype=torch.int32, device="cuda")
    v1, m1 = fa.fwd_fp8_varlen(q, k, v, cu, 476, causal=causal, rotate=True, seed=9)
    v2, m2 = fa.fwd_fp8_varlen(q, k, v, cu, 476, causal=causal, rotate=True, seed=9)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    k8a, v8a, sa = fa.fp8_workspace_views(ws1, B, H, N, d)
    k8b, v8b, sb = fa.fp8_workspace_views(ws2, B, H, N, d)
    assert torch.equal(k8a, k8b) and torch.equal(v8a, v8b) and torch.equal(sa, sb)
    assert torch.equal(v1, v2) and torch.equal(m1, m2)


def test_fp8_subnormal_blocks():
    # A K chunk and some Q rows whose rotated values all lie below 2^-128
    # (bf16 subnormals), where 1/amax overflows in fp32: the quantiser
    # rescales such blocks exactly, so the K codes and scales are the
    # model's, every output is finite and within the fp8 bound of exact
    # attention, and the LSE matches the model's.
    import tiled_attention_fattn_amd as fa
    from tiled_attention_fattn_amd.inputs import bf16_round
    B, H, N, d = 1, 2, 384, 128
    rng = np.random.default_rng(98)
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    k[:, :, 128:256] *= 2.0 ** -131
    q[:, :, 5:40] *= 2.0 ** -131
    (qf, qb), (kf, kb), (vf, vb) = bf16_round(q), bf16_round(k), bf16_round(v)
    assert np.abs(kf[:, :, 128:256]).max() < 2.0 ** -128
    scale = d ** -0.5
    ws = torch.zeros(fa.fp8_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    print("[fp8] subnormal blocks", flush=True)
    o, lse = fa.fwd_fp8(to_device_bf16(qb), to_device_bf16(kb), to_device_bf16(vb),
                        scale=scale, rotate=True, seed=7, workspace=ws)
    torch.cuda.synchronize()
    model = fp8_attention_model(qf, kf, vf, False, scale, rotate=True, seed=7)
    k8, _, sc = (t.cpu().numpy() for t in fa.fp8_workspace_views(ws, B, H, N, d))
    # the tiny chunk's scale (about 3e-42) is an fp32 subnormal: two steps of
    # 2^-149 on top of the relative tolerance
    np.testing.assert_allclose(sc[..., 0], model["sk"][..., ::128], rtol=1e-5, atol=2.0 ** -148)
    steps = _code_steps(k8, model["k8"])
    assert steps.max() <= 1 and np.mean(steps == 0) >= 0.999
    got = to_np(o)
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(to_np(lse)))
    ref_o, _ = attention_forward(qf, kf, vf, False, scale)
    assert rel_rms(got, ref_o) <= FP8_REL_RMS
    lse_err = np.abs(to_np(lse) - model["lse"])
    assert np.all(lse_err <= 2e-3 + 1e-3 * np.abs(model["lse"])), lse_err.max()


def test_fp8_causal_issue_groups_ragged():
    # Causal d = 128 with 4 to 8 query tiles per head runs in issue groups of
    # whole heads (as many as fill the resident workgroups once); 100 heads
    # of 640 rows (5 tiles) make groups of 96 and 4 heads. Every output
    # element must be written (NaN-poisoned), O within the fp8 bound of exact
    # attention and the LSE within the model's tolerance on every head.
    import tiled_attention_fattn_amd as fa
    shape = (4, 25, 640, 128)
    inp = _inputs(640, shape)
    q, k, v = (to_device_bf16(inp[n][1]) for n in ("q", "k", "v"))
    scale = shape[-1] ** -0.5
    o = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    print(f"[fp8] causal issue groups shape={shape}", flush=True)
    o, lse = fa.fwd_fp8(q, k, v, causal=True, scale=scale, rotate=True, seed=6, out=o)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any().item(), "elements left unwritten"
    ref_o, _ = attention_forward(inp["q"][0], inp["k"][0], inp["v"][0], True, scale)
    rr = rel_rms(to_np(o), ref_o)
    print(f"[fp8] causal issue groups rel-RMS {rr:.4e}", flush=True)
    assert rr <= FP8_REL_RMS
    model = fp8_attention_model(inp["q"][0], inp["k"][0], inp["v"][0], True, scale,
                                rotate=True, seed=6)
    # As in the packed-sequence tests: a row dominated by few scores (an
    # early causal row, or one with an outlier-sized score) moves its LSE by
    # the change of one score when one K' code is a step off the model's
    # (float32 against float64 rotation, opposite sides of a tie); across
    # 100 heads such rows occur (seen: one of 64000, 0.048). The strict bound
    # on 99% of the rows, a loose one on all.
    lse_err = np.abs(to_np(lse) - model["lse"])
    strict = lse_err <= 2e-3 + 1e-3 * np.abs(model["lse"])
    assert np.mean(strict) >= 0.99, (np.mean(strict), lse_err.max())
    assert np.all(lse_err <= 5e-2 + 1e-2 * np.abs(model["lse"])), lse_err.max()
    print(f"[fp8] causal issue groups: {np.sum(~strict)} rows outside the strict LSE bound, "
          f"rows {np.unique(np.nonzero(~strict)[2])[:10]}", flush=True)
