"""Pins for the OCP E4M3FN model and the fp8 quantisation model (CPU only).

torch's float8_e4m3fn dtype is an independent library implementation of the
same OCP format: its decode of every code, and its round-to-nearest-even
cast for in-range values, must agree with ``oracle.e4m3``.
"""
import numpy as np
import pytest
import torch

from oracle.attention import attention_forward
from oracle.e4m3 import E4M3_MAX, e4m3_decode, e4m3_encode, e4m3_values
from oracle.fp8_model import (dequantize, dequantize_rows, fp8_attention_model, pow2_scale,
                              quantize_per_block, quantize_per_block_pow2, quantize_per_head,
                              row_blocks)


def test_decode_known_codes():
    assert e4m3_decode(0x00) == 0.0
    assert e4m3_decode(0x01) == 2.0 ** -9
    assert e4m3_decode(0x07) == 7 * 2.0 ** -9
    assert e4m3_decode(0x08) == 2.0 ** -6
    assert e4m3_decode(0x38) == 1.0
    assert e4m3_decode(0x7E) == 448.0
    assert e4m3_decode(0xFE) == -448.0
    assert np.isnan(e4m3_decode(0x7F)) and np.isnan(e4m3_decode(0xFF))
    assert E4M3_MAX == 448.0


def test_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(theirs))
    ok = ~np.isnan(ours)
    np.testing.assert_array_equal(ours[ok], theirs[ok])


def test_encode_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    back = e4m3_encode(e4m3_decode(codes))
    expect = np.where(codes == 0x80, 0, codes)       # −0 encodes as +0
    np.testing.assert_array_equal(back, expect)


def test_encode_ties_to_even_and_saturation():
    vals = e4m3_values()
    mids = (vals[:-1] + vals[1:]) / 2
    codes = e4m3_encode(mids)
    lo = np.arange(len(mids))
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    np.testing.assert_array_equal(codes, expect)
    assert e4m3_encode(1e9) == 0x7E and e4m3_encode(-1e9) == 0xFE
    assert e4m3_encode(460.0) == 0x7E
    assert e4m3_encode(2.0 ** -11) == 0x00          # below half the smallest step
    assert e4m3_encode(3 * 2.0 ** -11) == 0x01      # 0.75 step rounds up


def test_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 50,
                        rng.standard_normal(20000) * 1e-2,
                        rng.uniform(-448, 448, 20000)])
    ours = e4m3_encode(x)
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch keeps the sign of a zero result; our encoder returns +0.
    theirs = np.where(theirs == 0x80, 0, theirs)
    np.testing.assert_array_equal(ours, theirs)


def test_quantize_per_head_amax_maps_to_max_code():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 3, 16, 8))
    x[1, 2] = 0.0                                      # an all-zero head
    codes, scales = quantize_per_head(x)
    assert scales[1, 2] == 1.0 and np.all(codes[1, 2] == 0)
    for b in range(2):
        for h in range(3):
            if b == 1 and h == 2:
                continue
            j = np.argmax(np.abs(x[b, h]))
            assert codes[b, h].flat[j] in (0x7E, 0xFE)
    # relative error of the round trip stays within half a step (2^-4 relative)
    xr = dequantize(codes, scales)
    big = np.abs(x) > scales[:, :, None, None] * 2.0 ** -6
    rel = np.abs(xr - x)[big] / np.abs(x)[big]
    assert rel.max() <= 2.0 ** -4 + 1e-12


def test_fp8_model_without_rotation_is_attention_on_dequantised():
    rng = np.random.default_rng(2)
    q, k, v = (rng.standard_normal((1, 2, 24, 16)) for _ in range(3))
    m = fp8_attention_model(q, k, v, False, 0.25, rotate=False, seed=0)
    from oracle.fp8_model import dequantize_split_rows
    o, _ = attention_forward(dequantize_split_rows(m["q8"], m["q8lo"], m["sq"]),
                             dequantize_rows(m["k8"], m["sk"]), dequantize_rows(m["v8"], m["sv"]),
                             False, 0.25)
    np.testing.assert_array_equal(m["o"], o)
    np.testing.assert_array_equal(m["q_rot"], q)
    exact, _ = attention_forward(q, k, v, False, 0.25)
    rel = np.linalg.norm(m["o"] - exact) / np.linalg.norm(exact)
    assert 1e-4 < rel < 6e-2


def test_fp8_model_with_rotation_quantises_rotated_operands():
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((1, 1, 8, 16)) for _ in range(3))
    m = fp8_attention_model(q, k, v, False, 0.25, rotate=True, seed=9)
    from oracle.hadamard import rotate
    np.testing.assert_allclose(m["q_rot"], rotate(q, 9), atol=0)
    # Eight keys are one scale block: K' as with one scale per head.
    codes, scales = quantize_per_head(rotate(k, 9))
    np.testing.assert_array_equal(m["k8"], codes)
    np.testing.assert_array_equal(m["sk"], np.broadcast_to(scales[:, :, None], (1, 1, 8)))


def test_quantisation_uses_the_exact_ratio_at_ties():
    # bf16 inputs make exact e4m3 midpoints common: with amax = 3.0625,
    # x = 1.4765625 gives x·448/amax = 216 exactly, the midpoint of 208 (odd
    # code 0x75) and 224 (even code 0x76): round-to-nearest-even picks 0x76.
    x = np.zeros((1, 1, 2, 1))
    x[0, 0, 0, 0] = 3.0625
    x[0, 0, 1, 0] = 1.4765625
    codes, scales = quantize_per_head(x)
    assert codes[0, 0, 0, 0] == 0x7E and codes[0, 0, 1, 0] == 0x76
    assert scales[0, 0] == 3.0625 / 448


def test_split_quantisation_residual():
    from oracle.fp8_model import dequantize_split, quantize_per_head_split
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 2, 64, 32))
    x[0, 1, 3, 5] = 40.0
    hi, lo, scales = quantize_per_head_split(x)
    hi1, sc1 = quantize_per_head(x)
    np.testing.assert_array_equal(hi, hi1)
    np.testing.assert_array_equal(scales, sc1)
    # the residual never saturates: |16·r| ≤ 16·(half the largest step, 16) = 256
    assert np.max(np.abs(e4m3_decode(lo))) <= 256
    xr = dequantize_split(hi, lo, scales)
    t = x / scales[:, :, None, None]
    big = np.abs(t) >= 1.0
    rel = np.abs(xr - x)[big] / np.abs(x)[big]
    assert rel.max() <= 2.0 ** -7
    # the two-term value is closer than the one-term value
    one = dequantize(hi, scales)
    assert np.linalg.norm(xr - x) < np.linalg.norm(one - x) / 8


def test_per_row_split_quantisation():
    # One scale per row: each row's amax maps to the largest code, a zero row
    # gets scale 1 and zero codes, and the row quantises exactly as a head of
    # its own would (the per-head quantiser applied to that row alone).
    from oracle.fp8_model import (dequantize_split_rows, quantize_per_head_split,
                                  quantize_per_row_split)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 2, 16, 32))
    x[0, 1, 3, 5] = 40.0
    x[1, 0, 7] = 0.0
    hi, lo, scales = quantize_per_row_split(x)
    assert scales.shape == (2, 2, 16)
    assert scales[1, 0, 7] == 1.0 and np.all(hi[1, 0, 7] == 0) and np.all(lo[1, 0, 7] == 0)
    for b in range(2):
        for h in range(2):
            for r in range(16):
                if b == 1 and h == 0 and r == 7:
                    continue
                assert hi[b, h, r, np.argmax(np.abs(x[b, h, r]))] in (0x7E, 0xFE)
                h1, l1, s1 = quantize_per_head_split(x[b, h, r][None, None, None, :])
                np.testing.assert_array_equal(hi[b, h, r], h1[0, 0, 0])
                np.testing.assert_array_equal(lo[b, h, r], l1[0, 0, 0])
                assert scales[b, h, r] == s1[0, 0]
    # the outlier only coarsens its own row
    assert scales[0, 1, 3] > 4 * np.max(np.delete(scales[0, 1], 3))
    xr = dequantize_split_rows(hi, lo, scales)
    t = x / scales[..., None]
    big = np.abs(t) >= 1.0
    rel = np.abs(xr - x)[big] / np.abs(x)[big]
    assert rel.max() <= 2.0 ** -7


def test_per_row_scale_is_invariant_under_row_scaling():
    # Multiplying a row by a power of two leaves its codes unchanged and
    # multiplies only its scale.
    from oracle.fp8_model import quantize_per_row_split
    rng = np.random.default_rng(6)
    x = rng.standard_normal((1, 1, 8, 16))
    y = x.copy()
    y[0, 0, 2] *= 2.0 ** 5
    a = quantize_per_row_split(x)
    b = quantize_per_row_split(y)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    assert b[2][0, 0, 2] == a[2][0, 0, 2] * 32
    np.testing.assert_array_equal(np.delete(a[2][0, 0], 2), np.delete(b[2][0, 0], 2))


def test_fp8_model_block_mask_is_attention_on_dequantised_with_the_mask():
    # The block mask leaves the quantisation alone and restricts the
    # attention of the dequantised operands: the same codes as without a mask,
    # the output equal to the masked attention of the dequantised operands,
    # and an all-ones mask equal to no mask.
    from oracle.fp8_model import dequantize_split_rows
    rng = np.random.default_rng(11)
    q, k, v = (rng.standard_normal((1, 2, 300, 16)) for _ in range(3))
    mask = (rng.random((3, 3)) < 0.6).astype(np.uint8)
    mask[1] = 0
    m = fp8_attention_model(q, k, v, False, 0.25, rotate=True, seed=2, block_mask=mask)
    m0 = fp8_attention_model(q, k, v, False, 0.25, rotate=True, seed=2)
    for key in ("q8", "q8lo", "k8", "v8"):
        np.testing.assert_array_equal(m[key], m0[key])
    o, lse = attention_forward(dequantize_split_rows(m["q8"], m["q8lo"], m["sq"]),
                               dequantize_rows(m["k8"], m["sk"]),
                               dequantize_rows(m["v8"], m["sv"]), False, 0.25, block_mask=mask)
    np.testing.assert_array_equal(m["o"], o)
    np.testing.assert_array_equal(m["lse"], lse)
    assert np.all(m["o"][:, :, 128:256] == 0) and np.all(np.isneginf(m["lse"][:, :, 128:256]))
    ones = fp8_attention_model(q, k, v, False, 0.25, rotate=True, seed=2,
                               block_mask=np.ones((3, 3), dtype=np.uint8))
    np.testing.assert_allclose(ones["o"], m0["o"], rtol=0, atol=1e-14)


def test_fp8_model_segments_are_sequences_of_their_own():
    # Packed segments: every segment's rows equal the model run on that
    # segment alone as a separate input (its own K'/V scales over its own
    # rows, its own keys only), one segment over all rows equals the plain
    # model, and scaling one segment's K and V by 32 changes no other
    # segment's codes or outputs.
    rng = np.random.default_rng(12)
    q, k, v = (rng.standard_normal((1, 2, 200, 16)) for _ in range(3))
    cu = [0, 37, 37, 130, 200]
    for causal in (False, True):
        m = fp8_attention_model(q, k, v, causal, 0.25, rotate=True, seed=4, cu_seqlens=cu)
        assert m["sk"].shape == (1, 2, 200) and m["sv"].shape == (1, 2, 200)
        for s in range(4):
            a, b = cu[s], cu[s + 1]
            if b == a:
                continue
            alone = fp8_attention_model(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], causal, 0.25,
                                        rotate=True, seed=4)
            np.testing.assert_array_equal(m["k8"][:, :, a:b], alone["k8"])
            np.testing.assert_array_equal(m["v8"][:, :, a:b], alone["v8"])
            np.testing.assert_array_equal(m["sk"][:, :, a:b], alone["sk"])
            np.testing.assert_array_equal(m["sv"][:, :, a:b], alone["sv"])
            np.testing.assert_allclose(m["o"][:, :, a:b], alone["o"], rtol=0, atol=1e-13)
            np.testing.assert_allclose(m["lse"][:, :, a:b], alone["lse"], rtol=0, atol=1e-13)
    whole = fp8_attention_model(q, k, v, True, 0.25, rotate=True, seed=4, cu_seqlens=[0, 200])
    plain = fp8_attention_model(q, k, v, True, 0.25, rotate=True, seed=4)
    for key in ("k8", "v8", "o", "lse"):
        np.testing.assert_array_equal(whole[key], plain[key])
    np.testing.assert_array_equal(whole["sk"], plain["sk"])
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 37:130] *= 32
    v2[:, :, 37:130] *= 32
    m1 = fp8_attention_model(q, k, v, False, 0.25, rotate=True, seed=4, cu_seqlens=cu)
    m2 = fp8_attention_model(q, k2, v2, False, 0.25, rotate=True, seed=4, cu_seqlens=cu)
    keep = np.r_[0:37, 130:200]
    for key in ("k8", "v8", "o", "lse"):
        np.testing.assert_array_equal(m1[key][:, :, keep], m2[key][:, :, keep])
    assert not np.array_equal(m1["o"][:, :, 37:130], m2["o"][:, :, 37:130])


def test_scale_blocks_cover_each_segment_from_its_start():
    assert row_blocks(300) == [(0, 128), (128, 256), (256, 300)]
    assert row_blocks(300, [0, 5, 5, 140, 300]) == [(0, 5), (5, 133), (133, 140), (140, 268),
                                                    (268, 300)]


def test_per_block_quantisation_is_per_head_quantisation_of_each_block():
    # K': each block of 128 rows is quantised exactly as a head of its own
    # (the pinned per-head quantisation), and blocks do not see each other:
    # scaling one block by 2.5 leaves every code alone and that block's scale
    # times 2.5 (x·448/amax is the same exact ratio).
    rng = np.random.default_rng(21)
    x = rng.standard_normal((1, 2, 300, 16))
    x[0, 1, 140, 3] = 40.0  # an outlier in the second block of head 1
    codes, sc = quantize_per_block(x)
    for a, b in row_blocks(300):
        c1, s1 = quantize_per_head(x[:, :, a:b])
        np.testing.assert_array_equal(codes[:, :, a:b], c1)
        assert np.all(sc[:, :, a:b] == s1[:, :, None])
    y = x.copy()
    y[:, :, 128:256] *= 2.5
    c2, s2 = quantize_per_block(y)
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_allclose(s2[:, :, 128:256], 2.5 * sc[:, :, 128:256], rtol=1e-15)
    np.testing.assert_array_equal(s2[:, :, :128], sc[:, :, :128])


def test_pow2_scale_is_the_least_power_of_two_that_fits():
    amax = np.array([448.0, 448.0 * 2 ** -5, 449.0, 100.0, 3.0, 0.0])
    np.testing.assert_array_equal(pow2_scale(amax), [1.0, 2.0 ** -5, 2.0, 0.25, 2.0 ** -7, 1.0])
    s = pow2_scale(amax[:-1])
    assert np.all(amax[:-1] / s <= 448.0) and np.all(amax[:-1] / s > 224.0)


def test_pow2_scale_floor_is_the_least_normal_fp32_power():
    # Blocks whose amax is below 448·2^-126 keep the scale 2^-126 (the codes
    # are then smaller than 448, down to e4m3 subnormals or zero); at
    # 448·2^-126 exactly the least fitting power is that floor itself.
    amax = np.array([448 * 2.0 ** -126, 448 * 2.0 ** -127, 2.0 ** -140, 448 * 2.0 ** -125])
    np.testing.assert_array_equal(pow2_scale(amax),
                                  [2.0 ** -126, 2.0 ** -126, 2.0 ** -126, 2.0 ** -125])
    x = np.zeros((1, 1, 4, 2))
    x[0, 0, 0, 0] = 448 * 2.0 ** -128
    x[0, 0, 1, 1] = -2.0 ** -130
    codes, sc = quantize_per_block_pow2(x)
    assert np.all(sc == 2.0 ** -126)
    assert codes[0, 0, 0, 0] == 0x6E       # 112 = 1.75·2^6: biased exponent 13, mantissa 6/8
    assert codes[0, 0, 1, 1] == 0x98       # −2^-4: sign, biased exponent 3, mantissa 0
    np.testing.assert_array_equal(dequantize_rows(codes, sc), x)


def test_pow2_block_quantisation():
    # V: code = E4M3FN(v / 2^e) with the block's least fitting power of two;
    # the block maximum lands in (224, 448]; 448·2^k maps to code 0x7E
    # exactly; scaling a block by a power of two moves only its scale.
    rng = np.random.default_rng(22)
    x = rng.standard_normal((1, 1, 200, 8))
    x[0, 0, 5, 0] = 448.0 * 2.0 ** -4  # block 0's amax, a scaled maximum
    codes, sc = quantize_per_block_pow2(x)
    assert sc[0, 0, 0] == 2.0 ** -4 and codes[0, 0, 5, 0] == 0x7E
    for a, b in row_blocks(200):
        blk = np.abs(x[0, 0, a:b])
        assert 224.0 < blk.max() / sc[0, 0, a] <= 448.0
        np.testing.assert_array_equal(codes[0, 0, a:b], e4m3_encode(x[0, 0, a:b] / sc[0, 0, a]))
    y = x.copy()
    y[:, :, 128:] *= 8.0
    c2, s2 = quantize_per_block_pow2(y)
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(s2[:, :, 128:], 8.0 * sc[:, :, 128:])
    np.testing.assert_array_equal(s2[:, :, :128], sc[:, :, :128])
    # dequantised values within e4m3's half step of the inputs
    rel = np.abs(dequantize_rows(codes, sc) - x) / np.maximum(np.abs(x), 1e-300)
    big = np.abs(x) / sc[..., None] >= 2.0 ** -6  # normal e4m3 range
    assert rel[big].max() <= 2.0 ** -4 + 1e-12


def test_fp8_model_quantises_k_and_v_per_block():
    rng = np.random.default_rng(23)
    q, k, v = (rng.standard_normal((1, 1, 260, 16)) for _ in range(3))
    m = fp8_attention_model(q, k, v, False, 0.25, rotate=True, seed=5)
    from oracle.hadamard import rotate as _rot
    ck, sk = quantize_per_block(_rot(k, 5))
    cv, sv = quantize_per_block_pow2(v)
    for got, ref in ((m["k8"], ck), (m["sk"], sk), (m["v8"], cv), (m["sv"], sv)):
        np.testing.assert_array_equal(got, ref)
    assert len(np.unique(m["sk"][0, 0])) == 3 and len(np.unique(m["sv"][0, 0])) <= 3
