"""Pins for the float64 attention forward of the oracle (CPU only).

Each test fixes a property that the plain definition S = scale·Q·Kᵀ,
P = row-softmax(S), O = P·V must have, so that a dropped term, a wrong sign,
a wrong causal direction, a missing scale or a transposed operand in
``oracle.attention`` fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle.attention import (attention_forward, attention_forward_rows,
                              softmax_rows)
from oracle.brute import brute_forward

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _closed(expr):
    return eval(expr, {"__builtins__": {}}, {"e": math.e, "log": math.log})


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def test_golden_two_tokens():
    g = json.load(open(os.path.join(GOLDEN, "two_token_forward.json")))
    q = np.array(g["q"])[None, None]
    k = np.array(g["k"])[None, None]
    v = np.array(g["v"])[None, None]
    for key, causal in (("non_causal", False), ("causal", True)):
        o, lse = attention_forward(q, k, v, causal, g["scale"])
        exp_o = [_closed(x) for x in g[key]["o"]]
        exp_l = [_closed(x) for x in g[key]["lse"]]
        np.testing.assert_allclose(o[0, 0, :, 0], exp_o, rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse[0, 0], exp_l, rtol=0, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 1), (2, 3), (5, 4), (7, 8), (16, 3)])
def test_matches_brute_force(n, d, causal):
    q, k, v = (_rand((1, 1, n, d), s) for s in (1, 2, 3))
    scale = 0.7
    o, lse = attention_forward(q, k, v, causal, scale)
    bo, bl = brute_forward(q[0, 0].tolist(), k[0, 0].tolist(),
                           v[0, 0].tolist(), causal, scale)
    np.testing.assert_allclose(o[0, 0], np.array(bo), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], np.array(bl), rtol=0, atol=1e-13)


def test_softmax_rows_sum_to_one_and_masked_rows():
    s = _rand((9, 13), 4, 5.0)
    s[2, 5:] = -np.inf
    s[7, :] = -np.inf                      # a row with nothing visible
    p, lse = softmax_rows(s)
    sums = p.sum(axis=1)
    np.testing.assert_allclose(np.delete(sums, 7), 1.0, rtol=0, atol=1e-12)
    assert np.all(p[2, 5:] == 0)
    assert np.all(p[7] == 0) and lse[7] == -np.inf
    # LSE definition on a plain row
    np.testing.assert_allclose(lse[0], math.log(np.sum(np.exp(s[0]))), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_closed_form(causal):
    n, d, scale = 12, 6, 0.4
    q = _rand((1, 1, n, d), 5)
    krow = _rand((d,), 6)
    k = np.broadcast_to(krow, (1, 1, n, d)).copy()
    v = _rand((1, 1, n, d), 7)
    o, lse = attention_forward(q, k, v, causal, scale)
    for i in range(n):
        visible = i + 1 if causal else n
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, :visible].mean(axis=0),
                                   rtol=0, atol=1e-13)
        np.testing.assert_allclose(
            lse[0, 0, i], scale * q[0, 0, i] @ krow + math.log(visible),
            rtol=0, atol=1e-12)


def test_causal_row_zero_and_n_equals_one():
    q, k, v = (_rand((2, 3, 9, 5), s) for s in (8, 9, 10))
    scale = 0.3
    o, lse = attention_forward(q, k, v, True, scale)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0],
                               scale * np.sum(q[:, :, 0] * k[:, :, 0], -1),
                               rtol=0, atol=1e-14)
    for causal in (False, True):
        o1, l1 = attention_forward(q[:, :, :1], k[:, :, :1], v[:, :, :1],
                                   causal, scale)
        np.testing.assert_array_equal(o1, v[:, :, :1])


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    n, d, scale = 10, 4, 0.5
    q, k, v = (_rand((1, 2, n, d), s) for s in (11, 12, 13))
    u = _rand((d,), 14)
    o, lse = attention_forward(q, k, v, causal, scale)
    o2, lse2 = attention_forward(q, k + u, v, causal, scale)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse + scale * (q @ u), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_affine_in_v(causal):
    n, d, scale = 11, 5, 0.9
    q, k, v = (_rand((1, 1, n, d), s) for s in (15, 16, 17))
    c = _rand((d,), 18)
    w = _rand((d, 3), 19)
    o, _ = attention_forward(q, k, v, causal, scale)
    o_shift, _ = attention_forward(q, k, v + c, causal, scale)
    np.testing.assert_allclose(o_shift, o + c, rtol=0, atol=1e-13)
    o_lin, _ = attention_forward(q, k, v @ w, causal, scale)
    np.testing.assert_allclose(o_lin, o @ w, rtol=0, atol=1e-12)


def test_permutation_equivariance():
    n, d, scale = 13, 4, 0.6
    q, k, v = (_rand((1, 1, n, d), s) for s in (20, 21, 22))
    o, lse = attention_forward(q, k, v, False, scale)
    perm = np.random.default_rng(23).permutation(n)
    o_kv, lse_kv = attention_forward(q, k[:, :, perm], v[:, :, perm], False, scale)
    np.testing.assert_allclose(o_kv, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse_kv, lse, rtol=0, atol=1e-13)
    o_q, lse_q = attention_forward(q[:, :, perm], k, v, False, scale)
    np.testing.assert_allclose(o_q, o[:, :, perm], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse_q, lse[:, :, perm], rtol=0, atol=1e-13)


def test_hard_attention_limit():
    # With a huge scale the softmax becomes an argmax: O_i = V[argmax_j S_ij].
    n, d = 8, 3
    q, k, v = (_rand((1, 1, n, d), s) for s in (24, 25, 26))
    o, _ = attention_forward(q, k, v, False, 1e4)
    arg = np.argmax(q[0, 0] @ k[0, 0].T, axis=1)
    np.testing.assert_allclose(o[0, 0], v[0, 0, arg], rtol=0, atol=1e-9)


def test_scale_only_multiplies_scores():
    # scale·(Q·Kᵀ) == (scale·Q)·Kᵀ: moving the scale into Q gives the same result.
    q, k, v = (_rand((1, 1, 7, 4), s) for s in (27, 28, 29))
    o, lse = attention_forward(q, k, v, True, 0.25)
    o2, lse2 = attention_forward(q * 0.25, k, v, True, 1.0)
    np.testing.assert_allclose(o, o2, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_variant_matches_full(causal):
    q, k, v = (_rand((2, 2, 33, 8), s) for s in (30, 31, 32))
    o, lse = attention_forward(q, k, v, causal, 0.35)
    rows = np.array([0, 5, 17, 32])
    o_r, lse_r = attention_forward_rows(q, k, v, causal, 0.35, 1, 0, rows)
    np.testing.assert_allclose(o_r, o[1, 0, rows], atol=1e-14)
    np.testing.assert_allclose(lse_r, lse[1, 0, rows], atol=1e-14)


# Variable-length (packed) sequences: segments [c_s, c_{s+1}) of the rows.
VARLEN_CU = [[0, 3, 4, 11, 16], [0, 16], [0, 1, 2, 3, 16], [0, 0, 9, 9, 16]]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("cu", VARLEN_CU)
def test_varlen_matches_brute_force(cu, causal):
    n, d = 16, 5
    q, k, v = (_rand((1, 1, n, d), s) for s in (31, 32, 33))
    o, lse = attention_forward(q, k, v, causal, 0.6, cu_seqlens=cu)
    bo, bl = brute_forward(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), causal, 0.6,
                           cu_seqlens=cu)
    np.testing.assert_allclose(o[0, 0], np.array(bo), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], np.array(bl), rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equals_independent_segments(causal):
    # Each segment is its own attention problem: the packed result equals the
    # plain attention of every slice, and a single segment is plain attention.
    cu = [0, 5, 6, 40, 41, 77]
    q, k, v = (_rand((2, 2, 77, 8), s) for s in (41, 42, 43))
    o, lse = attention_forward(q, k, v, causal, 0.4, cu_seqlens=cu)
    for a, b in zip(cu[:-1], cu[1:]):
        so, sl = attention_forward(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], causal, 0.4)
        np.testing.assert_allclose(o[:, :, a:b], so, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[:, :, a:b], sl, rtol=0, atol=1e-13)
    o1, l1 = attention_forward(q, k, v, causal, 0.4, cu_seqlens=[0, 77])
    o2, l2 = attention_forward(q, k, v, causal, 0.4)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_varlen_rows_variant_and_uncovered_rows():
    cu = [0, 7, 20]
    q, k, v = (_rand((1, 2, 24, 4), s) for s in (51, 52, 53))
    o, lse = attention_forward(q, k, v, True, 0.5, cu_seqlens=cu)
    rows = np.array([0, 6, 7, 13, 19, 21, 23])
    ro, rl = attention_forward_rows(q, k, v, True, 0.5, 0, 1, rows, cu_seqlens=cu)
    np.testing.assert_allclose(ro, o[0, 1][rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(rl, lse[0, 1][rows], rtol=0, atol=1e-14)
    # rows 20..23 lie in no segment: they see no key
    assert np.all(o[:, :, 20:] == 0) and np.all(np.isneginf(lse[:, :, 20:]))


# Block-sparse masks (blocks of `block` rows × `block` keys).
def _bmask(nb, seed, density=0.5):
    return (np.random.default_rng(seed).random((nb, nb)) < density).astype(np.uint8)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seed", [61, 62, 63])
def test_block_mask_matches_brute_force(seed, causal):
    n, d, block = 14, 3, 4
    q, k, v = (_rand((1, 1, n, d), seed + s) for s in (0, 1, 2))
    m = _bmask(4, seed)
    m[0, 0] = 0  # a block row that may see nothing
    o, lse = attention_forward(q, k, v, causal, 0.8, block_mask=m, block=block)
    bo, bl = brute_forward(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), causal, 0.8,
                           block_mask=m.tolist(), block=block)
    np.testing.assert_allclose(o[0, 0], np.array(bo), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], np.array(bl), rtol=0, atol=1e-13)


def test_block_mask_special_cases():
    # all ones = plain; block-diagonal = packed segments of one block each;
    # lower-triangular blocks under the causal mask = causal; rows of a block
    # row with no visible block see nothing (O = 0, LSE = −∞); per-head masks.
    n, block = 40, 8
    q, k, v = (_rand((1, 3, n, 5), s) for s in (71, 72, 73))
    nb = 5
    ones = np.ones((nb, nb), np.uint8)
    for causal in (False, True):
        a = attention_forward(q, k, v, causal, 0.5, block_mask=ones, block=block)
        b = attention_forward(q, k, v, causal, 0.5)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    diag = np.eye(nb, dtype=np.uint8)
    a = attention_forward(q, k, v, False, 0.5, block_mask=diag, block=block)
    b = attention_forward(q, k, v, False, 0.5, cu_seqlens=list(range(0, n + 1, block)))
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-14)
    tril = np.tril(ones)
    a = attention_forward(q, k, v, True, 0.5, block_mask=tril, block=block)
    b = attention_forward(q, k, v, True, 0.5)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-14)
    m = ones.copy()
    m[2] = 0
    o, lse = attention_forward(q, k, v, False, 0.5, block_mask=m, block=block)
    assert np.all(o[:, :, 16:24] == 0) and np.all(np.isneginf(lse[:, :, 16:24]))
    per_head = np.stack([ones, diag, tril])
    o3, l3 = attention_forward(q, k, v, False, 0.5, block_mask=per_head, block=block)
    for h, mh in enumerate((ones, diag, tril)):
        oh, lh = attention_forward(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], False, 0.5,
                                   block_mask=mh, block=block)
        assert np.array_equal(o3[:, h:h + 1], oh) and np.array_equal(l3[:, h:h + 1], lh)
    rows = np.array([0, 15, 16, 23, 39])
    ro, rl = attention_forward_rows(q, k, v, False, 0.5, 0, 1, rows, block_mask=per_head,
                                    block=block)
    np.testing.assert_allclose(ro, o3[0, 1][rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(rl, l3[0, 1][rows], rtol=0, atol=1e-14)
