"""Pins for the float64 attention backward of the oracle (CPU only).

Finite differences of L = Σ O∘dO fix every gradient independently of the
formulas in ``oracle.attention.attention_backward``; the brute-force loop uses
the full softmax Jacobian instead of the D shortcut; the invariants follow
from rows of P summing to one.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle.attention import attention_backward, attention_forward
from oracle.brute import brute_backward

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _loss(q, k, v, do, causal, scale):
    o, _ = attention_forward(q, k, v, causal, scale)
    return float(np.sum(o * do))


def _numeric_grad(f, x, h=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        old = x[idx]
        x[idx] = old + h
        fp = f()
        x[idx] = old - h
        fm = f()
        x[idx] = old
        g[idx] = (fp - fm) / (2 * h)
    return g


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 2), (2, 2), (3, 4), (7, 4)])
def test_finite_differences(n, d, causal):
    scale = 0.8
    q, k, v, do = (_rand((1, 1, n, d), s) for s in (1, 2, 3, 4))
    dq, dk, dv, _ = attention_backward(q, k, v, do, causal, scale)
    f = lambda: _loss(q, k, v, do, causal, scale)  # noqa: E731
    for analytic, x in ((dq, q), (dk, k), (dv, v)):
        num = _numeric_grad(f, x)
        err = np.max(np.abs(analytic - num))
        ref = max(1.0, np.max(np.abs(num)))
        assert err / ref <= 1e-6, (err, ref)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 1), (4, 3), (9, 5)])
def test_matches_brute_force(n, d, causal):
    scale = 0.45
    q, k, v, do = (_rand((1, 1, n, d), s) for s in (5, 6, 7, 8))
    dq, dk, dv, _ = attention_backward(q, k, v, do, causal, scale)
    bq, bk, bv = brute_backward(q[0, 0].tolist(), k[0, 0].tolist(),
                                v[0, 0].tolist(), do[0, 0].tolist(), causal, scale)
    np.testing.assert_allclose(dq[0, 0], np.array(bq), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk[0, 0], np.array(bk), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv[0, 0], np.array(bv), rtol=0, atol=1e-12)


def test_golden_two_tokens():
    g = json.load(open(os.path.join(GOLDEN, "two_token_backward.json")))
    arr = lambda key: np.array(g[key])[None, None]  # noqa: E731
    dq, dk, dv, _ = attention_backward(arr("q"), arr("k"), arr("v"), arr("do"),
                                       False, g["scale"])
    ev = lambda xs: [eval(x, {"__builtins__": {}}, {"e": math.e}) for x in xs]  # noqa: E731
    np.testing.assert_allclose(dq[0, 0, :, 0], ev(g["dq"]), atol=1e-15)
    np.testing.assert_allclose(dk[0, 0, :, 0], ev(g["dk"]), atol=1e-15)
    np.testing.assert_allclose(dv[0, 0, :, 0], ev(g["dv"]), atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    n, d, scale = 17, 6, 0.3
    q, k, v, do = (_rand((2, 2, n, d), s) for s in (9, 10, 11, 12))
    dq, dk, dv, dvec = attention_backward(q, k, v, do, causal, scale)
    # Σ_j dK_j = scale·Σ_i Q_i Σ_j dS_ij = 0 because rows of dS sum to 0.
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    # Σ_j dV_j = Σ_i dO_i Σ_j P_ij = Σ_i dO_i.
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)
    # D = rowsum(dO ∘ O).
    o, _ = attention_forward(q, k, v, causal, scale)
    np.testing.assert_allclose(dvec, np.sum(do * o, axis=-1), atol=1e-12)


def test_single_token():
    q, k, v, do = (_rand((1, 3, 1, 4), s) for s in (13, 14, 15, 16))
    for causal in (False, True):
        dq, dk, dv, _ = attention_backward(q, k, v, do, causal, 0.5)
        np.testing.assert_array_equal(dq, 0.0)
        np.testing.assert_array_equal(dk, 0.0)
        np.testing.assert_array_equal(dv, do)


def test_causal_last_key_only_seen_by_last_query():
    # Under the causal mask key N-1 is visible only to query N-1, so
    # dV_{N-1} = P_{N-1,N-1} · dO_{N-1}.
    n, d, scale = 6, 3, 0.7
    q, k, v, do = (_rand((1, 1, n, d), s) for s in (17, 18, 19, 20))
    _, _, dv, _ = attention_backward(q, k, v, do, True, scale)
    s_last = scale * q[0, 0, -1] @ k[0, 0].T
    p_last = np.exp(s_last - s_last.max())
    p_last /= p_last.sum()
    np.testing.assert_allclose(dv[0, 0, -1], p_last[-1] * do[0, 0, -1], atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_gradients_equal_independent_segments(causal):
    # Packed segments do not interact: every gradient equals that of the
    # segment's own attention problem.
    cu = [0, 1, 9, 10, 33]
    rng = np.random.default_rng(77)
    q, k, v, do = (rng.standard_normal((1, 2, 33, 6)) for _ in range(4))
    dq, dk, dv, dvec = attention_backward(q, k, v, do, causal, 0.5, cu_seqlens=cu)
    for a, b in zip(cu[:-1], cu[1:]):
        sl = (slice(None), slice(None), slice(a, b))
        rq, rk, rv, rd = attention_backward(q[sl], k[sl], v[sl], do[sl], causal, 0.5)
        for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
            np.testing.assert_allclose(got[sl], ref, rtol=0, atol=1e-13)
        np.testing.assert_allclose(dvec[sl], rd, rtol=0, atol=1e-13)


def test_varlen_finite_differences():
    # Central differences of L = <O, dO> through the segment-masked forward.
    cu = [0, 2, 3, 7]
    rng = np.random.default_rng(78)
    q, k, v, do = (rng.standard_normal((1, 1, 7, 3)) for _ in range(4))
    dq, dk, dv, _ = attention_backward(q, k, v, do, True, 0.9, cu_seqlens=cu)

    def loss(qq, kk, vv):
        return float(np.sum(attention_forward(qq, kk, vv, True, 0.9, cu_seqlens=cu)[0] * do))
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = loss(args["q"], args["k"], args["v"])
            args[name] = xm
            lm = loss(args["q"], args["k"], args["v"])
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


def test_block_mask_finite_differences_and_empty_rows():
    # Central differences through the block-masked forward; rows of a block
    # row that sees no key get zero dQ and contribute nothing to dK, dV.
    block = 3
    m = np.array([[1, 0, 1], [0, 0, 0], [1, 1, 0]], dtype=np.uint8)
    rng = np.random.default_rng(79)
    q, k, v, do = (rng.standard_normal((1, 1, 8, 3)) for _ in range(4))
    for causal in (False, True):
        dq, dk, dv, _ = attention_backward(q, k, v, do, causal, 0.7, block_mask=m, block=block)
        assert np.all(dq[0, 0, 3:6] == 0)

        def loss(qq, kk, vv):
            return float(np.sum(attention_forward(qq, kk, vv, causal, 0.7, block_mask=m,
                                                  block=block)[0] * do))
        h = 1e-6
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args = {"q": q, "k": k, "v": v}
                args[name] = xp
                lp = loss(args["q"], args["k"], args["v"])
                args[name] = xm
                lm = loss(args["q"], args["k"], args["v"])
                num[idx] = (lp - lm) / (2 * h)
            np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)
