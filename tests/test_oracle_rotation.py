"""Pins for the Hadamard rotation and SplitMix64 signs of the oracle (CPU only)."""
import numpy as np
import pytest

from oracle.attention import attention_forward
from oracle.hadamard import fwht, rotate, rotation_signs, splitmix64, sylvester


def test_splitmix64_published_sequences():
    # Outputs of the published SplitMix64 generator (Steele, Lea & Flood 2014;
    # S. Vigna's reference C code): state 1234567 and state 0.
    assert splitmix64(1234567, 5) == [
        6457827717110365317, 3203168211198807973, 9817491932198370423,
        4593380528125082431, 16408922859458223821]
    assert splitmix64(0, 3) == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                0x06C45D188009454F]


def test_signs_follow_top_bit():
    outs = splitmix64(42, 128)
    s = rotation_signs(42, 128)
    assert s.shape == (128,)
    for x, si in zip(outs, s):
        assert si == (-1.0 if x >> 63 else 1.0)
    # a fair generator gives both signs
    assert 30 < np.sum(s > 0) < 98


def test_sylvester_small_and_orthogonality():
    np.testing.assert_array_equal(sylvester(1), [[1]])
    np.testing.assert_array_equal(sylvester(2), [[1, 1], [1, -1]])
    np.testing.assert_array_equal(sylvester(4), [[1, 1, 1, 1], [1, -1, 1, -1],
                                                 [1, 1, -1, -1], [1, -1, -1, 1]])
    for d in (8, 64, 128):
        h = sylvester(d)
        np.testing.assert_array_equal(h @ h.T, d * np.eye(d))
        np.testing.assert_array_equal(h, h.T)
    with pytest.raises(ValueError):
        sylvester(12)


@pytest.mark.parametrize("d", [1, 2, 8, 64, 128])
def test_fwht_equals_matrix(d):
    x = np.random.default_rng(d).standard_normal((5, 3, d))
    np.testing.assert_allclose(fwht(x), x @ sylvester(d), rtol=0, atol=1e-12)


@pytest.mark.parametrize("d", [64, 128])
def test_rotation_is_orthogonal_and_preserves_scores(d):
    seed = 5
    r = np.diag(rotation_signs(seed, d)) @ sylvester(d) / np.sqrt(d)
    np.testing.assert_allclose(r @ r.T, np.eye(d), rtol=0, atol=1e-15)
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 2, 40, d))
    k = rng.standard_normal((1, 2, 40, d))
    q_r, k_r = rotate(q, seed), rotate(k, seed)
    np.testing.assert_allclose(q_r, q @ r, rtol=0, atol=1e-13)
    qk = q @ np.swapaxes(k, -1, -2)
    qk_r = q_r @ np.swapaxes(k_r, -1, -2)
    rel = np.max(np.abs(qk_r - qk)) / np.max(np.abs(qk))
    assert rel <= 1e-12
    # the whole attention is unchanged
    v = rng.standard_normal((1, 2, 40, d))
    o, lse = attention_forward(q, k, v, False, d ** -0.5)
    o_r, lse_r = attention_forward(q_r, k_r, v, False, d ** -0.5)
    np.testing.assert_allclose(o_r, o, atol=1e-12)
    np.testing.assert_allclose(lse_r, lse, atol=1e-12)


def test_rotation_spreads_an_outlier():
    # A single large coordinate is spread evenly: |x'| = |x_j|/√d everywhere.
    d = 128
    x = np.zeros((1, d))
    x[0, 17] = 20.0
    xr = rotate(x, 3)
    np.testing.assert_allclose(np.abs(xr), 20.0 / np.sqrt(d), rtol=0, atol=1e-13)
