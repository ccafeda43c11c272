"""Random-sign Hadamard rotation for incoherent processing — TEST INFRASTRUCTURE ONLY.

[FA3-wiki] innovation 3 ("Baja precisión (FP8) con reducción del error de
cuantización"): before fp8 quantisation, Q and K are multiplied by a random
orthogonal matrix, for example a Hadamard matrix; because the matrix is
orthogonal its effect cancels in Q·Kᵀ.

Reading used here (the page names no construction): the rotation is

    R = diag(s) · H_d / √d,     x' = x · R   for every row vector x,

where H_d is the Sylvester Hadamard matrix in natural order (H_1 = [1],
H_2m = [[H_m, H_m], [H_m, −H_m]]) and s ∈ {±1}^d is a sign vector drawn from
SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014): s_i = +1 when the top bit of the i-th output
(i = 0, 1, …) of the generator seeded with ``seed`` is 0, else −1. The same R
is applied to Q and to K.
"""
import numpy as np

_MASK = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15


def splitmix64(seed, count):
    """First ``count`` outputs of SplitMix64 started from state ``seed``.

    Each step adds the golden-ratio increment to the state and returns the
    state passed through the two xor-shift-multiply rounds and a final
    xor-shift. Returns a list of Python ints in [0, 2^64).
    """
    state = seed & _MASK
    out = []
    for _ in range(count):
        state = (state + _GAMMA) & _MASK
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK
        out.append(z ^ (z >> 31))
    return out


def rotation_signs(seed, d):
    """Sign vector s (float64 ±1, length d): +1 iff output i has top bit 0."""
    return np.array([-1.0 if (x >> 63) else 1.0 for x in splitmix64(seed, d)],
                    dtype=np.float64)


def sylvester(d):
    """Sylvester Hadamard matrix H_d (entries ±1) for d a power of two."""
    if d < 1 or (d & (d - 1)) != 0:
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def fwht(x):
    """Unnormalised fast Walsh–Hadamard transform along the last axis.

    Equals x @ H_d (H_d symmetric) computed with log2(d) butterfly stages:
    at stage with half-width w, pairs (a, b) at distance w become (a+b, a−b).
    """
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    if d < 1 or (d & (d - 1)) != 0:
        raise ValueError("last dimension must be a power of two")
    w = 1
    while w < d:
        y = y.reshape(y.shape[:-1] + (d // (2 * w), 2, w))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (d,))
        w *= 2
    return y


def rotate(x, seed):
    """x · diag(s) · H_d / √d along the last axis (float64)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    s = rotation_signs(seed, d)
    return fwht(x * s) / np.sqrt(d)
