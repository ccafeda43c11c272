"""Host check of the FMA-only exp2 used by the forward kernels (CPU only).

The kernel computes, in float32, n = floor(max(x, −200)), f = x − n,
p = fma(fma(fma(C3, f, C2), f, C1), f, 1) and ldexp(p, n). This test replays
those float32 steps in numpy (each fma rounded once to float32 from an exact
float64 product-sum) over a dense sweep of x ∈ [−126, 0] and checks the
relative error against float64 exp2: it must stay below 2^−12, eight times
under half a bfloat16 step (the pages only say the polynomial keeps the
precision BF16 needs; FlashAttention-4 gist, technical summary 2.B).
"""
import os
import re

import numpy as np

HDR = os.path.join(os.path.dirname(os.path.dirname(__file__)), "tiled_attention_fattn_amd",
                   "csrc", "exp2_poly_coeffs.h")


def coeffs():
    text = open(HDR).read()
    c = {int(m.group(1)): np.float32(float(m.group(2)))
         for m in re.finditer(r"kExp2PolyC(\d) = ([-0-9.e+]+)f", text)}
    return [c[i] for i in range(4)]


def fma32(a, b, c):
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def exp2_poly_emul(x):
    c0, c1, c2, c3 = coeffs()
    x = np.maximum(np.asarray(x, np.float32), np.float32(-200.0))
    n = np.floor(x)
    f = (x - n).astype(np.float32)
    p = fma32(np.full_like(f, c3), f, np.full_like(f, c2))
    p = fma32(p, f, np.full_like(f, c1))
    p = fma32(p, f, np.full_like(f, c0))
    return np.ldexp(p.astype(np.float64), n.astype(np.int64)).astype(np.float32)


def test_poly_relative_error_bound():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        -rng.uniform(0, 126, 2_000_000),
        -np.linspace(0, 1, 1_000_001),                       # one full fraction period
        -rng.uniform(0, 1e-3, 100_000),                      # tiny negatives
    ]).astype(np.float32)
    y = exp2_poly_emul(x).astype(np.float64)
    ref = np.exp2(x.astype(np.float64))
    rel = np.abs(y / ref - 1.0)
    assert rel.max() <= 2.0 ** -12, rel.max()


def test_poly_special_values():
    assert exp2_poly_emul(np.array([-np.inf], np.float32))[0] == 0.0
    ints = -np.arange(0, 127, dtype=np.float32)
    np.testing.assert_array_equal(exp2_poly_emul(ints), np.exp2(ints.astype(np.float64)))
    assert coeffs()[0] == 1.0
