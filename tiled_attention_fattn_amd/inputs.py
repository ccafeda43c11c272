"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds no attention arithmetic: it only draws random numbers,
rounds them to bfloat16 and describes the workloads. Both the HIP path and
the CPU oracle consume exactly the values produced here.

Recipe (per workload index k, tensor stream t):
  * ``numpy.random.default_rng([k, t])`` with t = 0 for Q, 1 for K, 2 for V,
    3 for dO, 4 and 5 for the positions of the Q and K outliers;
  * i.i.d. N(0, 1) in float64;
  * outliers (fp8 workload only): exactly round(0.001·numel) distinct
    positions per tensor, drawn without replacement, multiplied by 20 before
    rounding;
  * one rounding to bfloat16, to nearest with ties to even.
"""
import numpy as np

# The five workloads: one forward correctness case, two forward throughput
# cases (causal N=2048 and non-causal N=8192), one backward, one fp8 forward.
WORKLOADS = {
    1: dict(name="fwd_b1h2n256d64", kind="fwd", B=1, H=2, N=256, d=64, causal=False),
    2: dict(name="fwd_causal_b8h16n2048d128", kind="fwd", B=8, H=16, N=2048, d=128, causal=True),
    3: dict(name="fwd_b2h16n8192d128", kind="fwd", B=2, H=16, N=8192, d=128, causal=False),
    4: dict(name="bwd_causal_b4h16n4096d128", kind="bwd", B=4, H=16, N=4096, d=128, causal=True),
    5: dict(name="fp8_fwd_b4h16n4096d128", kind="fp8", B=4, H=16, N=4096, d=128, causal=False,
            outlier_frac=0.001, outlier_factor=20.0, rotate=True),
}

_STREAM = {"q": 0, "k": 1, "v": 2, "do": 3}
_OUTLIER_STREAM = {"q": 4, "k": 5}


def bf16_round(x):
    """Round float64 values to bfloat16, nearest-even.

    Returns (values as float64, raw bfloat16 bit patterns as uint16).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m·2^e, 0.5 <= |m| < 1
    normal = np.abs(x) >= 2.0 ** -126
    y_norm = np.ldexp(np.rint(m * 256.0) / 256.0, e)
    y_sub = np.rint(x * 2.0 ** 133) * 2.0 ** -133
    y = np.where(normal, y_norm, y_sub)
    if np.any(np.abs(y) > 3.3895313892515355e38):
        raise ValueError("value outside the bfloat16 range")
    bits = (y.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return y, bits


def gen_tensor(k, name, shape, outlier_frac=0.0, outlier_factor=1.0):
    """One input tensor of workload k. Returns (float64 values, uint16 bf16 bits)."""
    x = np.random.default_rng([k, _STREAM[name]]).standard_normal(shape)
    if outlier_frac > 0 and name in _OUTLIER_STREAM:
        count = int(round(outlier_frac * x.size))
        pos = np.random.default_rng([k, _OUTLIER_STREAM[name]]).choice(
            x.size, size=count, replace=False)
        flat = x.reshape(-1)
        flat[pos] *= outlier_factor
    return bf16_round(x)


def gen_workload(k, names=("q", "k", "v"), shape=None, **overrides):
    """Inputs of workload k (or of a custom shape with k as the seed)."""
    w = dict(WORKLOADS.get(k, {}))
    w.update(overrides)
    if shape is None:
        shape = (w["B"], w["H"], w["N"], w["d"])
    out = {}
    for n in names:
        out[n] = gen_tensor(k, n, shape, w.get("outlier_frac", 0.0), w.get("outlier_factor", 1.0))
    return out


def to_device_bf16(bits, device="cuda"):
    """uint16 bit patterns → torch.bfloat16 tensor on `device`."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def flops_fwd(B, H, N, d, causal):
    """Algorithmic FLOP of the forward: 4·B·H·N²·d, halved under causal."""
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def flops_bwd(B, H, N, d, causal):
    """Algorithmic FLOP of the backward: 2.5× the forward's."""
    return 2.5 * flops_fwd(B, H, N, d, causal)
