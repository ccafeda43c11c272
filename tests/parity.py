"""Error metrics and tolerances for comparing the HIP path with the oracle.

Tolerances: bf16 outputs (O, dQ, dK, dV) must be within max-abs 2e-2 and
relative RMS 5e-3 of the float64 oracle; the fp8 forward's O within relative
RMS 6e-2. LSE (fp32, computed from fp32 running statistics) is held to
max-abs 2e-3.
"""
import numpy as np

BF16_MAX_ABS = 2e-2
BF16_REL_RMS = 5e-3
FP8_REL_RMS = 6e-2
LSE_MAX_ABS = 2e-3


def max_abs(x, ref):
    return float(np.max(np.abs(np.asarray(x, np.float64) - np.asarray(ref, np.float64))))


def rel_rms(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    return float(num / den) if den > 0 else float(num)


def assert_bf16_close(x, ref, what):
    ma, rr = max_abs(x, ref), rel_rms(x, ref)
    assert np.all(np.isfinite(x)), f"{what}: non-finite values"
    assert ma <= BF16_MAX_ABS and rr <= BF16_REL_RMS, \
        f"{what}: max-abs {ma:.3e} (<= {BF16_MAX_ABS}), rel-RMS {rr:.3e} (<= {BF16_REL_RMS})"
    return ma, rr


def assert_lse_close(x, ref, what):
    ma = max_abs(x, ref)
    assert np.all(np.isfinite(x)), f"{what}: non-finite LSE"
    assert ma <= LSE_MAX_ABS, f"{what}: LSE max-abs {ma:.3e} (<= {LSE_MAX_ABS})"
    return ma


def to_np(t):
    """GPU tensor → float64 numpy array."""
    return t.detach().float().cpu().numpy().astype(np.float64)
