"""Shared helpers of the GPU parity tests (imported by tests only)."""
import numpy as np

import gen

# Tolerances.
#   NORTH_STAR: every layer output within 2e-3 * rms(out) of the oracle.
#   F32_BAR: with fp32 activations nothing is rounded below fp32; the error
#   of fp32 accumulation over K <= 6144 products, through SwiGLU and the down
#   projection, stays near 1e-5 relative; 1e-4 * rms leaves headroom while
#   still catching any dropped term or mis-scaled row (>= 1e-2 relative).
NORTH_STAR = 2e-3
F32_BAR = 1e-4


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt((ref ** 2).mean()))
    return float(np.abs(got - ref).max()) / rms, rms


def assert_close(got, ref, act_bf16, what=""):
    r, rms = rel_err(got, ref)
    assert r <= NORTH_STAR, f"{what}: max|err| = {r:.3e} * rms ({rms:.3e}) > {NORTH_STAR}"
    if not act_bf16:
        assert r <= F32_BAR, f"{what}: max|err| = {r:.3e} * rms > fp32 bar {F32_BAR}"
    return r


def oracle_eps(cfg):
    """The epsilon the C ABI receives is a float; hand the oracle the same value."""
    return float(np.float32(cfg.norm_eps))


def print_case(*parts):
    print("[case]", *parts, flush=True)
