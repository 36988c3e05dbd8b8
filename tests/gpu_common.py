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

# bf16 activations: h is rounded to bf16 on both sides, each side deciding in
# its own accumulation order, so an h lying within the kernels' error of a
# rounding midpoint may round either way; oracle.layer_band gives the output
# effect of all such alternatives.  The kernels' error on h is measured (by
# tests/test_gpu_h_error.py) in units of u * e, u = 2^-24 the fp32 unit
# roundoff and e the first-order error scale of h from rounding the terms of
# its sums (oracle.expert_h): the window is BF16_KAPPA such units.
BF16_KAPPA = 4.0
BF16_WINDOW = BF16_KAPPA * 2.0 ** -24


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


def assert_close_band(got, ref, band, what=""):
    """bf16 activations: |got - ref| <= 2e-3 * rms(ref) + band, elementwise,
    where band bounds the effect of valid alternative roundings of h."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt((ref ** 2).mean()))
    excess = np.abs(got - ref) - band
    r = float(excess.max()) / rms
    assert r <= NORTH_STAR, (f"{what}: max(|err| - band) = {r:.3e} * rms ({rms:.3e}) > "
                             f"{NORTH_STAR}; max|err| = {float(np.abs(got - ref).max()) / rms:.3e}"
                             f", max band = {float(band.max()) / rms:.3e}")
    return float(np.abs(got - ref).max()) / rms, float(band.max()) / rms


def oracle_eps(cfg):
    """The epsilon the C ABI receives is a float; hand the oracle the same value."""
    return float(np.float32(cfg.norm_eps))


def print_case(*parts):
    print("[case]", *parts, flush=True)
