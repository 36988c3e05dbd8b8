"""Pins of the oracle's dequant-on-use SwiGLU expert (CPU only)."""
import json
import os

import numpy as np
import pytest
from scipy.special import expit

import gen
import oracle


def _pack_int4_rows(q):
    q = np.asarray(q, dtype=np.int64)
    lo, hi = q[:, 0::2] & 15, q[:, 1::2] & 15
    return (lo | (hi << 4)).astype(np.uint8)


def _bf16_bits(v):
    return gen.f32_to_bf16_bits(np.asarray(v, np.float32))


def _hand_expert(g, dtype):
    I, H = g["inter"], g["hidden"]
    gu = np.array(g["gate_rows"] + g["up_rows"])
    dn = np.array(g["down_rows"])
    if dtype == oracle.BF16:
        return dict(gate_up=_bf16_bits(gu), down=_bf16_bits(dn), gate_up_scale=None,
                    down_scale=None)
    return dict(gate_up=_pack_int4_rows(gu), down=_pack_int4_rows(dn),
                gate_up_scale=np.ones(2 * I, np.float32), down_scale=np.ones(H, np.float32))


@pytest.mark.parametrize("dtype", [oracle.I4, oracle.BF16])
def test_hand_example(golden_dir, dtype):
    g = json.load(open(os.path.join(golden_dir, "ffn_hand_example.json")))
    d = oracle.Desc(hidden=g["hidden"], inter=g["inter"], n_experts=1, top_k=1, expert_dtype=dtype)
    es = oracle.ExpertSet(dtype, [_hand_expert(g, dtype)])
    x = np.array([g["x"]], np.float32)
    y = oracle.expert_ffn(d, es, 0, x, n_rows=1)
    assert y[0].tolist() == g["y"]


@pytest.mark.parametrize("dtype", [oracle.I4, oracle.BF16])
def test_hand_example_h(golden_dir, dtype):
    """The SwiGLU output before rounding, on the hand example: h = (logistic(1), 0)."""
    g = json.load(open(os.path.join(golden_dir, "ffn_hand_example.json")))
    d = oracle.Desc(hidden=g["hidden"], inter=g["inter"], n_experts=1, top_k=1, expert_dtype=dtype)
    es = oracle.ExpertSet(dtype, [_hand_expert(g, dtype)])
    x = np.array([g["x"]], np.float32)
    assert oracle.expert_h(d, es, 0, x, n_rows=1)[0].tolist() == g["h"]


def test_expert_h_matches_a_dense_swiglu():
    """expert_h on a random int4 expert equals silu(G x) * (U x) from the
    decoded codes and scales (numpy, fp64), and with f32 activations the
    expert's output is the down matrix applied to that h."""
    cfg = gen.shrink(gen.get_config("c0"), seed=12)
    ex = gen.expert(cfg, 0, 3)
    H, I = cfg.hidden, cfg.inter
    d = oracle.Desc(hidden=H, inter=I, n_experts=1, top_k=1, expert_dtype=oracle.I4)
    es = oracle.ExpertSet(oracle.I4, [ex])
    x = gen.x_tokens(cfg, 3, batch_id=2)
    h = oracle.expert_h(d, es, 0, x, n_rows=3)
    gu = _np_codes(ex["gate_up"], H, oracle.I4) * ex["gate_up_scale"].astype(np.float64)[:, None]
    dn = _np_codes(ex["down"], I, oracle.I4) * ex["down_scale"].astype(np.float64)[:, None]
    xv = x.astype(np.float64)
    g, u = xv @ gu[:I].T, xv @ gu[I:].T
    np.testing.assert_allclose(h, g * expit(g) * u, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(oracle.expert_ffn(d, es, 0, x, n_rows=3), h @ dn.T, rtol=1e-12,
                               atol=1e-14)


def test_hand_example_bf16_activation(golden_dir):
    """With bf16 activations h is rounded to bf16: logistic(1) -> 0.73046875."""
    g = json.load(open(os.path.join(golden_dir, "ffn_hand_example.json")))
    d = oracle.Desc(hidden=2, inter=2, n_experts=1, top_k=1, expert_dtype=oracle.I4, act_bf16=1)
    es = oracle.ExpertSet(oracle.I4, [_hand_expert(g, oracle.I4)])
    x = _bf16_bits(np.array([g["x"]], np.float32))
    y = oracle.expert_ffn(d, es, 0, x, n_rows=1)
    assert y[0].tolist() == [2 * 0.73046875, -0.73046875]


def _np_codes(packed, cols, dtype):
    packed = np.asarray(packed, np.uint8)
    if dtype == oracle.I4:
        lo = ((packed << 4).astype(np.int8) >> 4)
        hi = packed.astype(np.int8) >> 4
        out = np.empty((packed.shape[0], cols), np.int64)
        out[:, 0::2], out[:, 1::2] = lo, hi
        return out
    out = np.empty((packed.shape[0], cols), np.int64)
    for j in range(4):
        out[:, j::4] = (packed << (6 - 2 * j)).astype(np.int8) >> 6
    return out


@pytest.mark.parametrize("dtype", [oracle.I4, oracle.I2])
def test_integer_matrix_case(dtype):
    """Unit scales and integer activations: the projections are exact integer
    matmuls; silu from scipy's logistic."""
    H, I = 64, 32
    cfg = gen.shrink(gen.get_config("c0"), hidden=H, inter=I)
    ex = gen.expert(cfg, 0, 1, dtype=dtype)
    ex["gate_up_scale"] = np.ones(2 * I, np.float32)
    ex["down_scale"] = np.ones(H, np.float32)
    d = oracle.Desc(hidden=H, inter=I, n_experts=1, top_k=1, expert_dtype=dtype)
    rng = np.random.default_rng(2)
    x = rng.integers(-3, 4, size=(4, H)).astype(np.float32)
    y = oracle.expert_ffn(d, oracle.ExpertSet(dtype, [ex]), 0, x, n_rows=4)
    Q = _np_codes(ex["gate_up"], H, dtype).astype(np.float64)
    D = _np_codes(ex["down"], I, dtype).astype(np.float64)
    G, U = x.astype(np.float64) @ Q[:I].T, x.astype(np.float64) @ Q[I:].T
    h = G * expit(G) * U
    want = h @ D.T
    assert np.allclose(y, want, rtol=1e-13, atol=1e-13 * np.abs(want).max())


def test_power_of_two_scale_invariance():
    cfg = gen.get_config("c0")
    ex = gen.expert(cfg, 0, 3)
    d = oracle.Desc.from_config(cfg)
    x = gen.x_tokens(cfg, 3)
    y0 = oracle.expert_ffn(d, oracle.ExpertSet(oracle.I4, [ex]), 0, x, n_rows=3)
    ex2 = dict(ex, down_scale=ex["down_scale"] * np.float32(2))
    y2 = oracle.expert_ffn(d, oracle.ExpertSet(oracle.I4, [ex2]), 0, x, n_rows=3)
    assert np.array_equal(y2, 2 * y0)
    up2 = ex["gate_up_scale"].copy()
    up2[cfg.inter:] *= np.float32(4)
    ex3 = dict(ex, gate_up_scale=up2)
    y3 = oracle.expert_ffn(d, oracle.ExpertSet(oracle.I4, [ex3]), 0, x, n_rows=3)
    assert np.array_equal(y3, 4 * y0)


def test_rows_and_row_div():
    cfg = gen.get_config("c0")
    ex = gen.expert(cfg, 0, 2)
    d = oracle.Desc.from_config(cfg)
    es = oracle.ExpertSet(oracle.I4, [None, None, ex])
    x = gen.x_tokens(cfg, 5)
    full = oracle.expert_ffn(d, es, 2, x, n_rows=5)
    rows = np.array([9, 0, 4, 5], np.int32)          # slots f, token = f // 2
    y = oracle.expert_ffn(d, es, 2, x, rows=rows, row_div=2)
    assert np.array_equal(y, full[rows // 2])
    with pytest.raises(oracle.OracleError):
        oracle.expert_ffn(d, es, 1, x, n_rows=1)     # expert 1 not provided
