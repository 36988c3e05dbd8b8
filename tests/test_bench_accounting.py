"""The benchmark's algorithmic work figures (the numerators of its roofline)
against closed forms written out here from the layer's shapes.

GLM decode layer: H 6144, I 2048, int4 routed experts with per-row fp32
scales, top-8, f32 activations, a bf16 shared expert that runs with the
router at one token.  Prefill: 2048 tokens, bf16 activations, the shared
expert's gate/up in the same stage.
"""
import pytest

import gen

bench = pytest.importorskip("bench")

H, I, K = 6144, 2048, 8


def test_decode_gate_up_bytes_closed_form():
    cfg = gen.get_config("c2")
    assert (cfg.hidden, cfg.inter, cfg.top_k) == (H, I, K)
    codes = 2 * I * H // 2          # gate and up rows, two int4 codes per byte
    scales = 2 * I * 4              # one fp32 scale per row
    x_in = H * 4                    # one f32 activation row
    h_out = K * I * 4               # one f32 h row per slot
    want = K * (codes + scales) + x_in + h_out
    assert want == 100_884_480
    # the launch also runs the shared expert's down projection: its bf16
    # [H][I] weights, its f32 h row in, its f32 output row out
    s_down = H * I * 2 + I * 4 + H * 4
    assert bench.shared_runs_with_router(cfg, gen.I4, 1)
    assert bench.shared_down_in_gate_up(cfg, gen.I4, 1)
    assert bench.gate_up_bytes(cfg, gen.I4, K, 1) == want + s_down
    assert want + s_down == 126_083_072


def test_decode_gate_up_bytes_shared_in_launch():
    # with a batch past the decode size the shared expert shares the gate/up
    # launch, and its bf16 gate/up rows and h rows count there
    cfg = gen.get_config("c2")
    T = 17
    assert not bench.shared_runs_with_router(cfg, gen.I4, T)
    routed = 40 * (2 * I * H // 2 + 2 * I * 4) + T * H * 4 + T * K * I * 4
    shared = 2 * I * H * 2 + T * I * 4
    assert bench.gate_up_bytes(cfg, gen.I4, 40, T) == routed + shared


def test_int2_and_int8_rows_count_as_ring_streamed():
    cfg = gen.get_config("c4")
    for dt in (gen.I2, gen.I4, gen.I8):
        assert bench.shared_runs_with_router(cfg, dt, 16)
    assert not bench.shared_runs_with_router(cfg, gen.I4, 17)


def test_prefill_gate_up_flops_closed_form():
    cfg = gen.get_config("c3")
    T = 2048
    routed = 2 * T * K * (2 * I) * H      # 2 flops per weight, every (token, expert) pair
    shared = 2 * T * (2 * I) * H          # every token through the shared expert
    assert routed + shared == 927_712_935_936
    assert bench.gate_up_flops(cfg, T) == routed + shared
