"""GPU parity of the layer at the wider hidden sizes of DeepSeek-V3-class
layers (H 7168 and 8192, the GLM cases being H 6144).

The decode GEMV streams each weight row as 64 lanes times a slice of K/64
elements, compiled for slices of 32, 64, 96 and 128 elements (and, for bf16
weights, 8, 16, 112).  H 8192 therefore runs every format on the decode
path; H 7168 gives 112-element slices, which the bf16 kernels take but which
are not whole 32-code granules of the integer formats: int4 at H 7168 on a
decode batch reports MOE_EUNSUPPORTED, and the same layer runs on the grouped
GEMM for prefill batches.  Every case compares routing bit for bit and the
outputs with the oracle.
"""
import numpy as np
import pytest

import gen
import oracle
from tests.gpu_common import BF16_WINDOW, assert_close, assert_close_band, print_case

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gen import device as gdev
    from quantized_expert_ffn_sigmoid_amd import capi

DEV = "cuda:0"


def _cfg(kind, H):
    if kind in ("i4", "i8"):
        # GLM-shaped decode layer with fewer experts: fp32 activations, a bf16
        # shared expert, sigmoid router over 4 groups
        return gen.shrink(gen.get_config("c2"), hidden=H, n_experts=16, top_k=4, n_group=4,
                          topk_group=2, seed=41)
    if kind == "bf16":
        # Granite-shaped: bf16 experts, softmax top-k, no shared expert
        return gen.shrink(gen.get_config("c1"), hidden=H, n_experts=8, top_k=2, seed=42)
    if kind == "i4_prefill":
        # bf16 activations (the grouped GEMM's input)
        return gen.shrink(gen.get_config("c3"), hidden=H, n_experts=16, top_k=4, n_group=4,
                          topk_group=2, bias="normal", seed=43)
    raise ValueError(kind)


def _x_dev(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(DEV)
    return torch.from_numpy(x).to(DEV)


DECODE_CASES = [("i4", 8192, 1), ("i4", 8192, 3), ("i4", 8192, 16), ("i8", 8192, 1),
                ("i8", 8192, 2), ("bf16", 7168, 1), ("bf16", 7168, 5), ("bf16", 8192, 1)]


@pytest.mark.parametrize("kind,H,T", DECODE_CASES)
def test_decode_wide_hidden(kind, H, T):
    print_case("wide decode", kind, H, T)
    cfg = _cfg(kind, H)
    dtype = gen.I8 if kind == "i8" else None
    if kind == "bf16":
        hl = gen.host_layer(cfg, 0, experts="all")
        layer = gdev.upload_host_layer(hl, DEV)
    else:
        layer = gdev.generate_device_layer(cfg, 0, DEV, dtype=dtype)
        hl = gen.host_layer(cfg, 0, dtype=dtype)
    x = gen.x_tokens(cfg, T, batch_id=700 + T)
    out, idx, w = capi.layer_forward(layer, _x_dev(x))
    torch.cuda.synchronize()
    ref, ridx, rw = oracle.layer_forward_host(hl, x)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.allclose(w.cpu().numpy(), rw, rtol=1e-6, atol=0)
    r = assert_close(out.cpu().numpy(), ref, cfg.act_dtype == gen.BF16,
                     f"wide decode {kind} H={H} T={T}")
    print(f"  max|err|/rms = {r:.3e}")


def test_int4_h7168_decode_unsupported_prefill_runs():
    cfg = _cfg("i4_prefill", 7168)
    layer = gdev.generate_device_layer(cfg, 0, DEV)
    x1 = gen.x_tokens(cfg, 1, batch_id=5)
    with pytest.raises(capi.MoeError) as e:
        capi.layer_forward(layer, _x_dev(x1))
    assert e.value.status == capi.MOE_EUNSUPPORTED
    # a prefill batch of the same layer: the grouped GEMM
    T = 40
    x = gen.x_tokens(cfg, T, batch_id=6)
    out, idx, w = capi.layer_forward(layer, _x_dev(x))
    torch.cuda.synchronize()
    hl = gen.host_layer(cfg, 0)
    ref, ridx, rw = oracle.layer_forward_host(hl, x)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.allclose(w.cpu().numpy(), rw, rtol=1e-6, atol=0)
    band = oracle.layer_band_host(hl, x, BF16_WINDOW)
    r, b = assert_close_band(out.cpu().numpy(), ref, band, "int4 H=7168 prefill T=40")
    print(f"  max|err|/rms = {r:.3e}, max band/rms = {b:.3e}")
