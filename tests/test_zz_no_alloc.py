"""GPU test of moe_layer_forward_noalloc, the entry point that runs the layer
on the library's own per-GPU workspace (for callers that cannot allocate).

It must give the same bits as moe_layer_forward with a caller workspace, on
two calls in a row of which the second is smaller (so the second runs on a
workspace holding the first call's data), on the decode path (GEMV kernels,
GLM-scale layer) and on the grouped-GEMM path (bf16 activations, more tokens
than a decode batch); batches whose workspace exceeds the library's array
are rejected before anything is launched.
"""
import numpy as np
import pytest

import gen
from tests.gpu_common import print_case

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gen import device as gdev
    from quantized_expert_ffn_sigmoid_amd import capi

DEV = "cuda:0"


def _reference(layer, x):
    """moe_layer_forward on a caller workspace filled with garbage first."""
    desc = capi.make_desc(layer.desc_spec)
    T = x.shape[0]
    ws = torch.full((capi.moe_workspace_bytes(desc, T),), 0xFF, dtype=torch.uint8, device=DEV)
    out = torch.empty((T, desc.hidden), dtype=torch.float32, device=DEV)
    idx = torch.empty((T, desc.top_k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, desc.top_k), dtype=torch.float32, device=DEV)
    capi.moe_layer_forward(desc, capi.make_weights(layer.pointers()), x, T, out, idx, w, ws,
                           ws.numel())
    return out, idx, w


def _noalloc(layer, x):
    desc = capi.make_desc(layer.desc_spec)
    T = x.shape[0]
    out = torch.full((T, desc.hidden), float("nan"), dtype=torch.float32, device=DEV)
    idx = torch.full((T, desc.top_k), -7, dtype=torch.int32, device=DEV)
    w = torch.full((T, desc.top_k), float("nan"), dtype=torch.float32, device=DEV)
    capi.moe_layer_forward_noalloc(desc, capi.make_weights(layer.pointers()), x, T, out, idx, w)
    return out, idx, w


def _two_calls(layer, xs):
    for x in xs:
        print_case("noalloc", layer.cfg.name, "T =", x.shape[0])
        a = _noalloc(layer, x)
        b = _reference(layer, x)
        torch.cuda.synchronize()
        for got, want, what in zip(a, b, ("out", "topk_idx", "topk_w")):
            assert torch.equal(got, want), f"{what} differs at T={x.shape[0]}"


def test_noalloc_decode_glm_layer():
    cfg = gen.get_config("c2")
    layer = gdev.generate_device_layer(cfg, 0, DEV)
    xs = [torch.from_numpy(gen.x_tokens(cfg, T, batch_id=900 + T)).to(DEV) for T in (16, 1)]
    _two_calls(layer, xs)


def test_noalloc_grouped_gemm():
    cfg = gen.shrink(gen.get_config("c3"), hidden=512, inter=256, n_experts=16, top_k=4,
                     n_group=4, topk_group=2, bias="normal", seed=41, batches=(64,))
    layer = gdev.generate_device_layer(cfg, 0, DEV)
    xs = [torch.from_numpy(gen.x_tokens(cfg, T, batch_id=910 + T).view(np.int16)).to(DEV)
          for T in (300, 40)]
    _two_calls(layer, xs)


def test_noalloc_rejects_batches_beyond_its_workspace():
    cfg = gen.get_config("c2")
    layer = gdev.generate_device_layer(cfg, 0, DEV)
    desc = capi.make_desc(layer.desc_spec)
    T = 64
    assert capi.moe_workspace_bytes(desc, T) > capi.MOE_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, desc.hidden), dtype=torch.float32, device=DEV)
    out = torch.empty((T, desc.hidden), dtype=torch.float32, device=DEV)
    with pytest.raises(capi.MoeError) as e:
        capi.moe_layer_forward_noalloc(desc, capi.make_weights(layer.pointers()), x, T, out,
                                       None, None)
    assert e.value.status == capi.MOE_EWORKSPACE
