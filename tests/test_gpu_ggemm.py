"""GPU parity of the grouped-GEMM (matrix core) path of the layer.

Batches above the decode size with bf16 activations run the expert FFNs as a
grouped GEMM over 64-row bucket tiles.  These cases compare every output of
the layer with the oracle on small layers whose buckets span several tiles,
ragged last tiles and tiles of one row, for int4 and bf16 routed experts and
int4, bf16 or no shared expert, with n-tile counts from 1 to 8 and up to 583
active experts.  The GLM-scale prefill case lives in test_gpu_layer.py
(sampled tokens).
"""
import numpy as np
import pytest

import gen
import oracle
from tests.gpu_common import BF16_WINDOW, assert_close_band, print_case

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gen import device as gdev
    from quantized_expert_ffn_sigmoid_amd import capi

DEV = "cuda:0"


def _cfg(kind):
    base = gen.get_config("c3")
    small = dict(hidden=512, inter=256, n_experts=16, top_k=4, n_group=4, topk_group=2,
                 bias="normal", seed=31, batches=(64,))
    if kind == "i4_bf16shared":
        return gen.shrink(base, **small)
    if kind == "i4_i4shared":
        return gen.shrink(base, shared_dtype=gen.I4, **small)
    if kind == "i4_noshared":
        return gen.shrink(base, n_shared=0, **small)
    if kind == "i4_zipf":
        return gen.shrink(base, **dict(small, bias="zipf", seed=33))
    if kind == "i4_topp":
        return gen.shrink(base, **dict(small, top_p=0.6, seed=35))
    if kind == "i4_odd_k":
        # K steps of 128: 6 (gate/up) and 3 (down), an odd count
        return gen.shrink(base, **dict(small, hidden=768, inter=384, seed=34))
    if kind == "i4_xcd":
        # 8 gate/up and 8 down n-tiles, more m-tiles than XCDs
        return gen.shrink(base, **dict(small, hidden=2048, inter=1024, seed=36))
    if kind == "i4_xcd_i4shared":
        return gen.shrink(base, **dict(small, hidden=2048, inter=1024, shared_dtype=gen.I4,
                                       seed=37))
    if kind == "i4_many":
        # more active experts than one thread of the tile-list scan takes
        # (600 experts, 583 active)
        return gen.shrink(base, **dict(small, n_experts=600, top_k=8, seed=38))
    if kind == "bf16":
        return gen.shrink(base, hidden=256, inter=128, n_experts=8, top_k=2, n_group=2,
                          topk_group=1, expert_dtype=gen.BF16, shared_dtype=gen.BF16,
                          bias="normal", seed=32, batches=(40,))
    raise ValueError(kind)


CASES = [("i4_bf16shared", 17), ("i4_bf16shared", 100), ("i4_bf16shared", 300),
         ("i4_i4shared", 70), ("i4_noshared", 65), ("i4_zipf", 400), ("i4_odd_k", 50),
         ("i4_topp", 120), ("i4_xcd", 150), ("i4_xcd_i4shared", 90), ("i4_many", 300),
         ("bf16", 40), ("bf16", 129)]


@pytest.mark.parametrize("kind,T", CASES)
def test_grouped_gemm_layer(kind, T):
    cfg = _cfg(kind)
    print_case("grouped gemm layer", kind, T)
    hl = gen.host_layer(cfg, 0, experts="all")
    layer = gdev.upload_host_layer(hl, DEV)
    x = gen.x_tokens(cfg, T, batch_id=500 + T)
    xd = torch.from_numpy(x.view(np.int16)).to(DEV)
    out, idx, w = capi.layer_forward(layer, xd)
    torch.cuda.synchronize()
    ref, ridx, rw = oracle.layer_forward_host(hl, x)
    idx = idx.cpu().numpy()
    assert np.array_equal(idx, ridx)
    assert np.allclose(w.cpu().numpy(), rw, rtol=1e-6, atol=0)
    counts = np.bincount(idx[idx >= 0], minlength=cfg.n_experts)
    print(f"  bucket sizes: max {counts.max()}, min nonzero {counts[counts > 0].min()}")
    band = oracle.layer_band_host(hl, x, BF16_WINDOW)
    r, b = assert_close_band(out.cpu().numpy(), ref, band, f"grouped gemm {kind} T={T}")
    print(f"  max|err|/rms = {r:.3e}, max band/rms = {b:.3e}")


def test_grouped_gemm_deterministic():
    cfg = _cfg("i4_bf16shared")
    layer = gdev.generate_device_layer(cfg, 0, DEV)
    x = gen.x_tokens(cfg, 200, batch_id=7)
    xd = torch.from_numpy(x.view(np.int16)).to(DEV)
    a, ia, _ = capi.layer_forward(layer, xd)
    b, ib, _ = capi.layer_forward(layer, xd)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(ia, ib)
