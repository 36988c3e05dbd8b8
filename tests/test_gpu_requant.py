"""GPU parity of the FP8 -> int4 requantizer: codes and per-row scales
bit-exact against the oracle, on synthetic FP8 matrices (every byte value,
and normal weights rounded to E4M3) with ragged 128x128 blocks, at the GLM
expert shapes, and through the layer: experts requantized on the GPU give the
oracle's layer when the oracle reads its own requantization."""
import numpy as np
import pytest

import gen
import oracle
from tests.gpu_common import assert_close, print_case

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gen import device as gdev
    from quantized_expert_ffn_sigmoid_amd import capi

DEV = "cuda:0"


def _requant_gpu(b, bs, block=128):
    rows, cols = b.shape
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty(rows, dtype=torch.float32, device=DEV)
    capi.moe_requant_fp8_int4(torch.from_numpy(b).to(DEV), torch.from_numpy(bs).to(DEV), rows, cols,
                              block, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


CASES = [(1, 8, "bytes"), (200, 328, "bytes"), (129, 1024, "normal"), (4096, 6144, "normal"),
         (6144, 2048, "normal"), (64, 8192, "bytes")]


@pytest.mark.parametrize("rows,cols,kind", CASES)
def test_requant_bit_exact(rows, cols, kind):
    print_case("requant", rows, cols, kind)
    b, bs = gen.fp8_e4m3_matrix(seed=rows + cols, rows=rows, cols=cols, kind=kind)
    b[min(3, rows - 1)] = 0   # an all-zero row: scale 0, codes 0
    codes, scales = _requant_gpu(b, bs)
    rc, rs = oracle.requant_fp8_int4(b, bs)
    assert np.array_equal(scales.view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(codes, rc)


def test_requant_block_64_and_unsupported_shapes():
    b, bs = gen.fp8_e4m3_matrix(seed=9, rows=100, cols=200, block=64, kind="bytes")
    codes, scales = _requant_gpu(b, bs, block=64)
    rc, rs = oracle.requant_fp8_int4(b, bs, 64)
    assert np.array_equal(codes, rc) and np.array_equal(scales, rs)
    with pytest.raises(capi.MoeError):
        _requant_gpu(np.zeros((4, 12), np.uint8), np.ones((1, 1), np.float32))   # cols % 8


def test_requantized_experts_through_the_layer():
    """FP8 experts requantized on the GPU, then the layer: against the oracle
    layer over the oracle's requantization of the same FP8 (identical int4
    experts, so the usual layer tolerance)."""
    cfg = gen.shrink(gen.get_config("c2"), hidden=512, inter=256, n_experts=16, top_k=4,
                     n_group=4, topk_group=2, n_shared=0, seed=51)
    H, I = cfg.hidden, cfg.inter
    hl = gen.host_layer(cfg, 0)
    for e in range(cfg.n_experts):
        gu8, gubs = gen.fp8_e4m3_matrix(seed=1000 + e, rows=2 * I, cols=H)
        dn8, dnbs = gen.fp8_e4m3_matrix(seed=2000 + e, rows=H, cols=I)
        gc, gs = _requant_gpu(gu8, gubs)
        dc, ds = _requant_gpu(dn8, dnbs)
        ogc, ogs = oracle.requant_fp8_int4(gu8, gubs)
        odc, ods = oracle.requant_fp8_int4(dn8, dnbs)
        assert np.array_equal(gc, ogc) and np.array_equal(dc, odc)
        hl.experts[e] = dict(dtype=gen.I4, gate_up=gc, gate_up_scale=gs, down=dc, down_scale=ds)
    layer = gdev.upload_host_layer(hl, DEV)
    x = gen.x_tokens(cfg, 5, batch_id=8)
    out, idx, w = capi.layer_forward(layer, torch.from_numpy(x).to(DEV))
    torch.cuda.synchronize()
    ref, ridx, _ = oracle.layer_forward_host(hl, x)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    r = assert_close(out.cpu().numpy(), ref, False, "requantized layer")
    print(f"  max|err|/rms = {r:.3e}")
