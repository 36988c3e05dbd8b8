"""GPU parity of the whole routed layer and of stacked layers.

Every case compares the HIP path (through the C ABI) with the oracle on the
same seeded inputs: router indices bit-exact, outputs within the tolerances
of tests/gpu_common.py.  Large configurations compare every routing decision
and a sample of tokens the oracle evaluates one by one.
"""
import numpy as np
import pytest

import gen
import oracle
from tests.gpu_common import BF16_WINDOW, assert_close, assert_close_band, oracle_eps, print_case

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gen import device as gdev
    from quantized_expert_ffn_sigmoid_amd import capi

DEV = "cuda:0"


def _x_dev(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(DEV)
    return torch.from_numpy(x).to(DEV)


def _layer_gpu(layer, x):
    out, idx, w = capi.layer_forward(layer, _x_dev(x))
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def _oracle_layer(cfg, layer_idx, x, dtype=None, tokens=None):
    hl = gen.host_layer(cfg, layer_idx, dtype=dtype)
    xs = x if tokens is None else np.ascontiguousarray(x[tokens])
    return oracle.layer_forward_host(hl, xs)


LAYER_CASES = [("c0", None, 1), ("c0", None, 3), ("c0", None, 7), ("c2", None, 1),
               ("c2", gen.I8, 1), ("c2", gen.I8, 5),
               ("c2", None, 16), ("c4", gen.I4, 2), ("c4", gen.I2, 4), ("c4", gen.I4, 16),
               ("c4", gen.I2, 16), ("c4", gen.I2, 1), ("c4", gen.I2, 2), ("c2", gen.I2, 3),
               ("c1", None, 1), ("c1", None, 16)]


@pytest.mark.parametrize("name,dtype,T", LAYER_CASES)
def test_layer_forward(name, dtype, T):
    print_case("layer", name, dtype, T)
    cfg = gen.get_config(name)
    if name in ("c0", "c1"):
        layer = gdev.upload_host_layer(gen.host_layer(cfg, 0, experts="all"), DEV)
    else:
        layer = gdev.generate_device_layer(cfg, 0, DEV, dtype=dtype)
    x = gen.x_tokens(cfg, T, batch_id=100 + T)
    out, idx, w = _layer_gpu(layer, x)
    ref, ridx, rw = _oracle_layer(cfg, 0, x, dtype)
    assert np.array_equal(idx, ridx)
    assert np.allclose(w, rw, rtol=1e-6, atol=0)
    r = assert_close(out, ref, cfg.act_dtype == gen.BF16, f"layer {name} {dtype} T={T}")
    print(f"  max|err|/rms = {r:.3e}")


def test_layer_zero_input_and_determinism():
    cfg = gen.get_config("c2")
    layer = gdev.generate_device_layer(cfg, 0, DEV)
    x0 = np.zeros((2, cfg.hidden), np.float32)
    out, idx, _ = _layer_gpu(layer, x0)
    assert (out == 0).all()
    x = gen.x_tokens(cfg, 4, batch_id=9)
    a, ia, wa = _layer_gpu(layer, x)
    b, ib, wb = _layer_gpu(layer, x)
    assert np.array_equal(a, b) and np.array_equal(ia, ib) and np.array_equal(wa, wb)


def _c3_sample(idx, n_experts, tile=64):
    """Tokens that cover the grouped GEMM's tiles: the first, middle and last
    rows of the first, middle and last (ragged) m-tiles of the 8 largest
    buckets, the first and last rows of buckets that fill one tile of at most
    16 or of 17-32 rows (the tiles that compute one or two 16-row subtiles),
    and the first and last tokens of the batch."""
    T, K = idx.shape
    b = oracle.bucket(idx, n_experts)
    counts, offsets, entries = b["counts"], b["offsets"], b["entries"]
    tok = lambda p: int(entries[p]) // K
    pick = {0, 1, T - 2, T - 1}
    for e in np.argsort(-counts, kind="stable")[:8]:
        n, p0 = int(counts[e]), int(offsets[e])
        nt = (n + tile - 1) // tile
        for m in sorted({0, nt // 2, nt - 1}):
            rows = min(tile, n - m * tile)
            for r in sorted({0, rows // 2, rows - 1}):
                pick.add(tok(p0 + m * tile + r))
    for lo, hi in ((1, 16), (17, 32)):
        small = [e for e in np.nonzero((counts >= lo) & (counts <= hi))[0]][:24]
        for e in small:
            pick.add(tok(int(offsets[e])))
            pick.add(tok(int(offsets[e + 1]) - 1))
    return np.array(sorted(pick))


def test_layer_c3_prefill_sampled():
    """GLM-scale batch-union prefill: 2048 bf16 tokens, Zipf-skewed routing.
    All 2048 x 8 routing decisions are compared; outputs on at least 128
    tokens chosen to cover every kind of grouped-GEMM tile."""
    cfg = gen.get_config("c3")
    print_case("c3 prefill", cfg.batches[0])
    layer = gdev.generate_device_layer(cfg, 0, DEV)
    T = cfg.batches[0]
    x = gen.x_tokens(cfg, T)
    out, idx, w = _layer_gpu(layer, x)
    hl = gen.host_layer(cfg, 0)
    ridx, rw, _ = oracle.route(oracle.Desc.from_config(cfg), hl.w_router, hl.bias, x, T)
    assert np.array_equal(idx, ridx)
    assert np.allclose(w, rw, rtol=1e-6, atol=0)
    sample = _c3_sample(ridx, cfg.n_experts)
    print(f"  {len(sample)} tokens compared")
    assert len(sample) >= 128
    ref, sidx, _ = oracle.layer_forward_host(hl, np.ascontiguousarray(x[sample]))
    assert np.array_equal(sidx, ridx[sample])
    band = oracle.layer_band_host(hl, np.ascontiguousarray(x[sample]), BF16_WINDOW)
    r, b = assert_close_band(out[sample], ref, band, "c3 sampled tokens")
    print(f"  max|err|/rms = {r:.3e}, max band/rms = {b:.3e}; "
          f"experts active = {len(np.unique(idx))}")


def _stack_gpu(layers, x, cfg):
    desc = capi.make_desc(layers[0].desc_spec)
    T = x.shape[0]
    arr = (capi.MoeLayerWeights * len(layers))(*[capi.make_weights(l.pointers()) for l in layers])
    xd = torch.from_numpy(x.copy()).to(DEV)
    ys = torch.empty((len(layers), T, cfg.hidden), dtype=torch.float32, device=DEV)
    nb = capi.moe_workspace_bytes(desc, T)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    capi.moe_stack_forward(desc, arr, len(layers), xd, T, ys, ws, nb)
    torch.cuda.synchronize()
    return xd.cpu().numpy(), ys.cpu().numpy()


def _teacher_forced(layers, cfg, xs_oracle, ys_oracle, host_layers):
    """Layer l on the GPU from the oracle's input x_l: RMSNorm then the layer."""
    T = xs_oracle[0].shape[0]
    for l, layer in enumerate(layers):
        xd = torch.from_numpy(xs_oracle[l]).to(DEV)
        xn = torch.empty_like(xd)
        capi.moe_rmsnorm(xd, T, cfg.hidden, np.float32(cfg.norm_eps), xn)
        out, idx, w = capi.layer_forward(layer, xn)
        torch.cuda.synchronize()
        xn_ref = oracle.rmsnorm(xs_oracle[l], oracle_eps(cfg))
        assert np.array_equal(xn.cpu().numpy(), xn_ref), f"rmsnorm layer {l}"
        ridx, _, _ = oracle.route(oracle.Desc.from_config(cfg, host_layers[l].dtype),
                                  host_layers[l].w_router, host_layers[l].bias, xn_ref, T)
        assert np.array_equal(idx.cpu().numpy(), ridx), f"routing layer {l}"
        assert_close(out.cpu().numpy(), ys_oracle[l], False, f"layer {l} (teacher-forced)")


def test_stack_c1_granite_24_layers():
    cfg = gen.get_config("c1")
    print_case("c1 stack", cfg.n_layers)
    hls = [gen.host_layer(cfg, l, experts="all") for l in range(cfg.n_layers)]
    layers = [gdev.upload_host_layer(h, DEV) for h in hls]
    x = gen.x_tokens(cfg, 1)
    xf, xs, ys = oracle.stack_forward_host(hls, x, oracle_eps(cfg))
    _teacher_forced(layers, cfg, xs, ys, hls)
    gx, gys = _stack_gpu(layers, x, cfg)
    for l in range(cfg.n_layers):
        assert_close(gys[l], ys[l], False, f"free-running layer {l}")
    assert_close(gx, xf, False, "final residual stream")


@pytest.mark.parametrize("dtype,T", [(gen.I4, 2), (gen.I2, 4)])
def test_stack_c4_8_layers(dtype, T):
    cfg = gen.get_config("c4")
    print_case("c4 stack", dtype, T)
    layers = [gdev.generate_device_layer(cfg, l, DEV, dtype=dtype) for l in range(cfg.n_layers)]
    hls = [gen.host_layer(cfg, l, dtype=dtype) for l in range(cfg.n_layers)]
    x = gen.x_tokens(cfg, T, batch_id=T)
    xf, xs, ys = oracle.stack_forward_host(hls, x, oracle_eps(cfg))
    _teacher_forced(layers, cfg, xs, ys, hls)
    gx, gys = _stack_gpu(layers, x, cfg)
    for l in range(cfg.n_layers):
        assert_close(gys[l], ys[l], False, f"free-running layer {l}")
    assert_close(gx, xf, False, "final residual stream")


def _widened(hl4):
    cfg = hl4.cfg
    hl8 = gen.HostLayer(cfg=cfg, layer=hl4.layer, w_router=hl4.w_router, bias=hl4.bias,
                        dtype=gen.I8)
    for e in range(cfg.n_experts):
        hl8.experts[e] = gen.expert_i8_from_i4(hl4.get(e), cfg.hidden, cfg.inter)
    hl8.shared = hl4.shared
    return hl8


@pytest.mark.parametrize("act", [gen.F32, gen.BF16])
def test_int8_container_of_int4_codes_bitwise(act):
    """int4 codes re-packed into the int8 container give bit-identical layer
    outputs on the GPU (the int8 kernels read each code as the operand the
    int4 kernels read and accumulate in the same order), at the GLM layer's
    widths (gate/up rows of 6144, down rows of 2048) on 16 experts."""
    cfg = gen.shrink(gen.get_config("c2"), n_experts=16, top_k=4, n_group=4, topk_group=2,
                     act_dtype=act, seed=44)
    hl4 = gen.host_layer(cfg, 0, experts="all")
    hl8 = _widened(hl4)
    l4 = gdev.upload_host_layer(hl4, DEV)
    l8 = gdev.upload_host_layer(hl8, DEV)
    for T in (1, 2, 5, 16):
        print_case("int8 vs int4 container", act, T)
        x = gen.x_tokens(cfg, T, batch_id=60 + T)
        o4, i4, w4 = _layer_gpu(l4, x)
        o8, i8, w8 = _layer_gpu(l8, x)
        assert np.array_equal(i4, i8) and np.array_equal(w4.view(np.uint32), w8.view(np.uint32))
        assert np.array_equal(o4.view(np.uint32), o8.view(np.uint32)), f"T={T}"


@pytest.mark.parametrize("T", [1, 4, 9])
def test_int8_small_layer(T):
    """The int8 container with full-range codes on a small layer whose shared
    expert is int8 too (K-slices of one granule: the register path)."""
    cfg = gen.shrink(gen.get_config("c0"), expert_dtype=gen.I8, shared_dtype=gen.I8,
                     hidden=128, inter=64, seed=45)
    hl = gen.host_layer(cfg, 0, experts="all")
    layer = gdev.upload_host_layer(hl, DEV)
    x = gen.x_tokens(cfg, T, batch_id=70 + T)
    print_case("int8 small layer", T)
    out, idx, w = _layer_gpu(layer, x)
    ref, ridx, rw = oracle.layer_forward_host(hl, x)
    assert np.array_equal(idx, ridx)
    r = assert_close(out, ref, False, f"int8 small T={T}")
    print(f"  max|err|/rms = {r:.3e}")


# Batches past the decode size on formats (or activations) the grouped GEMM
# does not take: the GEMV kernels in token mode, with the grouping's lookups
# (no per-slot records at these sizes).
GEMV_BEYOND_DECODE = [("c0", None, 40, None), ("c0", gen.I8, 33, None), ("c2", gen.I8, 24, [0, 7, 23])]


@pytest.mark.parametrize("name,dtype,T,sample", GEMV_BEYOND_DECODE)
def test_layer_gemv_beyond_decode(name, dtype, T, sample):
    cfg = gen.get_config(name)
    if name == "c0" and dtype == gen.I8:
        cfg = gen.shrink(cfg, expert_dtype=gen.I8, shared_dtype=gen.I8, hidden=128, inter=64,
                         seed=46)
    print_case("gemv beyond decode", name, dtype, T)
    if name == "c0":
        hl = gen.host_layer(cfg, 0, experts="all")
        layer = gdev.upload_host_layer(hl, DEV)
    else:
        layer = gdev.generate_device_layer(cfg, 0, DEV, dtype=dtype)
        hl = gen.host_layer(cfg, 0, dtype=dtype)
    x = gen.x_tokens(cfg, T, batch_id=300 + T)
    out, idx, w = _layer_gpu(layer, x)
    ridx, rw, _ = oracle.route(oracle.Desc.from_config(cfg, dtype), hl.w_router, hl.bias, x, T)
    assert np.array_equal(idx, ridx)
    assert np.allclose(w, rw, rtol=1e-6, atol=0)
    rows = np.arange(T) if sample is None else np.array(sample)
    ref, sidx, _ = oracle.layer_forward_host(hl, np.ascontiguousarray(x[rows]))
    assert np.array_equal(sidx, ridx[rows])
    r = assert_close(out[rows], ref, False, f"{name} T={T}")
    print(f"  max|err|/rms = {r:.3e}")


TOPP_LAYER_CASES = [("c2", 1, 0.7), ("c2", 4, 0.5), ("c4", 16, 0.6)]


@pytest.mark.parametrize("name,T,p", TOPP_LAYER_CASES)
def test_layer_top_p(name, T, p):
    """The layer with adaptive expert top-p against the oracle: routing
    bit-exact (dropped slots included), outputs within tolerance."""
    cfg = gen.get_config(name, top_p=p)
    print_case("layer top-p", name, T, p)
    layer = gdev.generate_device_layer(cfg, 0, DEV)
    x = gen.x_tokens(cfg, T, batch_id=300 + T)
    out, idx, w = _layer_gpu(layer, x)
    ref, ridx, rw = _oracle_layer(cfg, 0, x)
    assert np.array_equal(idx, ridx) and (idx < 0).any()
    assert np.allclose(w, rw, rtol=1e-6, atol=0)
    r = assert_close(out, ref, cfg.act_dtype == gen.BF16, f"layer top-p {name} T={T}")
    print(f"  max|err|/rms = {r:.3e}, experts kept {int((idx >= 0).sum())} of {idx.size}")


# Codes over each container's whole range (int4 [-8, 7], int2 [-2, 1], int8
# [-128, 127]) through every unpacking path: the GEMV's LDS ring (rows of at
# least 64 granules: H and I of 2048), its register path (rows of 16 and 8
# granules: H 512, I 256), the decode launches that carry the router
# (shared expert of the same format), and the grouped GEMM (bf16
# activations, more tokens than a decode batch).
FULL_CASES = [
    ("ring", gen.I4, 1), ("ring", gen.I4, 3), ("ring", gen.I2, 2), ("ring", gen.I8, 2),
    ("regs", gen.I4, 2), ("regs", gen.I2, 3), ("regs", gen.I8, 1),
    ("gemm", gen.I4, 150),
]


@pytest.mark.parametrize("path,dtype,T", FULL_CASES)
def test_layer_full_code_range(path, dtype, T):
    base = gen.get_config("c2")
    small = dict(n_experts=16, top_k=4, n_group=4, topk_group=2, bias="normal",
                 full_codes=True, seed=71, expert_dtype=dtype, shared_dtype=dtype)
    if path == "ring":
        cfg = gen.shrink(base, hidden=2048, inter=2048, **small)
    elif path == "regs":
        cfg = gen.shrink(base, hidden=512, inter=256, **small)
    else:
        cfg = gen.shrink(gen.get_config("c3"), hidden=512, inter=256, **small)
    print_case("full code range", path, dtype, T)
    hl = gen.host_layer(cfg, 0, experts="all")
    q = oracle.decode_codes(dtype, hl.get(0)["gate_up"], 2 * cfg.inter * cfg.hidden)
    assert q.min() == {gen.I4: -8, gen.I2: -2, gen.I8: -128}[dtype]
    layer = gdev.upload_host_layer(hl, DEV)
    x = gen.x_tokens(cfg, T, batch_id=700 + T)
    out, idx, w = _layer_gpu(layer, x)
    ref, ridx, rw = oracle.layer_forward_host(hl, x)
    assert np.array_equal(idx, ridx)
    assert np.allclose(w, rw, rtol=1e-6, atol=0)
    if cfg.act_dtype == gen.BF16:
        band = oracle.layer_band_host(hl, x, BF16_WINDOW)
        r, b = assert_close_band(out, ref, band, f"full codes {path} {dtype} T={T}")
        print(f"  max|err|/rms = {r:.3e}, max band/rms = {b:.3e}")
    else:
        r = assert_close(out, ref, False, f"full codes {path} {dtype} T={T}")
        print(f"  max|err|/rms = {r:.3e}")
