"""GPU parity of the individual C ABI calls against the oracle.

Bit-exact: dequantized weights, router indices, buckets, and the device twin
of the input generator.  Within tolerance: router weights, expert outputs.
"""
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


@pytest.fixture(scope="module")
def c2_layer():
    cfg = gen.get_config("c2")
    return cfg, gdev.generate_device_layer(cfg, 0, DEV)


@pytest.fixture(scope="module")
def c2_layers_i4_i2():
    cfg = gen.get_config("c4")
    return cfg, gdev.generate_device_layer(cfg, 0, DEV, also_int2=True)


def _blob_host(t, e):
    return t[e].cpu().numpy()


def test_device_twin_is_bit_identical(c2_layers_i4_i2):
    cfg, (l4, l2) = c2_layers_i4_i2
    torch.cuda.synchronize()
    for e in (0, 131, 255):
        print_case("twin", e)
        b4, lay4 = _blob_host(l4.routed, e), l4.routed_layout
        ex = gen.expert(cfg, 0, e, gen.I4)
        for key in ("gate_up", "down", "gate_up_scale", "down_scale"):
            a = np.ascontiguousarray(ex[key]).view(np.uint8).ravel()
            off = lay4[key]
            assert np.array_equal(b4[off:off + a.size], a), (e, key)
        b2, lay2 = _blob_host(l2.routed, e), l2.routed_layout
        ex2 = gen.expert(cfg, 0, e, gen.I2)
        for key in ("gate_up", "down", "gate_up_scale", "down_scale"):
            a = np.ascontiguousarray(ex2[key]).view(np.uint8).ravel()
            off = lay2[key]
            assert np.array_equal(b2[off:off + a.size], a), (e, "int2", key)


@pytest.mark.parametrize("dtype", [gen.I4, gen.I2, gen.I8, gen.BF16])
def test_dequant_bit_exact(dtype):
    cfg = gen.shrink(gen.get_config("c2"), hidden=512, inter=256)
    ex = gen.expert(cfg, 0, 5, dtype)
    cols = cfg.hidden
    codes = torch.from_numpy(np.ascontiguousarray(ex["gate_up"])).to(DEV)
    scales = None if dtype == gen.BF16 else torch.from_numpy(ex["gate_up_scale"]).to(DEV)
    for row0, n in ((0, 7), (100, 156), (511, 1)):
        print_case("dequant", dtype, row0, n)
        out = torch.empty((n, cols), dtype=torch.float32, device=DEV)
        ob = None if dtype == gen.BF16 else torch.empty((n, cols), dtype=torch.int16, device=DEV)
        capi.moe_dequant_rows(dtype, codes, scales, cols, row0, n, out, ob)
        ref = oracle.dequant_rows(dtype, ex["gate_up"], ex["gate_up_scale"], cols, row0, n)
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))
        if ob is not None:
            q = oracle.decode_codes(dtype, ex["gate_up"][row0:row0 + n], n * cols)
            want = gen.f32_to_bf16_bits(q.astype(np.float32)).view(np.int16)
            assert np.array_equal(ob.cpu().numpy().ravel(), want)


@pytest.mark.parametrize("dtype", [gen.I4, gen.I2, gen.I8])
def test_dequant_every_code(dtype):
    """Every byte value through the kernels' unpacking: rows of 256 bytes
    holding 0..255 (int4: every pair of codes in [-8, 7]; int2: every four
    codes in [-2, 1]; int8: every code in [-128, 127]), each byte in every
    position of its dword across the rows, under scales of several binades
    and a zero scale."""
    per = {gen.I4: 2, gen.I2: 4, gen.I8: 1}[dtype]
    cols = 256 * per
    rows = 8
    codes = np.stack([np.roll(np.arange(256, dtype=np.uint8), r) for r in range(rows)])
    scales = np.array([1.0, 0.0137, 3.5e-3, 2.0 ** -20, 7.25, 0.0, 1e-30, 1.3e5], np.float32)
    cd = torch.from_numpy(codes).to(DEV)
    sd = torch.from_numpy(scales).to(DEV)
    print_case("dequant every code", dtype)
    out = torch.empty((rows, cols), dtype=torch.float32, device=DEV)
    ob = torch.empty((rows, cols), dtype=torch.int16, device=DEV)
    capi.moe_dequant_rows(dtype, cd, sd, cols, 0, rows, out, ob)
    ref = oracle.dequant_rows(dtype, codes, scales, cols, 0, rows)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    q = oracle.decode_codes(dtype, codes, rows * cols)
    lo, hi = {gen.I4: (-8, 7), gen.I2: (-2, 1), gen.I8: (-128, 127)}[dtype]
    assert q.min() == lo and q.max() == hi and len(np.unique(q)) == hi - lo + 1
    want = gen.f32_to_bf16_bits(q.astype(np.float32)).view(np.int16)
    assert np.array_equal(ob.cpu().numpy().ravel(), want)


def _desc(cfg, dtype=None):
    spec = type("S", (), {})()
    for k in ("hidden", "inter", "n_experts", "top_k", "router", "n_group", "topk_group",
              "routed_scaling", "act_dtype", "n_shared", "shared_dtype", "top_p"):
        setattr(spec, k, getattr(cfg, k))
    spec.expert_dtype = cfg.expert_dtype if dtype is None else dtype
    spec.norm_eps = cfg.norm_eps or 0.0
    return capi.make_desc(spec)


def _x_dev(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(DEV)
    return torch.from_numpy(x).to(DEV)


def route_on_gpu(cfg, w_r, bias, x):
    d = _desc(cfg)
    T = x.shape[0]
    idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, cfg.top_k), dtype=torch.float32, device=DEV)
    nb = capi.moe_workspace_bytes(d, T)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    capi.moe_route(d, torch.from_numpy(w_r).to(DEV),
                   None if bias is None else torch.from_numpy(bias).to(DEV), _x_dev(x), T, idx, w,
                   ws, nb)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy()


ROUTE_CASES = [("c0", 1), ("c0", 5), ("c2", 1), ("c2", 16), ("c2", 77), ("c1", 1), ("c1", 16),
               ("c1", 40), ("c3", 2048)]


@pytest.mark.parametrize("name,T", ROUTE_CASES)
def test_route_bit_exact(name, T):
    cfg = gen.get_config(name)
    print_case("route", name, T)
    w_r, bias = gen.router(cfg)
    x = gen.x_tokens(cfg, T, batch_id=T)
    idx, w = route_on_gpu(cfg, w_r, bias, x)
    ridx, rw, _ = oracle.route(oracle.Desc.from_config(cfg), w_r, bias, x, T)
    assert np.array_equal(idx, ridx)
    assert np.allclose(w, rw, rtol=1e-6, atol=0)


TOPP_ROUTE_CASES = [("c2", 1, 0.7), ("c2", 16, 0.5), ("c2", 77, 0.9), ("c1", 16, 0.6),
                    ("c3", 2048, 0.7), ("c0", 5, 0.3)]


@pytest.mark.parametrize("name,T,p", TOPP_ROUTE_CASES)
def test_route_top_p_bit_exact(name, T, p):
    """Adaptive expert top-p: the kept prefix (indices, -1 for dropped slots)
    bit-exact, the renormalized weights to the float rounding of the oracle's."""
    cfg = gen.get_config(name, top_p=p)
    print_case("route top-p", name, T, p)
    w_r, bias = gen.router(cfg)
    x = gen.x_tokens(cfg, T, batch_id=T + 5)
    idx, w = route_on_gpu(cfg, w_r, bias, x)
    ridx, rw, _ = oracle.route(oracle.Desc.from_config(cfg), w_r, bias, x, T)
    assert (ridx < 0).any() or p >= 0.9
    assert np.array_equal(idx, ridx)
    assert np.allclose(w, rw, rtol=1e-6, atol=0)
    assert (w[idx < 0] == 0).all()


@pytest.mark.parametrize("name", ["c0", "c2", "c1"])
def test_route_exact_ties(name):
    cfg = gen.get_config(name)
    w_r, _ = gen.router(cfg)
    x = np.zeros((3, cfg.hidden), np.float32)
    bias = np.zeros(cfg.n_experts, np.float32) if cfg.bias else None
    idx, w = route_on_gpu(cfg, w_r, bias, x)
    assert (idx == np.arange(cfg.top_k)).all()
    assert (w == np.float32(cfg.routed_scaling / cfg.top_k)).all()
    # duplicated router rows with equal bias: the lower index wins
    if cfg.bias:
        w2 = w_r.copy()
        w2[cfg.n_experts - 1] = w2[0]
        xr = gen.x_tokens(cfg, 8, batch_id=3)
        idx, _ = route_on_gpu(cfg, w2, np.zeros(cfg.n_experts, np.float32), xr)
        ridx, _, _ = oracle.route(oracle.Desc.from_config(cfg), w2,
                                  np.zeros(cfg.n_experts, np.float32), xr, 8)
        assert np.array_equal(idx, ridx)


# (5000, 8, 256): 40000 slots, more than one chunk of the 1024-thread block's
# read-ahead (16 slots per thread) and a ragged last round
BUCKET_CASES = [(1, 8, 256), (16, 8, 256), (2048, 8, 256), (7, 2, 8), (33, 5, 1000), (0, 8, 256),
                (1, 1, 1), (300, 4, 3), (5000, 8, 256)]
# slots dropped by adaptive top-p (index -1): small and large slot counts
BUCKET_DROP_CASES = [(1, 8, 256), (16, 8, 256), (2048, 8, 256), (33, 5, 1000), (3000, 8, 256)]


@pytest.mark.parametrize("T,K,E", BUCKET_DROP_CASES)
def test_bucket_dropped_slots_bit_exact(T, K, E):
    print_case("bucket dropped", T, K, E)
    rng = np.random.default_rng(T * 7 + K)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    keep = rng.integers(1, K + 1, size=T)   # a kept prefix per token
    idx[np.arange(K)[None, :] >= keep[:, None]] = -1
    ref = oracle.bucket(idx, E)
    F = T * K
    n = int(ref["offsets"][-1])
    dev = lambda m: torch.full((max(m, 1),), -7, dtype=torch.int32, device=DEV)
    counts, offsets, entries, inverse, active, na = dev(E), dev(E + 1), dev(F), dev(F), dev(E), dev(1)
    capi.moe_bucket(T, K, E, torch.from_numpy(idx.ravel().copy()).to(DEV), counts, offsets,
                    entries, inverse, active, na)
    torch.cuda.synchronize()
    assert np.array_equal(counts.cpu().numpy(), ref["counts"])
    assert np.array_equal(offsets.cpu().numpy(), ref["offsets"])
    assert int(na.cpu().item()) == ref["n_active"]
    assert np.array_equal(active.cpu().numpy()[:ref["n_active"]], ref["active"])
    assert np.array_equal(entries.cpu().numpy()[:n], ref["entries"][:n])
    assert np.array_equal(inverse.cpu().numpy(), ref["inverse"])


@pytest.mark.parametrize("T,K,E", BUCKET_CASES)
def test_bucket_bit_exact(T, K, E):
    print_case("bucket", T, K, E)
    rng = np.random.default_rng(T * 31 + K)
    if T == 0:
        idx = np.zeros((0, K), np.int32)
    elif K <= E:
        idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32).reshape(T, K)
    else:
        idx = rng.integers(0, E, size=(T, K)).astype(np.int32)
    if T == 300:   # heavy skew: most slots on one expert
        idx[:] = np.where(rng.random((T, K)) < 0.9, 1, idx)
    ref = oracle.bucket(idx, E)
    F = T * K
    dev = lambda n: torch.full((max(n, 1),), -7, dtype=torch.int32, device=DEV)
    counts, offsets, entries, inverse, active, na = dev(E), dev(E + 1), dev(F), dev(F), dev(E), dev(1)
    capi.moe_bucket(T, K, E, torch.from_numpy(idx.ravel().copy()).to(DEV) if F else None, counts,
                    offsets, entries, inverse, active, na)
    torch.cuda.synchronize()
    assert np.array_equal(counts.cpu().numpy(), ref["counts"])
    assert np.array_equal(offsets.cpu().numpy(), ref["offsets"])
    assert int(na.cpu().item()) == ref["n_active"]
    assert np.array_equal(active.cpu().numpy()[:ref["n_active"]], ref["active"])
    if F:
        assert np.array_equal(entries.cpu().numpy(), ref["entries"])
        assert np.array_equal(inverse.cpu().numpy(), ref["inverse"])


def _ffn_gpu(cfg, layer, shared, e, x, rows, n_rows, row_div):
    d = _desc(cfg, layer.expert_dtype)
    eset = capi.make_set(layer.pointers()["shared" if shared else "routed"])
    y = torch.empty((n_rows, cfg.hidden), dtype=torch.float32, device=DEV)
    nb = capi.moe_workspace_bytes(d, n_rows)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    capi.moe_expert_ffn(d, eset, 1 if shared else 0, e, _x_dev(x),
                        None if rows is None else torch.from_numpy(rows).to(DEV), n_rows, row_div,
                        y, ws, nb)
    torch.cuda.synchronize()
    return y.cpu().numpy()


FFN_CASES = [
    # (config, expert dtype, shared?, expert, n_tokens, row list?)
    ("c0", gen.I4, False, 3, 3, False),
    ("c0", gen.I4, True, 0, 4, False),
    ("c2", gen.I4, False, 17, 1, False),
    ("c2", gen.I4, False, 200, 5, True),
    ("c2", gen.I4, True, 0, 2, False),
    ("c4", gen.I2, False, 9, 4, True),
    ("c4", gen.I2, False, 70, 1, False),
    ("c2", gen.I2, False, 5, 2, False),
    ("c0", gen.I8, False, 5, 3, False),
    ("c2", gen.I8, False, 33, 1, False),
    ("c2", gen.I8, False, 150, 6, True),
    ("c1", gen.BF16, False, 5, 3, False),
    ("c3", gen.I4, False, 42, 37, True),
    ("c3", gen.I4, True, 0, 19, False),
]


@pytest.mark.parametrize("case", FFN_CASES, ids=lambda c: "-".join(map(str, c)))
def test_expert_ffn(case):
    name, dtype, shared, e, n, use_rows = case
    print_case("ffn", *case)
    cfg = gen.get_config(name)
    if name in ("c0", "c1"):
        hl = gen.host_layer(cfg, 0, experts="all", dtype=dtype)
        layer = gdev.upload_host_layer(hl, DEV)
    else:
        layer = gdev.generate_device_layer(cfg, 0, DEV, dtype=dtype)
    x = gen.x_tokens(cfg, max(n, 1) * 2, batch_id=7)
    rows = None
    row_div = 1
    if use_rows:   # ragged row list of slots, token = slot // 8
        rows = (np.random.default_rng(e).permutation(x.shape[0])[:n] * 8 + 3).astype(np.int32)
        row_div = 8
    y = _ffn_gpu(cfg, layer, shared, e, x, rows, n, row_div)
    d = oracle.Desc.from_config(cfg, expert_dtype=dtype)
    if shared:
        es = oracle.ExpertSet(cfg.shared_dtype, [gen.expert(cfg, 0, 0, shared=True)])
        ref = oracle.expert_ffn(d, es, 0, x, rows=rows, n_rows=n, row_div=row_div,
                                inter=cfg.inter * cfg.n_shared)
    else:
        exs = [None] * cfg.n_experts
        exs[e] = gen.expert(cfg, 0, e, dtype)
        ref = oracle.expert_ffn(d, oracle.ExpertSet(dtype, exs), e, x, rows=rows, n_rows=n,
                                row_div=row_div)
    r = assert_close(y, ref, cfg.act_dtype == gen.BF16, f"ffn {case}")
    print(f"  max|err|/rms = {r:.3e}")
