"""The kernels' error on the SwiGLU output h before its bf16 rounding.

With bf16 activations both sides round h to bf16, each from its own
accumulation (the oracle in fp64, the kernels in fp32), so an h lying within
the kernels' error of a rounding midpoint may round either way; the parity
tests of such layers allow those alternatives through the oracle's band,
whose window (tests/gpu_common.BF16_WINDOW) must cover the kernels'
error.  These tests measure that error: the layer's test hook returns h in
fp32 before rounding, compared here with the oracle's fp64 h of the same
(token, expert), on the grouped-GEMM path (int4 and bf16 weights, the
GLM-scale prefill at full width on sampled rows) and on the GEMV path.

The error is measured in units of u * e, u = 2^-24 the fp32 unit roundoff
and e the first-order scale of the error that rounding the terms of g and u
makes in h (oracle.expert_h), the unit the band's window is given in: an h
much smaller than the terms of its sums carries a large relative error, but
not a large error in these units.  The window must be at least twice the
largest error measured.
"""
import numpy as np
import pytest

import gen
import oracle
from tests.gpu_common import BF16_KAPPA, print_case

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gen import device as gdev
    from quantized_expert_ffn_sigmoid_amd import capi

DEV = "cuda:0"
U = 2.0 ** -24


def _run_with_probe(layer, xd):
    desc = capi.make_desc(layer.desc_spec)
    T = xd.shape[0]
    K, I, Is = desc.top_k, desc.inter, desc.inter * max(desc.n_shared, 1)
    nb = capi.moe_workspace_bytes(desc, T)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    out = torch.empty((T, desc.hidden), dtype=torch.float32, device=DEV)
    idx = torch.empty((T, K), dtype=torch.int32, device=DEV)
    w = torch.empty((T, K), dtype=torch.float32, device=DEV)
    hp = torch.full((T * K * I + T * Is,), float("nan"), dtype=torch.float32, device=DEV)
    capi.moe_layer_forward_ex(desc, capi.make_weights(layer.pointers()), xd, T, out, idx, w, ws,
                              nb, h_f32=hp)
    torch.cuda.synchronize()
    hp = hp.cpu().numpy()
    return idx.cpu().numpy(), hp[:T * K * I].reshape(T * K, I), hp[T * K * I:].reshape(T, Is)


def _kappa(got, ref, scale):
    """The largest |got - ref| in units of u * e (e > 0 wherever h != 0)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.asarray(scale, np.float64)
    assert np.isfinite(got).all()
    err = np.abs(got - ref)
    assert (err[scale == 0] == 0).all()
    live = scale > 0
    return float((err[live] / (U * scale[live])).max())


def _measure(hl, layer, x, xd, n_pos=None, n_tok_shared=None, seed=0):
    cfg = hl.cfg
    d = oracle.Desc.from_config(cfg, expert_dtype=hl.dtype)
    idx, hr, hs = _run_with_probe(layer, xd)
    T, K = idx.shape
    b = oracle.bucket(idx, cfg.n_experts)
    nvalid = int(b["offsets"][-1])
    rng = np.random.default_rng(seed)
    pos = np.arange(nvalid) if n_pos is None or n_pos >= nvalid else \
        np.sort(rng.choice(nvalid, n_pos, replace=False))
    got, ref, sc = [], [], []
    for p in pos:
        f = int(b["entries"][p])
        t, e = f // K, int(idx[f // K, f % K])
        es = oracle.ExpertSet(hl.get(e)["dtype"], [hl.get(i) if i == e else None
                                                   for i in range(cfg.n_experts)])
        h, sce = oracle.expert_h(d, es, e, x, rows=np.array([t], np.int32), with_scale=True)
        ref.append(h[0])
        sc.append(sce[0])
        got.append(hr[p])
    routed = _kappa(got, ref, sc)
    shared = None
    if cfg.n_shared:
        toks = np.arange(T) if n_tok_shared is None or n_tok_shared >= T else \
            np.sort(rng.choice(T, n_tok_shared, replace=False))
        ss = oracle.ExpertSet(hl.shared["dtype"], [hl.shared])
        ref_s, sc_s = oracle.expert_h(d, ss, 0, x, rows=toks.astype(np.int32),
                                      inter=cfg.inter * cfg.n_shared, with_scale=True)
        shared = _kappa(hs[toks], ref_s, sc_s)
    return routed, shared


def _report(what, routed, shared):
    print(f"  {what}: max h error in units of 2^-24 e: routed {routed:.3f}"
          + (f", shared {shared:.3f}" if shared is not None else "")
          + f"; window {BF16_KAPPA:g}")
    assert routed <= BF16_KAPPA / 2, (routed, BF16_KAPPA)
    if shared is not None:
        assert shared <= BF16_KAPPA / 2, (shared, BF16_KAPPA)


@pytest.mark.parametrize("kind,T", [("i4", 300), ("i4_wide", 150), ("bf16", 129)])
def test_h_error_grouped_gemm_small(kind, T):
    base = gen.get_config("c3")
    if kind == "bf16":
        cfg = gen.shrink(base, hidden=256, inter=128, n_experts=8, top_k=2, n_group=2,
                         topk_group=1, expert_dtype=gen.BF16, shared_dtype=gen.BF16,
                         bias="normal", seed=52)
    else:
        H, I = (2048, 1024) if kind == "i4_wide" else (512, 256)
        cfg = gen.shrink(base, hidden=H, inter=I, n_experts=16, top_k=4, n_group=4,
                         topk_group=2, bias="normal", seed=51)
    print_case("h error, grouped gemm", kind, T)
    hl = gen.host_layer(cfg, 0, experts="all")
    layer = gdev.upload_host_layer(hl, DEV)
    x = gen.x_tokens(cfg, T, batch_id=600 + T)
    xd = torch.from_numpy(x.view(np.int16)).to(DEV)
    _report(kind, *_measure(hl, layer, x, xd, n_pos=400, n_tok_shared=64))


def test_h_error_glm_prefill_full_width():
    """GLM-scale prefill (H 6144, I 2048, 2048 tokens, Zipf routing): sampled
    bucket rows of the routed experts and sampled tokens of the shared one."""
    cfg = gen.get_config("c3")
    print_case("h error, GLM prefill, 2048 tokens")
    layer = gdev.generate_device_layer(cfg, 0, DEV)
    hl = gen.host_layer(cfg, 0)
    x = gen.x_tokens(cfg, 2048, batch_id=0)
    xd = torch.from_numpy(x.view(np.int16)).to(DEV)
    _report("c3", *_measure(hl, layer, x, xd, n_pos=48, n_tok_shared=8, seed=3))


def test_h_error_gemv_decode_bf16_activations():
    """Decode-sized batches with bf16 activations run the GEMV kernels (int4
    routed experts on the LDS ring, bf16 shared expert)."""
    cfg = gen.get_config("c3")
    print_case("h error, GEMV, 16 tokens")
    layer = gdev.generate_device_layer(cfg, 0, DEV)
    hl = gen.host_layer(cfg, 0)
    x = gen.x_tokens(cfg, 16, batch_id=5)
    xd = torch.from_numpy(x.view(np.int16)).to(DEV)
    _report("gemv", *_measure(hl, layer, x, xd, n_pos=48, n_tok_shared=4, seed=4))
