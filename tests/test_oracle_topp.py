"""Pins of the oracle's adaptive expert top-p (CPU only).

The rule (the knob of the "colibri" README, "Quick start"; our reading): of
the top_k chosen experts in rank order, keep the shortest prefix whose share
of the routing mass reaches top_p (at least one), renormalize the kept
weights, and mark dropped slots with index -1 and weight 0.  These tests fix
it by a worked example with exact masses, reductions to the plain router,
and properties any correct implementation has: a prefix of the plain choice,
minimal and sufficient mass, weights proportional to the plain ones and
summing to the scaling, more experts for larger top_p.
"""
import math

import numpy as np
import pytest

import gen
import oracle


def _desc(E, k, G=1, g=1, scaling=1.0, router=oracle.SIGMOID_NOAUX_TC, top_p=0.0):
    return oracle.Desc(hidden=8, inter=8, n_experts=E, top_k=k, router=router, n_group=G,
                       topk_group=g, routed_scaling=scaling, top_p=top_p)


def test_worked_example_softmax():
    """Softmax masses 5 : 3 : 2 (logits ln 5, ln 3, ln 2): shares 0.5, 0.3, 0.2."""
    z = np.array([[math.log(2.0), math.log(5.0), -3.0, math.log(3.0)]])
    for p, keep in ((0.3, 1), (0.5, 1), (0.7, 2), (0.79, 2), (0.81, 3), (0.99, 3)):
        d = _desc(4, 3, router=oracle.SOFTMAX_TOPK, top_p=p)
        idx, w, w64 = oracle.select(d, z, None, 1)
        assert idx[0].tolist() == [1, 3, 0][:keep] + [-1] * (3 - keep), (p, idx)
        masses = np.array([5.0, 3.0, 2.0])[:keep]
        np.testing.assert_allclose(w64[0, :keep], masses / masses.sum(), rtol=1e-15)
        assert (w64[0, keep:] == 0).all() and (w[0, keep:] == 0).all()


@pytest.mark.parametrize("p", [0.0, 1.0, 1.5])
def test_off_values_give_the_plain_router(p):
    rng = np.random.default_rng(1)
    z = rng.normal(size=(20, 32))
    bias = (0.1 * rng.normal(size=32)).astype(np.float32)
    plain = oracle.select(_desc(32, 6, 4, 2, 2.5), z, bias, 20)
    got = oracle.select(_desc(32, 6, 4, 2, 2.5, top_p=p), z, bias, 20)
    for a, b in zip(plain, got):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("router", [oracle.SIGMOID_NOAUX_TC, oracle.SOFTMAX_TOPK])
def test_prefix_minimal_sufficient_and_renormalized(router):
    rng = np.random.default_rng(2)
    T, E, k, scaling = 200, 64, 8, 2.5
    z = rng.normal(scale=2.0, size=(T, E))
    bias = None if router == oracle.SOFTMAX_TOPK else (0.05 * rng.normal(size=E)).astype(np.float32)
    G, g = (8, 4) if router == oracle.SIGMOID_NOAUX_TC else (1, 1)
    pi, _, pw = oracle.select(_desc(E, k, G, g, scaling, router), z, bias, T)
    for p in (0.2, 0.5, 0.7, 0.9):
        idx, w, w64 = oracle.select(_desc(E, k, G, g, scaling, router, top_p=p), z, bias, T)
        for t in range(T):
            m = int((idx[t] >= 0).sum())
            assert m >= 1
            assert np.array_equal(idx[t, :m], pi[t, :m]) and (idx[t, m:] == -1).all()
            share = np.cumsum(pw[t]) / pw[t].sum()
            before = 0.0 if m == 1 else share[m - 2]
            if abs(before - p) > 1e-9 and abs(share[m - 1] - p) > 1e-9:
                assert before < p <= share[m - 1] or m == 1 and share[0] >= p
            np.testing.assert_allclose(w64[t, :m].sum(), scaling, rtol=1e-13)
            ratio = w64[t, :m] / pw[t, :m]
            np.testing.assert_allclose(ratio, ratio[0], rtol=1e-13)
            assert (w64[t, m:] == 0).all()


def test_more_mass_keeps_more_experts():
    rng = np.random.default_rng(3)
    z = rng.normal(size=(50, 32))
    prev = None
    for p in np.linspace(0.05, 0.95, 19):
        idx, _, _ = oracle.select(_desc(32, 8, 4, 2, 1.0, top_p=float(p)), z, None, 50)
        kept = (idx >= 0).sum(axis=1)
        if prev is not None:
            assert (kept >= prev).all()
        prev = kept


def test_bucket_skips_dropped_slots():
    idx = np.array([[3, 1, -1], [1, -1, -1], [0, 3, 2]], np.int32)
    b = oracle.bucket(idx, 4)
    flat = idx.ravel()
    valid = np.flatnonzero(flat >= 0)
    order = valid[np.argsort(flat[valid], kind="stable")]
    n = len(valid)
    assert b["offsets"][-1] == n
    assert np.array_equal(b["entries"][:n], order)
    assert np.array_equal(b["counts"], np.bincount(flat[valid], minlength=4))
    assert (b["inverse"][flat < 0] == -1).all()
    pos = np.empty(len(flat), np.int64)
    pos[order] = np.arange(n)
    assert np.array_equal(b["inverse"][valid], pos[valid])
    assert b["active"].tolist() == [0, 1, 2, 3]


def test_layer_with_top_p_is_the_layer_of_the_kept_experts():
    """The layer output equals the sum over the kept experts only (dense
    per-token evaluation with the renormalized weights)."""
    cfg = gen.shrink(gen.get_config("c0"), hidden=128, inter=64, n_experts=16, top_k=6,
                     n_group=4, topk_group=2, top_p=0.6, seed=9)
    hl = gen.host_layer(cfg, 0, experts="all")
    x = gen.x_tokens(cfg, 7, batch_id=3)
    out, idx, w = oracle.layer_forward_host(hl, x)
    assert (idx < 0).any() and (idx >= 0).any()
    d = oracle.Desc.from_config(cfg)
    routed = oracle.expert_set_from_host_layer(hl)
    shared = oracle.shared_set_from_host_layer(hl)
    pt = oracle.layer_forward_per_token(d, hl.w_router, hl.bias, routed, shared, x, 7)
    assert np.array_equal(out, pt)
    # against the plain layer restricted by hand: same experts, the kept
    # weights, each expert FFN from the oracle's single-expert call
    _, _, w64 = oracle.route(d, hl.w_router, hl.bias, x, 7)
    for t in range(7):
        acc = np.zeros(cfg.hidden)
        for j in range(cfg.top_k):
            e = int(idx[t, j])
            if e < 0:
                continue
            y = oracle.expert_ffn(d, routed, e, x[t:t + 1], n_rows=1)
            acc += w64[t, j] * y[0]
        if cfg.n_shared:
            acc += oracle.expert_ffn(d, shared, 0, x[t:t + 1], n_rows=1,
                                     inter=cfg.inter * cfg.n_shared)[0]
        np.testing.assert_allclose(out[t], acc, rtol=1e-12, atol=1e-15)
