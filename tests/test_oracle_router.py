"""Pins of the oracle's router (CPU only).

The selection rule (sigmoid noaux_tc: groups scored by their two best
biased scores, top groups kept, top-k inside them; weights renormalised over
the chosen and scaled) is checked against an exhaustive subset search, exact
ties, reductions to a plain sort, and closed-form weights.
"""
import itertools
import math

import numpy as np
import pytest
from scipy.special import expit, softmax

import gen
import oracle


def _desc(E, k, G=1, g=1, scaling=1.0, router=oracle.SIGMOID_NOAUX_TC, H=8):
    return oracle.Desc(hidden=H, inter=8, n_experts=E, top_k=k, router=router, n_group=G,
                       topk_group=g, routed_scaling=scaling)


def _lex_best_subset(values, pool, size):
    """Max-sum subset of `pool` of `size`; among equal sums the lexicographically
    smallest sorted index tuple (== greedy with lowest index on ties)."""
    best, best_key = None, None
    for sub in itertools.combinations(sorted(pool), size):
        s = math.fsum(values[i] for i in sub)
        key = (-s, sub)
        if best_key is None or key < best_key:
            best, best_key = sub, key
    return best


def _brute_noaux(z, bias, G, g, k):
    E = len(z)
    c = expit(z) + (bias if bias is not None else 0.0)
    per = E // G
    gscore = []
    for grp in range(G):
        members = range(grp * per, (grp + 1) * per)
        if per == 1:
            gscore.append(c[grp * per])
        else:
            gscore.append(max(c[a] + c[b] for a, b in itertools.combinations(members, 2)))
    kept = _lex_best_subset(gscore, range(G), g)
    cand = [e for grp in kept for e in range(grp * per, (grp + 1) * per)]
    chosen = _lex_best_subset(c, cand, k)
    order = sorted(chosen, key=lambda e: (-c[e], e))
    return np.array(order, dtype=np.int32)


@pytest.mark.parametrize("E,G,g,k", [(8, 2, 1, 2), (8, 4, 2, 3), (12, 3, 2, 4), (6, 6, 3, 2),
                                     (8, 1, 1, 3), (9, 3, 3, 5)])
def test_select_matches_subset_search(E, G, g, k):
    rng = np.random.default_rng(E * 100 + G * 10 + k)
    d = _desc(E, k, G, g, scaling=2.5)
    for trial in range(40):
        z = rng.normal(size=(1, E))
        bias = rng.normal(scale=0.05, size=E).astype(np.float32)
        if trial % 5 == 0:   # quantised values create exact ties
            z = np.round(z * 2) / 2
            bias = np.zeros(E, np.float32)
        idx, w, w64 = oracle.select(d, z, bias, 1)
        want = _brute_noaux(z[0], bias.astype(np.float64), G, g, k)
        assert idx[0].tolist() == want.tolist(), (z, bias)
        s = expit(z[0][want])
        assert np.allclose(w64[0], s / s.sum() * 2.5, rtol=1e-14, atol=0)


@pytest.mark.parametrize("shape", ["c0", "c2"])
def test_exact_ties_x_zero(shape):
    """x = 0 and bias = 0: every score is 1/2, so the lowest groups and then the
    lowest experts win, with weights scaling/k exactly."""
    cfg = gen.get_config(shape)
    d = oracle.Desc.from_config(cfg)
    w_r, _ = gen.router(cfg)
    x = np.zeros((3, cfg.hidden), np.float32)
    idx, w, _ = oracle.route(d, w_r, np.zeros(cfg.n_experts, np.float32), x, 3)
    assert (idx == np.arange(cfg.top_k)).all()
    assert (w == np.float32(cfg.routed_scaling / cfg.top_k)).all()


def test_duplicate_rows_lower_index_wins():
    cfg = gen.get_config("c2")
    d = oracle.Desc.from_config(cfg)
    w_r, bias = gen.router(cfg)
    x = gen.x_tokens(cfg, 4)
    idx0, _, _ = oracle.route(d, w_r, bias, x, 4)
    # copy the top expert's row and bias onto a higher index in the same group
    for t in range(4):
        top = int(idx0[t, 0])
        grp = top // (cfg.n_experts // cfg.n_group)
        twin = (grp + 1) * (cfg.n_experts // cfg.n_group) - 1
        if twin == top:
            continue
        w2, b2 = w_r.copy(), bias.copy()
        w2[twin], b2[twin] = w2[top], b2[top]
        idx, _, _ = oracle.route(d, w2, b2, x[t:t + 1], 1)
        assert idx[0, 0] == top and idx[0, 1] == twin


def test_reduces_to_plain_topk_when_all_groups_kept():
    rng = np.random.default_rng(5)
    E, k = 64, 6
    d = _desc(E, k, G=8, g=8, scaling=1.0)
    z = rng.normal(size=(20, E))
    bias = rng.normal(scale=0.01, size=E).astype(np.float32)
    idx, _, _ = oracle.select(d, z, bias, 20)
    c = expit(z) + bias.astype(np.float64)
    for t in range(20):
        order = np.lexsort((np.arange(E), -c[t]))[:k]
        assert idx[t].tolist() == order.tolist()


def test_unbiased_ungrouped_is_topk_of_logits():
    rng = np.random.default_rng(6)
    E, k = 256, 8
    d = _desc(E, k, G=1, g=1)
    z = rng.normal(size=(10, E))
    idx, _, _ = oracle.select(d, z, None, 10)
    for t in range(10):
        assert idx[t].tolist() == np.lexsort((np.arange(E), -z[t]))[:k].tolist()


def test_closed_form_weights():
    """z = +-ln 3 gives sigmoid scores 3/4 and 1/4 exactly (up to rounding of
    ln 3): weights (3/4, 1/4) * scaling."""
    d = _desc(4, 2, G=2, g=2, scaling=2.5)
    z = np.array([[math.log(3.0), -math.log(3.0), -5.0, -6.0]])
    idx, w, w64 = oracle.select(d, z, None, 1)
    assert idx[0].tolist() == [0, 1]
    assert np.allclose(w64[0], [1.875, 0.625], rtol=1e-15)
    assert w[0].tolist() == [1.875, 0.625]


def test_softmax_router():
    rng = np.random.default_rng(7)
    E, k = 32, 8
    d = _desc(E, k, router=oracle.SOFTMAX_TOPK, scaling=1.0)
    z = rng.normal(size=(16, E))
    idx, w, w64 = oracle.select(d, z, None, 16)
    for t in range(16):
        order = np.lexsort((np.arange(E), -z[t]))[:k]
        assert idx[t].tolist() == order.tolist()
        assert np.allclose(w64[t], softmax(z[t][order]), rtol=1e-14)
        # full softmax renormalised over the chosen gives the same weights
        p = softmax(z[t])
        assert np.allclose(w64[t], p[order] / p[order].sum(), rtol=1e-13)
    d1 = _desc(E, 1, router=oracle.SOFTMAX_TOPK, scaling=1.0)
    _, w1, _ = oracle.select(d1, z, None, 16)
    assert (w1 == 1.0).all()


def test_invariants_glm_shape():
    cfg = gen.get_config("c2")
    d = oracle.Desc.from_config(cfg)
    w_r, bias = gen.router(cfg)
    x = gen.normal_f32((64, cfg.hidden), 99, 0, gen.T_X, 0, 1.0)
    idx, w, w64 = oracle.route(d, w_r, bias, x, 64)
    per = cfg.n_experts // cfg.n_group
    for t in range(64):
        assert len(set(idx[t].tolist())) == cfg.top_k
        assert len(set((idx[t] // per).tolist())) <= cfg.topk_group
        assert abs(w64[t].sum() / cfg.routed_scaling - 1.0) <= 1e-12
        assert abs(float(w[t].astype(np.float64).sum()) / cfg.routed_scaling - 1.0) <= 1e-6


def test_logits_exact_cases():
    cfg = gen.get_config("c0")
    d = oracle.Desc.from_config(cfg)
    w_r, _ = gen.router(cfg)
    x = np.zeros((cfg.hidden, cfg.hidden), np.float32)
    np.fill_diagonal(x, 1.0)
    z = oracle.logits(d, w_r, x, cfg.hidden)
    assert np.array_equal(z, w_r.T.astype(np.float64))
    rng = np.random.default_rng(1)
    xi = rng.integers(-50, 50, size=(5, cfg.hidden)).astype(np.float32)
    wi = rng.integers(-50, 50, size=(cfg.n_experts, cfg.hidden)).astype(np.float32)
    z = oracle.logits(d, wi, xi, 5)
    assert np.array_equal(z, xi.astype(np.float64) @ wi.T.astype(np.float64))
