"""Pins of the oracle's batch-union grouping (CPU only): it must equal a
stable sort of the flat slots by expert."""
import numpy as np
import pytest

import oracle


def _check(idx, E):
    b = oracle.bucket(idx, E)
    flat = idx.reshape(-1)
    order = np.argsort(flat, kind="stable")
    assert np.array_equal(b["entries"], order.astype(np.int32))
    assert np.array_equal(b["counts"], np.bincount(flat, minlength=E).astype(np.int32))
    assert np.array_equal(b["offsets"], np.concatenate([[0], np.cumsum(b["counts"])]).astype(np.int32))
    assert np.array_equal(b["inverse"][b["entries"]], np.arange(flat.size, dtype=np.int32))
    assert np.array_equal(b["active"], np.flatnonzero(b["counts"]).astype(np.int32))
    assert b["n_active"] == len(b["active"])
    return b


@pytest.mark.parametrize("T,k,E", [(1, 8, 256), (16, 8, 256), (2048, 8, 256), (7, 2, 8),
                                   (33, 5, 1000), (1, 1, 1)])
def test_bucket_equals_stable_sort(T, k, E):
    rng = np.random.default_rng(T * 7 + k)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _check(idx, E)


def test_bucket_skewed_and_empty():
    idx = np.zeros((50, 1), np.int32)           # all slots on one expert
    b = _check(idx, 16)
    assert b["n_active"] == 1 and b["counts"][0] == 50
    b = oracle.bucket(np.zeros((0, 8), np.int32), 16)
    assert b["n_active"] == 0 and (b["counts"] == 0).all() and (b["offsets"] == 0).all()


def test_uniform_overlap_band():
    """Under independent uniform top-8 of 256, B tokens touch 256(1-(1-8/256)^B)
    experts on average (15.75 / 30.53 / 101.96 for B = 2 / 4 / 16)."""
    rng = np.random.default_rng(3)
    for B, expect in ((2, 15.75), (4, 30.53), (16, 101.96)):
        n = [oracle.bucket(np.stack([rng.permutation(256)[:8] for _ in range(B)]).astype(np.int32),
                           256)["n_active"] for _ in range(400)]
        assert abs(np.mean(n) - expect) < 0.02 * expect + 0.1
