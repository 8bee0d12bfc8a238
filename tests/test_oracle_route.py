"""Pins of the oracle's routing and grouping.

* top-k ids: brute force with numpy's lexsort on (expert index, -logit);
* weights: scipy's softmax over the selected logits; sum to 1, non-increasing;
* grouping: numpy's stable argsort of the pair experts; every routed (token, expert)
  pair appears exactly once; pos o sorted is the identity; empty experts have equal
  offsets.
"""

import numpy as np
import pytest
from scipy.special import softmax

from oracle.route import group_pairs, permute_rows, topk_route
from synth import CONFIGS, moe_inputs


@pytest.mark.parametrize("T,E,k", [(50, 8, 2), (40, 64, 8), (10, 5, 5), (7, 1, 1)])
def test_topk_vs_lexsort(T, E, k):
    rng = np.random.default_rng(T * E + k)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[:, : E // 2] = np.round(lg[:, : E // 2])  # plenty of exact ties
    ids, w = topk_route(lg, k)
    for t in range(T):
        order = np.lexsort((np.arange(E), -lg[t].astype(np.float64)))[:k]
        assert list(ids[t]) == list(order)
        assert len(set(ids[t])) == k
        ref = softmax(lg[t, order].astype(np.float64))
        assert np.allclose(w[t], ref, rtol=1e-14, atol=0)
        assert abs(w[t].sum() - 1) < 1e-12 and np.all(np.diff(w[t]) <= 1e-15)


def test_topk_renormalised_equals_full_softmax_renormalised():
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((20, 16)).astype(np.float32)
    ids, w = topk_route(lg, 4)
    full = softmax(lg.astype(np.float64), axis=1)
    sel = np.take_along_axis(full, ids.astype(np.int64), axis=1)
    assert np.allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-13)


@pytest.mark.parametrize("cfg", ["moe_tiny", "moe_prefill"])
def test_grouping_invariants(cfg):
    c = CONFIGS[cfg]
    inp = moe_inputs(c)
    ids, _ = topk_route(inp["logits"], c.k)
    off, sorted_, pos = group_pairs(ids, c.E)
    R = c.T * c.k
    flat = ids.reshape(-1)
    assert off[0] == 0 and off[-1] == R and np.all(np.diff(off) >= 0)
    # the library's stable sort gives the same order
    assert np.array_equal(sorted_, np.argsort(flat, kind="stable"))
    # every routed pair exactly once
    assert np.array_equal(np.sort(sorted_), np.arange(R))
    assert np.array_equal(pos[sorted_], np.arange(R))
    for e in range(c.E):
        rows = sorted_[off[e]:off[e + 1]]
        assert np.all(flat[rows] == e) and np.all(np.diff(rows) > 0)
    x = np.arange(c.T)[:, None]
    assert np.array_equal(permute_rows(x, sorted_, c.k)[:, 0], sorted_ // c.k)


def test_empty_experts_and_skew():
    ids = np.array([[0, 3], [3, 0], [0, 3]], dtype=np.int32)
    off, sorted_, pos = group_pairs(ids, 6)
    assert list(off) == [0, 3, 3, 3, 6, 6, 6]
    assert list(sorted_) == [0, 3, 4, 1, 2, 5]


def test_skewed_config_has_empty_experts():
    c = CONFIGS["moe_skewed"]
    from synth.inputs import router_logits
    lg = router_logits(c.seed, f"{c.name}.logits", c.T, c.E, c.zipf_s)
    # top-k by logit with lexsort (library) -- the histogram only
    top = np.argsort(-lg, axis=1, kind="stable")[:, : c.k]
    counts = np.bincount(top.reshape(-1), minlength=c.E)
    assert (counts == 0).sum() >= 1 and counts.max() > 10 * counts.mean()
