"""Top-k routing and token grouping -- oracle side (test infrastructure).

The FP8 grouped-expert prefill note (section 1) replaces one dispatch per routed token
with one grouped expert GEMM per layer. That needs the routed (token, expert) pairs
grouped by expert, with per-expert row offsets, so one launch can cover every expert.

Readings where the pages are silent:
* selection is by fp32 logit, descending; equal logits go to the lower expert index
  first (softmax is monotone, so this is the same set as selecting by probability, and
  it avoids ties that softmax rounding would create); a NaN logit ranks as -inf;
* the weights are the softmax renormalised over the selected k experts, which equals
  the full softmax renormalised over the top k;
* pairs are numbered p = t*k + j; within an expert, pairs keep increasing p order (a
  stable counting sort), so tokens ascend within each expert's rows.
"""

from __future__ import annotations

import numpy as np


def topk_route(logits: np.ndarray, k: int):
    """fp32 logits [T, E] -> (ids int32 [T, k], weights float64 [T, k])."""
    lg = np.asarray(logits, dtype=np.float32)
    lg = np.where(np.isnan(lg), np.float32(-np.inf), lg)
    T, E = lg.shape
    assert 1 <= k <= E
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        # order by (logit descending, expert index ascending)
        order = sorted(range(E), key=lambda e: (-float(lg[t, e]), e))[:k]
        ids[t] = order
        sel = lg[t, order].astype(np.float64)
        ex = np.exp(sel - sel.max())
        w[t] = ex / ex.sum()
    return ids, w


def group_pairs(ids: np.ndarray, E: int):
    """Counting sort of the routed pairs by expert.

    Returns offsets int32 [E+1] (offsets[e]..offsets[e+1] are expert e's rows),
    sorted int32 [R] (sorted[i] = pair id p = t*k + j placed at row i) and
    pos int32 [R] (pos[p] = the row of pair p; pos is the inverse of sorted).
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    R = T * k
    counts = np.zeros(E, dtype=np.int64)
    for e in ids.reshape(-1):
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    fill = offsets[:-1].copy()
    sorted_ = np.empty(R, dtype=np.int64)
    for p, e in enumerate(ids.reshape(-1)):  # increasing p: stable
        sorted_[fill[e]] = p
        fill[e] += 1
    pos = np.empty(R, dtype=np.int64)
    pos[sorted_] = np.arange(R)
    return offsets.astype(np.int32), sorted_.astype(np.int32), pos.astype(np.int32)


def permute_rows(rows: np.ndarray, sorted_: np.ndarray, k: int) -> np.ndarray:
    """Row i of the permuted tensor is the token row of pair sorted[i] (token p // k)."""
    return np.asarray(rows)[np.asarray(sorted_, dtype=np.int64) // k]
