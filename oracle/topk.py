"""Top-k position selection.

Source: "长上下文：稀疏注意力 / DSA / IndexShare" tutorial, section
"DSA 与 IndexShare" (each query keeps only its top-k positions); CLSA
explainer section 2.3 (the indexer outputs, per query, the indices of the
k most important tokens; the index set is a small integer array).

Readings where the pages are silent:

* Order: score descending, then position ascending, so among equal scores
  the lowest position wins.  Exactly one set satisfies this total order.
* Only positions ``[0, valid_len)`` are candidates.  When fewer than ``k``
  are valid, all valid positions are returned.
* The output row lists the chosen positions in ascending order, padded on
  the right with -1 up to ``k``.
"""

from __future__ import annotations

import numpy as np


def select_topk(scores: np.ndarray, k: int, valid_len=None) -> np.ndarray:
    """Index sets ``[..., k]`` (int32) for score rows ``[..., n]``.

    ``scores`` may be integer or floating point; comparisons use the values
    exactly as given.  ``valid_len`` is None (all ``n`` valid), an int, or
    an integer array broadcastable to ``scores.shape[:-1]``.
    """
    scores = np.asarray(scores)
    lead = scores.shape[:-1]
    n = scores.shape[-1]
    flat = scores.reshape(-1, n)
    if valid_len is None:
        vl = np.full(flat.shape[0], n, dtype=np.int64)
    else:
        vl = np.broadcast_to(np.asarray(valid_len, dtype=np.int64), lead).reshape(-1)
    out = np.full((flat.shape[0], k), -1, dtype=np.int32)
    for r in range(flat.shape[0]):
        nv = int(min(max(vl[r], 0), n))
        row = flat[r, :nv]
        pos = np.arange(nv, dtype=np.int64)
        # np.lexsort sorts by the last key first: score descending, then
        # position ascending.
        order = np.lexsort((pos, -row.astype(np.float64) if row.dtype.kind == "f" else -row.astype(np.int64)))
        take = np.sort(order[: min(k, nv)])
        out[r, : take.size] = take
    return out.reshape(lead + (k,))


def select_topk_threshold(scores: np.ndarray, k: int, valid_len=None) -> np.ndarray:
    """The same index sets as :func:`select_topk`, found without a full sort.

    For score rows ``[R, n]`` (integer or float): the k-th largest valid value T comes
    from a partition; every valid position scoring above T is chosen, and of
    the positions scoring exactly T the lowest-numbered ones fill the rest
    (the tie rule).  Rows with at most k valid positions keep all of them.
    Used for whole-group checks at the large workloads.
    """
    scores = np.asarray(scores)
    R, n = scores.shape
    vl = np.broadcast_to(np.asarray(n if valid_len is None else valid_len, dtype=np.int64), (R,))
    vl = np.clip(vl, 0, n)
    out = np.full((R, k), -1, dtype=np.int32)
    if scores.dtype.kind == "f":
        masked, low = scores.astype(np.float64, copy=True), -np.inf
    else:
        masked, low = scores.astype(np.int64, copy=True), np.iinfo(np.int64).min
    pos = np.arange(n)
    masked[pos[None, :] >= vl[:, None]] = low
    short = vl <= k
    for r in np.where(short)[0]:
        out[r, : vl[r]] = np.arange(vl[r])
    long_rows = np.where(~short)[0]
    if long_rows.size:
        m = masked[long_rows]
        T = np.partition(m, n - k, axis=1)[:, n - k]                 # k-th largest value
        above = m > T[:, None]
        need = k - above.sum(axis=1)                                 # ties at T to take
        eq = m == T[:, None]
        take = above | (eq & (np.cumsum(eq, axis=1) <= need[:, None]))
        for j, r in enumerate(long_rows):
            out[r] = np.nonzero(take[j])[0]
    return out
