"""Lightning-indexer scores, exact integers.

Source: "长上下文：稀疏注意力 / DSA / IndexShare" tutorial, section
"DSA 与 IndexShare": a lightweight indexer gives every history token a
relevance score for the current query, and only the top-k are attended.

Reading (the pages give no formula): the score of cached position ``t`` for
query row ``r`` is the plain sum over indexer heads of the per-head int8 dot
products,

    s[b, r, t] = sum_h sum_j Qi[b, r, h, j] * Ki[b, t, h, j],

with no per-head weight, no nonlinearity and no scale.  The sum over heads
of per-head dot products equals one dot product over the concatenated
``H_idx * d_idx`` features, which is how the arrays are laid out here:
``Qi[B, Lq, H_idx*d_idx]`` and ``Ki[B, L, H_idx*d_idx]`` (head-major inside
a row).
"""

from __future__ import annotations

import numpy as np


def index_scores(qi: np.ndarray, ki: np.ndarray, n_heads: int) -> np.ndarray:
    """Exact int64 scores ``[B, Lq, L]``.

    ``qi``: int8 ``[B, Lq, n_heads*d]``; ``ki``: int8 ``[B, L, n_heads*d]``.
    No masking is applied here: which positions are candidates is decided
    by the valid length given to :func:`oracle.topk.select_topk`.
    """
    B, Lq, HD = qi.shape
    assert ki.shape[0] == B and ki.shape[2] == HD and HD % n_heads == 0
    d = HD // n_heads
    q = qi.astype(np.int64).reshape(B, Lq, n_heads, d)
    k = ki.astype(np.int64).reshape(B, ki.shape[1], n_heads, d)
    s = np.zeros((B, Lq, ki.shape[1]), dtype=np.int64)
    for h in range(n_heads):  # sum of per-head dot products
        for b in range(B):
            s[b] += q[b, :, h, :] @ k[b, :, h, :].T
    return s


def index_scores_row(qi_row: np.ndarray, ki: np.ndarray) -> np.ndarray:
    """Scores of one query row against ``ki[L, HD]`` (int64), any head split.

    Provided for sampled checks at full size: it touches only one query row.
    """
    return ki.astype(np.int64) @ qi_row.astype(np.int64)


def index_scores_f32(qi: np.ndarray, ki: np.ndarray) -> np.ndarray:
    """Scores ``[R, L]`` (int64) of query rows ``qi[R, HD]`` against ``ki[L, HD]``
    through a float32 matrix product.

    Exact, not approximate: every product of two int8 values and every partial
    sum of at most ``HD`` of them is an integer of magnitude at most
    ``HD * 128 * 128``, and while that stays below 2**24 float32 represents
    each of them exactly, so any summation order gives the exact integer.  The
    bound is checked.  Used for whole-group checks at the large workloads,
    where the int64 product is too slow.
    """
    HD = qi.shape[-1]
    if HD * 128 * 128 >= (1 << 24):
        raise ValueError("float32 sums are exact only for HD * 2**14 < 2**24")
    s = qi.astype(np.float32) @ ki.astype(np.float32).T
    return s.astype(np.int64)
