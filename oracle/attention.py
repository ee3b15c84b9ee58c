"""Softmax attention restricted to a selected key set, float64.

Source: CLSA explainer, section 1.1: Attention(Q, K, V) =
softmax(Q K^T / sqrt(d_k)) V.  Sparse attention (tutorial page, DSA
section; CLSA section 2.3 "selector") is the same formula evaluated only
over the selected keys: once the index set is fixed the result is exact,
so the oracle is the definition itself.

Readings: inputs are post-projection tensors (no RoPE, no norms); query
head ``h`` reads KV head ``h // (Hq // Hkv)``; the output is float.
"""

from __future__ import annotations

import numpy as np

ROW_SUM_TOL = 1e-12


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """``q[m, D]``, ``k[n, D]``, ``v[n, Dv]`` -> ``[m, Dv]`` in float64.

    With ``n == 0`` the result is all zeros (nothing to attend to).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    z = (q @ k.T) * scale                      # [m, n] logits
    z = z - z.max(axis=1, keepdims=True)       # subtract the row maximum
    e = np.exp(z)
    p = e / e.sum(axis=1, keepdims=True)       # softmax over keys
    row = p.sum(axis=1)
    if np.any(np.abs(row - 1.0) > ROW_SUM_TOL):
        raise AssertionError("softmax row does not sum to 1")
    return p @ v


def sparse_attention_gqa(q: np.ndarray, k_sel: np.ndarray, v_sel: np.ndarray,
                         scale: float) -> np.ndarray:
    """One query position, all heads, over already-gathered keys.

    ``q[Hq, D]``; ``k_sel``/``v_sel`` ``[n, Hkv, D]`` (the selected rows of
    the cache, any order).  Returns ``[Hq, D]`` float64.
    """
    Hq = q.shape[0]
    Hkv = k_sel.shape[1]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    out = np.zeros((Hq, v_sel.shape[2]), dtype=np.float64)
    for h in range(Hq):
        kvh = h // G
        out[h] = softmax_attention(q[h : h + 1], k_sel[:, kvh, :], v_sel[:, kvh, :], scale)[0]
    return out
