"""Gist-chunk selection and selective unfolding (GSA / SSA), float64.

Sources:

* SSA article (arXiv 2604.20920), section 2: the sequence is cut into
  chunks of fixed length (16 tokens in the example) and one gist token is
  inserted after each chunk.
* Same article, section 3, and the GSA summary page, section 2.2: at each
  decode step the query is compared with every gist (dot product), the
  top-k chunks are chosen, and their raw tokens are unfolded into the
  attention context together with the chosen chunks' own gists; gists of
  unchosen chunks are left out (the "SG+SR" composition that the ablation
  in section 8 of the SSA article finds best).

Readings where the pages are silent or disagree:

* The GSA summary page also describes attending over "selected raw chunks
  + all gists"; the SSA article's ablation and the workload definition use
  the selected gists only, which is what is computed here.
* Chunk selection uses the unscaled dot product ``q . gK``; the attention
  itself uses scale ``1/sqrt(D)``.  Ties go to the lower chunk number.
* The current token opens an unfinished chunk; its first ``tail_len`` raw
  positions (including the current token) are always attended.
* The gist logit in attention is the same ``q . gK`` product, scaled.

Hierarchical routing (H-GSA / H-SSA): SSA article section 5 (a meta-gist
token after every few gist tokens summarises them; the query first picks the
best meta-gists, then the best gists inside their groups, then unfolds those
chunks' raw tokens) and the GSA summary page section 2.4 (gist-of-gist,
coarse-to-fine selection, O(log N) routing).  Readings: meta-gist ``g``
covers gists ``[g*group, (g+1)*group)`` (the last group may be short); its
routing score is the unscaled ``q . mK`` like the gists'; ties go to the
lower group, then to the lower chunk; meta-gists only route: the attention
is the GSA one over the chosen chunks' raw tokens and gists plus the tail.
"""

from __future__ import annotations

import numpy as np

from .attention import softmax_attention
from .topk import select_topk


def gist_scores(q: np.ndarray, gk: np.ndarray) -> np.ndarray:
    """``q[..., D]``, ``gk[..., Nc, D]`` -> ``[..., Nc]`` float64 dot products."""
    q = np.asarray(q, dtype=np.float64)
    gk = np.asarray(gk, dtype=np.float64)
    return np.einsum("...d,...cd->...c", q, gk)


def gsa_key_positions(chunk_idx: np.ndarray, chunk: int, n_chunks: int, tail_len: int):
    """Raw positions and gist ids that one query attends to.

    ``chunk_idx``: selected chunk ids (ascending, -1 padded).  Returns
    ``(raw_positions, gist_ids)``: the raw tokens of every chosen chunk,
    then the tail of the unfinished chunk; and the chosen gists.
    """
    sel = np.asarray([c for c in chunk_idx if c >= 0], dtype=np.int64)
    raw = (sel[:, None] * chunk + np.arange(chunk)[None, :]).reshape(-1)
    tail = n_chunks * chunk + np.arange(tail_len, dtype=np.int64)
    return np.concatenate([raw, tail]), sel


def gsa_attention(q: np.ndarray, raw_k: np.ndarray, raw_v: np.ndarray, gist_k: np.ndarray,
                  gist_v: np.ndarray, scale: float) -> np.ndarray:
    """One head: attention over the unfolded raw rows plus the chosen gists.

    All key/value arguments are the already-gathered rows ``[n, D]``.
    """
    keys = np.concatenate([np.asarray(raw_k, np.float64), np.asarray(gist_k, np.float64)], axis=0)
    vals = np.concatenate([np.asarray(raw_v, np.float64), np.asarray(gist_v, np.float64)], axis=0)
    return softmax_attention(np.asarray(q, np.float64)[None, :], keys, vals, scale)[0]


def gsa_select(q: np.ndarray, gk: np.ndarray, kc: int) -> np.ndarray:
    """Chosen chunk ids ``[..., kc]`` (ascending, -1 padded)."""
    return select_topk(gist_scores(q, gk), kc)


def hgsa_select(q: np.ndarray, mk: np.ndarray, gk: np.ndarray, group: int, km: int,
                kc: int) -> np.ndarray:
    """Coarse-to-fine chunk choice for one query: ``q[D]``, meta-gist keys
    ``mk[Nm, D]``, gist keys ``gk[Nc, D]`` -> chosen chunk ids ``[kc]``
    (ascending, -1 padded when the chosen groups hold fewer than kc chunks).
    """
    gk = np.asarray(gk)
    nc = gk.shape[0]
    groups = select_topk(gist_scores(q, mk), km)           # the km best meta-gists
    groups = groups[groups >= 0]
    cand = np.concatenate([np.arange(g * group, min((g + 1) * group, nc)) for g in groups])
    s = gist_scores(q, gk[cand])
    order = np.lexsort((cand, -s))                        # score desc, then chunk asc
    chosen = np.sort(cand[order[:kc]])
    out = np.full(kc, -1, dtype=np.int32)
    out[:chosen.size] = chosen
    return out
