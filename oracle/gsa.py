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

Prefill under the gist mask: SSA article section 4 (continued pretraining:
the text is cut into segments with gist tokens; a segment's raw tokens see
one another and every earlier segment's gists, never earlier segments' raw
tokens), section 6 (prefill kernel: the global columns -- gists and
attention anchors -- are moved in front of the keys, which softmax does not
mind, so the pattern becomes a dense thin block plus a diagonal band).
Readings: causal order is the interleaved one (chunk c's raw tokens, then
its gist); a segment's raw tokens see one another causally; a gist token
sees its own segment's raw tokens, the earlier gists and itself; the
attention anchors are the first ``n_sink`` raw positions of the sequence,
seen by every later token (none in the workload).

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


def gsa_prefill_visible(n_chunks: int, chunk: int, n_sink: int = 0):
    """The gist-mask pattern over the interleaved sequence: returns
    ``(is_gist[T], chunk_of[T], raw_pos[T], vis[T, T])`` with T = n_chunks *
    (chunk + 1); ``vis[t, s]`` is whether token t may attend to token s."""
    T = n_chunks * (chunk + 1)
    t = np.arange(T)
    seg, off = t // (chunk + 1), t % (chunk + 1)
    is_gist = off == chunk
    raw_pos = np.where(is_gist, -1, seg * chunk + off)
    earlier = t[None, :] <= t[:, None]                       # causal: s <= t
    same_seg = seg[None, :] == seg[:, None]
    sink = (~is_gist) & (raw_pos < n_sink)
    vis = earlier & (is_gist[None, :] | same_seg | sink[None, :])
    return is_gist, seg, raw_pos, vis


def gsa_prefill(q_raw, q_gist, k_raw, v_raw, k_gist, v_gist, chunk: int, scale: float,
                n_sink: int = 0):
    """Attention of every raw and gist token under the gist mask.

    Raw arrays ``[n_chunks*chunk, D]`` in token order, gist arrays
    ``[n_chunks, D]``.  Returns ``(out_raw, out_gist)`` in float64.
    """
    n_chunks = np.asarray(k_gist).shape[0]
    is_gist, seg, raw_pos, vis = gsa_prefill_visible(n_chunks, chunk, n_sink)
    # the interleaved sequence's rows
    idx_raw = np.where(is_gist, 0, raw_pos)
    def seq(raw, gist):
        raw, gist = np.asarray(raw, np.float64), np.asarray(gist, np.float64)
        return np.where(is_gist[:, None], gist[seg], raw[idx_raw])
    q, k, v = seq(q_raw, q_gist), seq(k_raw, k_gist), seq(v_raw, v_gist)
    out = np.zeros((q.shape[0], v.shape[1]))
    for t in range(q.shape[0]):
        keys = np.nonzero(vis[t])[0]
        out[t] = softmax_attention(q[t][None], k[keys], v[keys], scale)[0]
    return out[~is_gist], out[is_gist]


def gsa_prefill_rows(q_raw, q_gist, k_raw, v_raw, k_gist, v_gist, chunk: int, scale: float,
                     raw_rows=(), gist_rows=(), n_sink: int = 0):
    """Selected rows of :func:`gsa_prefill` (raw token ids, gist ids), each
    from its own visible key list, without the full mask: raw token i of
    chunk c sees the gists of chunks < c, the anchors before it and chunk c's
    raw tokens up to itself; gist c sees the gists up to itself, the anchors
    and chunk c's raw tokens."""
    kr, vr = np.asarray(k_raw, np.float64), np.asarray(v_raw, np.float64)
    kg, vg = np.asarray(k_gist, np.float64), np.asarray(v_gist, np.float64)

    def run(q, c, last_raw, gists_upto):
        raw_ids = set(range(c * chunk, last_raw + 1)) | set(range(min(n_sink, last_raw + 1)))
        raw_ids = sorted(raw_ids)
        keys = np.vstack([kg[:gists_upto], kr[raw_ids]])
        vals = np.vstack([vg[:gists_upto], vr[raw_ids]])
        return softmax_attention(np.asarray(q, np.float64)[None], keys, vals, scale)[0]

    out_r = np.array([run(q_raw[t], t // chunk, t, t // chunk) for t in raw_rows]).reshape(-1, vr.shape[1])
    out_g = np.array([run(q_gist[c], c, (c + 1) * chunk - 1, c + 1) for c in gist_rows]).reshape(-1, vg.shape[1])
    return out_r, out_g
