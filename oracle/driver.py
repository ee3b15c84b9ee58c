"""Layer-group driver: one indexer call per group, index set shared by the group.

Sources:

* CLSA explainer, section 2.3 workflow: the indexer computes the top-k
  index set once, the shared index goes to every layer, and each layer's
  selector gathers K/V by that index without recomputing top-k.
* Tutorial page, DSA / IndexShare section: every 4 sparse-attention layers
  share one indexer's result.
* IndexCache article, sections 2 and 6: Full layers run their indexer and
  write the result to one temporary buffer; Shared layers read the most
  recent Full layer's buffer, which the next Full layer overwrites.

Reading: group ``g`` is layers ``[g*G, (g+1)*G)``; its first layer is the
Full layer and owns the group's indexer inputs ``Qi_g``/``Ki_g``; the others
are Shared.  With a free Full/Shared pattern (IndexCache article, section 3)
group ``g`` runs from the ``g``-th Full layer up to the next one.  All inputs come from the seeded generator in ``synth`` and
only the rows a computation reads are regenerated.
"""

from __future__ import annotations

import numpy as np

import synth
from synth import configs as C

from .attention import sparse_attention_gqa
from .indexer import index_scores
from .topk import select_topk


def _f(kind, raw):
    return synth.as_float(kind, raw)


def decode_group(cfg: C.DecodeConfig, g: int, batch=None) -> np.ndarray:
    """Index sets ``[len(batch), Lq, k]`` of group ``g`` (Full layer's indexer)."""
    batch = list(range(cfg.B)) if batch is None else list(batch)
    out = []
    for b in batch:
        qi = C.rows(cfg, cfg.qi_spec(g), (np.array([b]),))          # [1, Lq, HD]
        ki = C.rows(cfg, cfg.ki_spec(g), (np.array([b]),))          # [1, L, HD]
        s = index_scores(qi, ki, cfg.H_idx)                         # [1, Lq, L]
        out.append(select_topk(s[0], cfg.topk, cfg.L))
    return np.stack(out)


def decode_layers(cfg: C.DecodeConfig, layer: int, idx: np.ndarray, batch=None,
                  qrows=None) -> np.ndarray:
    """Layer outputs ``[len(batch), len(qrows), Hq, D]`` (float64) given index sets.

    ``idx`` is ``[len(batch), Lq, k]`` as returned by :func:`decode_group`
    (the shared buffer of the layer's group).
    """
    batch = list(range(cfg.B)) if batch is None else list(batch)
    qrows = list(range(cfg.Lq)) if qrows is None else list(qrows)
    kq, _, _ = cfg.q_spec(layer)
    kk, _, _ = cfg.k_spec(layer)
    kv, _, _ = cfg.v_spec(layer)
    out = np.zeros((len(batch), len(qrows), cfg.Hq, cfg.D))
    for i, b in enumerate(batch):
        for j, r in enumerate(qrows):
            sel = idx[i, r]
            sel = sel[sel >= 0].astype(np.int64)
            q = _f(kq, C.rows(cfg, cfg.q_spec(layer), (np.array(b), np.array(r))))   # [Hq, D]
            ks = _f(kk, C.rows(cfg, cfg.k_spec(layer), (np.full_like(sel, b), sel)))  # [n, Hkv, D]
            vs = _f(kv, C.rows(cfg, cfg.v_spec(layer), (np.full_like(sel, b), sel)))
            out[i, j] = sparse_attention_gqa(q, ks, vs, cfg.scale)
    return out


def decode_step(cfg: C.DecodeConfig, batch=None, layers=None):
    """Whole decode step: ``({group: idx}, {layer: out})``.

    The group's index array is computed once and the very same array is
    handed to every layer of the group.
    """
    layers = list(range(cfg.n_layers)) if layers is None else list(layers)
    groups = sorted({l // cfg.group for l in layers})
    idx = {g: decode_group(cfg, g, batch) for g in groups}
    outs = {l: decode_layers(cfg, l, idx[l // cfg.group], batch) for l in layers}
    return idx, outs


def layer_owner(layer_full) -> list:
    """Ordinal of the Full layer whose index set each layer reads.

    IndexCache article, section 2: a Shared layer inherits the index of the
    most recent Full layer.  Section 3: the training-free greedy search drops
    indexers one at a time by their effect on quality, so the Full layers it
    keeps need not be evenly spaced.  Layer 0 has no earlier index to inherit
    and must be Full.
    """
    owner, g = [], -1
    for f in layer_full:
        if f:
            g += 1
        elif g < 0:
            raise ValueError("the first layer must be a Full layer")
        owner.append(g)
    return owner


def decode_step_pattern(cfg: C.DecodeConfig, layer_full, batch=None, layers=None):
    """Decode step with the Full layers placed by ``layer_full``.

    Returns ``({g: idx}, {layer: out})`` where ``g`` counts the Full layers
    in order; the ``g``-th Full layer owns the indexer inputs ``Qi_g``/``Ki_g``
    and every layer attends over the set of its owner (:func:`layer_owner`).
    """
    assert len(layer_full) == cfg.n_layers
    owner = layer_owner(layer_full)
    layers = list(range(cfg.n_layers)) if layers is None else list(layers)
    groups = sorted({owner[l] for l in layers})
    idx = {g: decode_group(cfg, g, batch) for g in groups}
    outs = {l: decode_layers(cfg, l, idx[owner[l]], batch) for l in layers}
    return idx, outs


def prefill_index_rows(cfg: C.DecodeConfig, g: int, rows) -> np.ndarray:
    """Causal prefill index sets for query rows ``rows`` of group ``g``.

    Query row ``i`` sits at position ``i`` and may choose among positions
    ``0..i``; it keeps ``min(k, i+1)`` of them.
    """
    assert cfg.causal and cfg.B == 1
    rows = np.asarray(list(rows), dtype=np.int64)
    qi = C.rows(cfg, cfg.qi_spec(g), (np.zeros_like(rows), rows))            # [R, HD]
    ki = C.rows(cfg, cfg.ki_spec(g), (np.array([0]),))[0]                      # [L, HD]
    s = index_scores(qi[None], ki[None], cfg.H_idx)[0]                         # [R, L]
    return select_topk(s, cfg.topk, rows + 1)


def prefill_attention_rows(cfg: C.DecodeConfig, layer: int, rows, idx_rows: np.ndarray) -> np.ndarray:
    """Causal prefill outputs ``[len(rows), Hq, D]`` for the given rows."""
    rows = list(rows)
    kq, _, _ = cfg.q_spec(layer)
    kk, _, _ = cfg.k_spec(layer)
    kv, _, _ = cfg.v_spec(layer)
    out = np.zeros((len(rows), cfg.Hq, cfg.D))
    for j, r in enumerate(rows):
        sel = idx_rows[j]
        sel = sel[sel >= 0].astype(np.int64)
        q = _f(kq, C.rows(cfg, cfg.q_spec(layer), (np.array(0), np.array(r))))
        ks = _f(kk, C.rows(cfg, cfg.k_spec(layer), (np.zeros_like(sel), sel)))
        vs = _f(kv, C.rows(cfg, cfg.v_spec(layer), (np.zeros_like(sel), sel)))
        out[j] = sparse_attention_gqa(q, ks, vs, cfg.scale)
    return out


def gsa_step(cfg: C.GsaConfig, pairs=None):
    """GSA decode for (b, h) pairs: ``(chunk_idx[P, kc], out[P, D])``."""
    from .gsa import gist_scores, gsa_attention, gsa_key_positions

    pairs = [(b, h) for b in range(cfg.B) for h in range(cfg.H)] if pairs is None else list(pairs)
    kq, _, _ = cfg.q_spec()
    kgk, _, _ = cfg.gk_spec()
    kgv, _, _ = cfg.gv_spec()
    krk, _, _ = cfg.rk_spec()
    krv, _, _ = cfg.rv_spec()
    idx = np.full((len(pairs), cfg.kc), -1, dtype=np.int32)
    out = np.zeros((len(pairs), cfg.D))
    for i, (b, h) in enumerate(pairs):
        q = _f(kq, C.rows(cfg, cfg.q_spec(), (np.array(b), np.array(h))))                 # [D]
        gk = _f(kgk, C.rows(cfg, cfg.gk_spec(), (np.array(b), np.array(h))))              # [Nc, D]
        sc = gist_scores(q, gk)
        idx[i] = select_topk(sc, cfg.kc)
        raw_pos, gist_ids = gsa_key_positions(idx[i], cfg.chunk, cfg.Nc, cfg.tail_len)
        bb, hh = np.full_like(raw_pos, b), np.full_like(raw_pos, h)
        rk = _f(krk, C.rows(cfg, cfg.rk_spec(), (bb, hh, raw_pos)))
        rv = _f(krv, C.rows(cfg, cfg.rv_spec(), (bb, hh, raw_pos)))
        gb, gh = np.full_like(gist_ids, b), np.full_like(gist_ids, h)
        gks = _f(kgk, C.rows(cfg, cfg.gk_spec(), (gb, gh, gist_ids)))
        gvs = _f(kgv, C.rows(cfg, cfg.gv_spec(), (gb, gh, gist_ids)))
        out[i] = gsa_attention(q, rk, rv, gks, gvs, cfg.scale)
    return idx, out


def hgsa_step(cfg: C.GsaConfig, pairs=None):
    """Hierarchically routed GSA decode for (b, h) pairs: ``(chunk_idx[P, kc], out[P, D])``."""
    from .gsa import gsa_attention, gsa_key_positions, hgsa_select

    pairs = [(b, h) for b in range(cfg.B) for h in range(cfg.H)] if pairs is None else list(pairs)
    kq, _, _ = cfg.q_spec()
    kgk, _, _ = cfg.gk_spec()
    kgv, _, _ = cfg.gv_spec()
    kmk, _, _ = cfg.mk_spec()
    krk, _, _ = cfg.rk_spec()
    krv, _, _ = cfg.rv_spec()
    idx = np.full((len(pairs), cfg.kc), -1, dtype=np.int32)
    out = np.zeros((len(pairs), cfg.D))
    for i, (b, h) in enumerate(pairs):
        q = _f(kq, C.rows(cfg, cfg.q_spec(), (np.array(b), np.array(h))))
        gk = _f(kgk, C.rows(cfg, cfg.gk_spec(), (np.array(b), np.array(h))))
        mk = _f(kmk, C.rows(cfg, cfg.mk_spec(), (np.array(b), np.array(h))))
        idx[i] = hgsa_select(q, mk, gk, cfg.group, cfg.km, cfg.kc)
        raw_pos, gist_ids = gsa_key_positions(idx[i], cfg.chunk, cfg.Nc, cfg.tail_len)
        bb, hh = np.full_like(raw_pos, b), np.full_like(raw_pos, h)
        rk = _f(krk, C.rows(cfg, cfg.rk_spec(), (bb, hh, raw_pos)))
        rv = _f(krv, C.rows(cfg, cfg.rv_spec(), (bb, hh, raw_pos)))
        gb, gh = np.full_like(gist_ids, b), np.full_like(gist_ids, h)
        gks = gk[gist_ids]
        gvs = _f(kgv, C.rows(cfg, cfg.gv_spec(), (gb, gh, gist_ids)))
        out[i] = gsa_attention(q, rk, rv, gks, gvs, cfg.scale)
    return idx, out
