"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each test swaps one oracle function for a copy with a plausible slip (a
dropped term, a wrong index, a reversed tie rule, ...) and checks that the
pin covering it raises.  The real oracle passes the same pins in
``test_oracle_pins.py``.
"""

import numpy as np
import pytest

import oracle
import oracle.attention as A
import oracle.driver as DRV
import oracle.gsa as GSA
import oracle.indexer as IDX
import oracle.topk as TK
from tests import oracle_pins as P


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


# ---- top-k ----

def _topk_highest_index_wins(scores, k, valid_len=None):
    s = np.asarray(scores)
    flipped = s[..., ::-1]
    n = s.shape[-1]
    if valid_len is not None and np.any(np.asarray(valid_len) != n):
        return TK.select_topk(scores, k, valid_len)
    r = TK.select_topk(flipped, k)
    out = np.where(r >= 0, n - 1 - r, -1)
    out = np.sort(np.where(out < 0, 1 << 30, out), axis=-1)
    return np.where(out == 1 << 30, -1, out)


def _topk_unsorted_output(scores, k, valid_len=None):
    s = np.asarray(scores)
    r = TK.select_topk(scores, k, valid_len)
    flat = r.reshape(-1, k).copy()
    sf = s.reshape(-1, s.shape[-1])
    for i in range(flat.shape[0]):
        sel = flat[i][flat[i] >= 0]
        order = np.argsort(-sf[i][sel].astype(np.float64), kind="stable")
        flat[i, :sel.size] = sel[order]
    return flat.reshape(r.shape)


def _topk_valid_off_by_one(scores, k, valid_len=None):
    n = np.asarray(scores).shape[-1]
    vl = n if valid_len is None else valid_len
    return TK.select_topk(scores, k, np.maximum(np.asarray(vl) - 1, 0))


@pytest.mark.parametrize("mutant", [_topk_highest_index_wins, _topk_unsorted_output,
                                    _topk_valid_off_by_one])
def test_topk_mutants_caught(mutant):
    _fails(P.pin_topk, mutant)


# ---- indexer ----

def _scores_first_head_only(qi, ki, n_heads):
    d = qi.shape[-1] // n_heads
    return IDX.index_scores(qi[..., :d], ki[..., :d], 1)


def _scores_features_reversed(qi, ki, n_heads):
    return IDX.index_scores(qi[..., ::-1].copy(), ki, n_heads)


@pytest.mark.parametrize("mutant", [_scores_first_head_only, _scores_features_reversed])
def test_indexer_mutants_caught(mutant):
    _fails(P.pin_index_scores, mutant)


# ---- attention ----

def _attn_no_scale(q, k, v, scale):
    return A.softmax_attention(q, k, v, 1.0)


def _attn_softmax_wrong_axis(q, k, v, scale):
    q = np.asarray(q, np.float64)
    z = q @ np.asarray(k, np.float64).T * scale
    e = np.exp(z - z.max(axis=0, keepdims=True))
    p = e / e.sum(axis=0, keepdims=True)
    return p @ np.asarray(v, np.float64)


def _gqa_wrong_map(q, k_sel, v_sel, scale):
    Hq, Hkv = q.shape[0], k_sel.shape[1]
    out = np.zeros((Hq, v_sel.shape[2]))
    for h in range(Hq):
        kvh = h % Hkv
        out[h] = A.softmax_attention(q[h:h + 1], k_sel[:, kvh], v_sel[:, kvh], scale)[0]
    return out


def test_attention_mutants_caught():
    _fails(P.pin_attention, _attn_no_scale, lambda q, k, v, s: _gqa_scaled(q, k, v, s, _attn_no_scale))
    _fails(P.pin_attention, _attn_softmax_wrong_axis,
           lambda q, k, v, s: _gqa_scaled(q, k, v, s, _attn_softmax_wrong_axis))
    _fails(P.pin_attention, A.softmax_attention, _gqa_wrong_map)


def _gqa_scaled(q, k_sel, v_sel, scale, attn):
    Hq, Hkv = q.shape[0], k_sel.shape[1]
    G = Hq // Hkv
    out = np.zeros((Hq, v_sel.shape[2]))
    for h in range(Hq):
        out[h] = attn(q[h:h + 1], k_sel[:, h // G], v_sel[:, h // G], scale)[0]
    return out


# ---- driver ----

def _step_no_sharing(cfg, batch=None, layers=None):
    layers = list(range(cfg.n_layers)) if layers is None else list(layers)
    idx, outs = {}, {}
    for l in layers:
        ix = DRV.decode_group(cfg, l // cfg.group, batch)   # indexer rerun for every layer
        idx[l // cfg.group] = ix
        outs[l] = DRV.decode_layers(cfg, l, ix, batch)
    return idx, outs


def test_driver_mutant_caught():
    _fails(P.pin_driver_sharing, _step_no_sharing, oracle)


def test_driver_group_mapping_mutant_caught(monkeypatch):
    real = DRV.decode_layers

    def wrong_group(cfg, layer, idx, batch=None, qrows=None):
        return real(cfg, layer, idx, batch, qrows)

    def step_wrong_group(cfg, batch=None, layers=None):
        layers = list(range(cfg.n_layers)) if layers is None else list(layers)
        groups = sorted({l // cfg.group for l in layers})
        idx = {g: DRV.decode_group(cfg, g, batch) for g in groups}
        outs = {l: real(cfg, l, idx[(l // cfg.group + 1) % len(groups)], batch) for l in layers}
        return idx, outs

    _fails(P.pin_driver_sharing, step_wrong_group, oracle)


def _owner_next_full(layer_full):
    """Shared layers read the upcoming Full layer's set instead of the last one."""
    full = list(layer_full)
    owner, g = [], sum(1 for f in full if f) - 1
    for l in range(len(full) - 1, -1, -1):
        owner.append(g)
        if full[l]:
            g -= 1
    owner = owner[::-1]
    n_full = sum(1 for f in full if f)
    return [min(o + (0 if full[l] else 1), n_full - 1) for l, o in enumerate(owner)]


def _owner_counts_from_one(layer_full):
    """Off by one: the first Full layer is numbered 1."""
    return [o + 1 for o in DRV.layer_owner(layer_full)]


def _step_pattern_ignored(cfg, layer_full, batch=None, layers=None):
    """Uses the evenly spaced groups whatever the pattern says."""
    return DRV.decode_step(cfg, batch, layers)


@pytest.mark.parametrize("owner", [_owner_next_full, _owner_counts_from_one])
def test_layer_owner_mutants_caught(owner):
    _fails(P.pin_layer_pattern, owner, DRV.decode_step_pattern, DRV.decode_step)


def test_pattern_ignored_mutant_caught():
    _fails(P.pin_layer_pattern, DRV.layer_owner, _step_pattern_ignored, DRV.decode_step)


# ---- prefill ----

def _prefill_excludes_self(cfg, g, rows):
    rows = np.asarray(list(rows), dtype=np.int64)
    from synth import configs as C
    qi = C.rows(cfg, cfg.qi_spec(g), (np.zeros_like(rows), rows))
    ki = C.rows(cfg, cfg.ki_spec(g), (np.array([0]),))[0]
    s = IDX.index_scores(qi[None], ki[None], cfg.H_idx)[0]
    return TK.select_topk(s, cfg.topk, rows)          # should be rows + 1


def test_prefill_mutant_caught():
    _fails(P.pin_prefill, _prefill_excludes_self, oracle.prefill_attention_rows)


# ---- GSA ----

def test_gsa_all_gists_mutant_caught(monkeypatch):
    real = GSA.gsa_key_positions

    def all_gists(chunk_idx, chunk, n_chunks, tail_len):
        raw, _ = real(chunk_idx, chunk, n_chunks, tail_len)
        return raw, np.arange(n_chunks, dtype=np.int64)

    monkeypatch.setattr(GSA, "gsa_key_positions", all_gists)
    _fails(P.pin_gsa_sg_sr, oracle.gsa_step)


def test_gsa_tail_dropped_mutant_caught(monkeypatch):
    real = GSA.gsa_key_positions

    def no_tail(chunk_idx, chunk, n_chunks, tail_len):
        return real(chunk_idx, chunk, n_chunks, 0)

    monkeypatch.setattr(GSA, "gsa_key_positions", no_tail)
    _fails(P.pin_gsa_dense, oracle.gsa_step)


def test_gsa_gists_dropped_mutant_caught(monkeypatch):
    real = GSA.gsa_key_positions

    def raw_only(chunk_idx, chunk, n_chunks, tail_len):
        raw, _ = real(chunk_idx, chunk, n_chunks, tail_len)
        return raw, np.zeros(0, dtype=np.int64)

    monkeypatch.setattr(GSA, "gsa_key_positions", raw_only)
    _fails(P.pin_gsa_dense, oracle.gsa_step)


# ---- sizes ----

def test_sizes_mutant_caught():
    _fails(P.pin_sizes, lambda L, H, D, n, b=2: L * H * D * b * n / 1024**3,   # K only, V dropped
           oracle.kv_bytes_per_token, oracle.scored_pairs)


# ---- hierarchical GSA ----

def _hgsa_meta_ties_high(q, mk, gk, group, km, kc):
    """Meta-gist ties go to the higher group."""
    nm = len(mk)
    ms = np.asarray(mk, float) @ np.asarray(q, float)
    order = np.lexsort((-np.arange(nm), -ms))
    groups = np.sort(order[:km])
    nc = len(gk)
    cand = np.concatenate([np.arange(g * group, min((g + 1) * group, nc)) for g in groups])
    s = np.asarray(gk, float)[cand] @ np.asarray(q, float)
    chosen = np.sort(cand[np.lexsort((cand, -s))[:kc]])
    out = np.full(kc, -1, dtype=np.int32)
    out[:chosen.size] = chosen
    return out


def _hgsa_flat(q, mk, gk, group, km, kc):
    """Ignores the groups: the flat top-kc over every chunk."""
    return GSA.gsa_select(q, gk, kc)


def _hgsa_drops_short_group(q, mk, gk, group, km, kc):
    """Leaves out the last group when it is short."""
    nc = len(gk)
    full = (nc // group) * group
    if full == 0:
        return GSA.hgsa_select(q, mk, gk, group, km, kc)
    return GSA.hgsa_select(q, np.asarray(mk)[: nc // group], np.asarray(gk)[:full], group, km, kc)


@pytest.mark.parametrize("mut", [_hgsa_meta_ties_high, _hgsa_flat, _hgsa_drops_short_group])
def test_hgsa_mutants_caught(mut):
    _fails(P.pin_hgsa_select, mut, GSA.gsa_select)


# ---- GSA prefill (gist mask) ----

_VISIBLE = GSA.gsa_prefill_visible


def _visible_mutant(kind):
    def vis_fn(n_chunks, chunk, n_sink=0):
        is_gist, seg, raw_pos, vis = _VISIBLE(n_chunks, chunk, n_sink)
        T = len(is_gist)
        t = np.arange(T)
        if kind == "full_causal":        # earlier raw tokens visible
            vis = t[None, :] <= t[:, None]
        elif kind == "non_causal":       # future tokens of the segment visible
            vis = vis | (seg[None, :] == seg[:, None])
        elif kind == "gist_not_self":    # a gist does not see itself
            vis = vis & ~(np.eye(T, dtype=bool) & is_gist[:, None])
        return is_gist, seg, raw_pos, vis
    return vis_fn


@pytest.mark.parametrize("kind", ["full_causal", "non_causal", "gist_not_self"])
def test_gsa_prefill_mask_mutants_caught(kind, monkeypatch):
    monkeypatch.setattr(GSA, "gsa_prefill_visible", _visible_mutant(kind))
    _fails(P.pin_gsa_prefill, GSA.gsa_prefill, GSA.gsa_prefill_visible)


# ---- one-row indexer scores ----

def _row_no_upcast(qi_row, ki):
    return np.asarray(ki) @ np.asarray(qi_row)          # int8 accumulation wraps


def _row_int16(qi_row, ki):
    return np.asarray(ki, np.int16) @ np.asarray(qi_row, np.int16)


def _row_drops_last_feature(qi_row, ki):
    return IDX.index_scores_row(np.asarray(qi_row)[:-1], np.asarray(ki)[:, :-1])


def _row_transposed_key(qi_row, ki):
    k = np.asarray(ki).astype(np.int64)
    return (k[:, ::-1] @ np.asarray(qi_row, np.int64))


@pytest.mark.parametrize("mutant", [_row_no_upcast, _row_int16, _row_drops_last_feature, _row_transposed_key])
def test_index_scores_row_mutants_caught(mutant):
    _fails(P.pin_index_scores_row, mutant)


# ---- hierarchical GSA step ----

def _hgsa_step_mutant(slip):
    """hgsa_step with one planted slip in its gathers."""
    from synth import configs as C

    def step(cfg, pairs=None):
        pairs = [(b, h) for b in range(cfg.B) for h in range(cfg.H)] if pairs is None else list(pairs)
        f = DRV._f
        kq, kgk, kgv, kmk = cfg.q_spec()[0], cfg.gk_spec()[0], cfg.gv_spec()[0], cfg.mk_spec()[0]
        krk, krv = cfg.rk_spec()[0], cfg.rv_spec()[0]
        idx = np.full((len(pairs), cfg.kc), -1, dtype=np.int32)
        out = np.zeros((len(pairs), cfg.D))
        for i, (b, h) in enumerate(pairs):
            q = f(kq, C.rows(cfg, cfg.q_spec(), (np.array(b), np.array(h))))
            gk = f(kgk, C.rows(cfg, cfg.gk_spec(), (np.array(b), np.array(h))))
            mk = f(kmk, C.rows(cfg, cfg.mk_spec(), (np.array(b), np.array(h))))
            idx[i] = GSA.hgsa_select(q, mk, gk, cfg.group, cfg.km, cfg.kc)
            tail = 0 if slip == "tail_dropped" else cfg.tail_len
            raw_pos, gist_ids = GSA.gsa_key_positions(idx[i], cfg.chunk, cfg.Nc, tail)
            bb, hh = np.full_like(raw_pos, b), np.full_like(raw_pos, h)
            rk = f(krk, C.rows(cfg, cfg.rk_spec(), (bb, hh, raw_pos)))
            rv = f(krv, C.rows(cfg, cfg.rv_spec(), (bb, hh, raw_pos)))
            gv_ids = np.minimum(gist_ids + 1, cfg.Nc - 1) if slip == "gist_value_shifted" else gist_ids
            gb, gh = np.full_like(gv_ids, b), np.full_like(gv_ids, h)
            if slip == "gist_key_from_meta":
                gks = mk[np.minimum(gist_ids // cfg.group, cfg.Nm - 1)]
            elif slip == "gist_key_shifted":
                gks = gk[np.maximum(gist_ids - 1, 0)]
            else:
                gks = gk[gist_ids]
            gvs = f(kgv, C.rows(cfg, cfg.gv_spec(), (gb, gh, gv_ids)))
            out[i] = GSA.gsa_attention(q, rk, rv, gks, gvs, cfg.scale)
        return idx, out
    return step


@pytest.mark.parametrize("slip", ["tail_dropped", "gist_value_shifted", "gist_key_from_meta", "gist_key_shifted"])
def test_hgsa_step_mutants_caught(slip):
    _fails(P.pin_hgsa_step, _hgsa_step_mutant(slip), oracle.gsa_step)


def test_hgsa_step_mutant_harness_is_faithful():
    """The mutant copy without a slip passes, so each caught slip is the slip."""
    P.pin_hgsa_step(_hgsa_step_mutant("none"), oracle.gsa_step)
