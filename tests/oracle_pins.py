"""Pins for the CPU oracle: checks against facts that do not come from the oracle.

Each ``pin_*`` function takes the oracle functions it checks as arguments
and raises ``AssertionError`` on any mismatch, so the same pin can be run
against the real oracle (must pass) and against a copy with a planted
mistake (must fail, see ``test_oracle_mutants.py``).

What the pins compare against:

* closed forms and invariants of the indexer's bilinear score (one-hot
  keys pick out coordinates, the best key for a query has a closed-form
  score, additivity in the key),
* a rank-counting characterisation of top-k, brute force over tiny rows,
* ``torch.nn.functional.scaled_dot_product_attention`` (float64, CPU) for
  the dense special cases (k >= number of valid keys; causal prefill rows
  below k; GSA with every chunk chosen),
* numbers printed on the pages (``tests/golden/pages_worked_values.json``).
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_worked_values.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _sdpa(q, k, v, scale, causal=False, gqa=False):
    """Textbook attention via torch (float64, CPU). q[H, m, D], k/v[Hk, n, D]."""
    q = torch.as_tensor(np.asarray(q, np.float64))
    k = torch.as_tensor(np.asarray(k, np.float64))
    v = torch.as_tensor(np.asarray(v, np.float64))
    o = torch.nn.functional.scaled_dot_product_attention(
        q[None], k[None], v[None], scale=scale, is_causal=causal, enable_gqa=gqa)
    return o[0].numpy()


# --------------------------------------------------------------------------
# indexer
# --------------------------------------------------------------------------

def pin_index_scores(index_scores):
    rng = np.random.default_rng(11)
    B, Lq, H, d = 2, 3, 3, 5
    HD = H * d
    qi = rng.integers(-128, 128, size=(B, Lq, HD)).astype(np.int8)
    # keys 0..HD-1 are one-hot (+1 at feature t), key HD.. are per-head blocks,
    # then the best key per query row of batch 0, then random keys.
    keys = []
    for j in range(HD):
        e = np.zeros(HD, np.int64)
        e[j] = 1
        keys.append(e)
    for h in range(H):
        e = np.zeros(HD, np.int64)
        e[h * d:(h + 1) * d] = -3
        keys.append(e)
    n_fixed = len(keys)
    rand = rng.integers(-128, 128, size=(6, HD))
    L = n_fixed + Lq + rand.shape[0]
    ki = np.zeros((B, L, HD), np.int8)
    for b in range(B):
        ki[b, :n_fixed] = np.stack(keys)
        best = np.where(qi[b].astype(np.int64) >= 0, 127, -128)   # maximises every product
        ki[b, n_fixed:n_fixed + Lq] = best
        ki[b, n_fixed + Lq:] = rand
    s = np.asarray(index_scores(qi, ki, H), dtype=np.int64)
    assert s.shape == (B, Lq, L), s.shape
    q64 = qi.astype(np.int64)
    # one-hot keys pick out single query features
    assert np.array_equal(s[:, :, :HD], q64), "one-hot key must return that query coordinate"
    # a constant block on head h returns -3 x (sum of head h's query features)
    for h in range(H):
        exp = -3 * q64[:, :, h * d:(h + 1) * d].sum(-1)
        assert np.array_equal(s[:, :, HD + h], exp), "per-head block key"
    # the best key for row r scores sum_j max(127 q_j, -128 q_j)
    for r in range(Lq):
        exp = np.maximum(127 * q64[:, r], -128 * q64[:, r]).sum(-1)
        assert np.array_equal(s[:, r, n_fixed + r], exp), "closed-form maximum score"
        assert np.all(s[:, r, :] <= exp[:, None]), "no key may beat the maximising key"
    # additivity in the key: s(q, a + b) = s(q, a) + s(q, b) for keys that stay in int8
    a = rng.integers(-60, 60, size=(1, 4, HD)).astype(np.int8)
    b2 = rng.integers(-60, 60, size=(1, 4, HD)).astype(np.int8)
    ab = (a.astype(np.int64) + b2.astype(np.int64)).astype(np.int8)
    q1 = qi[:1]
    assert np.array_equal(index_scores(q1, ab, H),
                          np.asarray(index_scores(q1, a, H)) + np.asarray(index_scores(q1, b2, H)))


def pin_index_scores_row(index_scores_row):
    """One query row against a key matrix ``[L, HD]``.

    One-hot keys return single query coordinates; the maximising key has the
    closed-form score sum_j max(127 q_j, -128 q_j), here at the int8 extremes
    (a query of -128 everywhere and a key of -128 everywhere give
    256 x 16384 = 4194304, which wraps in any int8 or int16 accumulation);
    a pure-Python sum of products over the features agrees on random rows.
    """
    rng = np.random.default_rng(23)
    HD = 256
    for q in (np.full(HD, -128, np.int8), rng.integers(-128, 128, HD).astype(np.int8)):
        q64 = [int(x) for x in q]
        onehot = np.eye(HD, dtype=np.int8)[::17]                       # 16 one-hot keys
        best = np.where(q.astype(np.int64) >= 0, 127, -128).astype(np.int8)[None]
        worst = np.where(q.astype(np.int64) >= 0, -128, 127).astype(np.int8)[None]
        rand = rng.integers(-128, 128, size=(12, HD)).astype(np.int8)
        ki = np.concatenate([onehot, best, worst, rand])
        s = np.asarray(index_scores_row(q, ki))
        assert s.shape == (ki.shape[0],), s.shape
        assert [int(x) for x in s[:16]] == q64[::17], "one-hot key must return that query coordinate"
        want_best = sum(max(127 * x, -128 * x) for x in q64)
        assert int(s[16]) == want_best, ("closed-form maximum", int(s[16]), want_best)
        assert int(s[17]) == sum(min(127 * x, -128 * x) for x in q64), "closed-form minimum"
        assert all(int(v) <= want_best for v in s), "no key may beat the maximising key"
        for t in range(18, ki.shape[0]):
            assert int(s[t]) == sum(a * int(b) for a, b in zip(q64, ki[t])), ("brute force", t)
    assert int(np.asarray(index_scores_row(np.full(HD, -128, np.int8),
                                           np.full((1, HD), -128, np.int8)))[0]) == 4194304


def pin_index_scores_f32(index_scores_f32):
    """The float32 product path: exact integers on full-range int8 rows (a
    pure-Python sum of products), at the extremes (-128 everywhere: 4194304),
    and a refusal past the exactness bound (HD = 1024 could reach 2**24)."""
    rng = np.random.default_rng(31)
    HD = 256
    q = rng.integers(-128, 128, size=(5, HD)).astype(np.int8)
    k = rng.integers(-128, 128, size=(9, HD)).astype(np.int8)
    q[0] = -128
    k[0] = -128
    k[1] = 127
    s = np.asarray(index_scores_f32(q, k))
    assert s.shape == (5, 9) and s.dtype.kind == "i"
    for i in range(5):
        for t in range(9):
            assert int(s[i, t]) == sum(int(a) * int(b) for a, b in zip(q[i], k[t])), (i, t)
    assert int(s[0, 0]) == 4194304 and int(s[0, 1]) == -128 * 127 * 256
    try:
        index_scores_f32(np.zeros((1, 1024), np.int8), np.zeros((1, 1024), np.int8))
    except ValueError:
        pass
    else:
        raise AssertionError("HD = 1024 is past the float32 exactness bound")


# --------------------------------------------------------------------------
# top-k
# --------------------------------------------------------------------------

def _rank_select(row, k, nv):
    """Brute force: position i is chosen iff fewer than k valid positions precede it.

    j precedes i when s_j > s_i, or s_j == s_i and j < i.
    """
    chosen = []
    for i in range(nv):
        rank = 0
        for j in range(nv):
            if row[j] > row[i] or (row[j] == row[i] and j < i):
                rank += 1
        if rank < k:
            chosen.append(i)
    return chosen


def pin_topk(select_topk):
    rng = np.random.default_rng(5)
    alphabets = [[0], [0, 1], [-1, 0, 1], list(range(-4, 5)), list(range(-1000, 1000))]
    for alpha in alphabets:
        for n in (1, 2, 5, 17, 40):
            rows = rng.choice(alpha, size=(3, n)).astype(np.int64)
            for k in sorted({1, 2, n // 2 + 1, n, n + 3}):
                for nv in sorted({n, max(0, n - 3), 0, min(n, 1)}):
                    got = np.asarray(select_topk(rows, k, nv))
                    assert got.shape == (3, k)
                    for r in range(3):
                        exp = _rank_select(rows[r], k, nv)
                        want = np.full(k, -1)
                        want[:len(exp)] = exp
                        assert np.array_equal(got[r], want), (alpha[:3], n, k, nv, got[r], want)
    # per-row valid lengths
    rows = rng.integers(-3, 3, size=(6, 12))
    vl = np.array([0, 1, 5, 12, 7, 3])
    got = np.asarray(select_topk(rows, 4, vl))
    for r in range(6):
        exp = _rank_select(rows[r], 4, vl[r])
        assert list(got[r][got[r] >= 0]) == exp
    # floats, including signed zeros (equal values) and exact ties
    f = np.array([[0.0, -0.0, 1.5, 1.5, -2.0, 0.0, 3.25, -0.0]], dtype=np.float32)
    got = np.asarray(select_topk(f, 5))
    assert list(got[0]) == _rank_select(list(f[0]), 5, 8), got


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def pin_attention(softmax_attention, sparse_attention_gqa):
    rng = np.random.default_rng(7)
    n, D, Hq, Hkv = 37, 16, 8, 2
    q = rng.standard_normal((Hq, D))
    k = rng.standard_normal((n, Hkv, D))
    v = rng.standard_normal((n, Hkv, D))
    scale = 1.0 / math.sqrt(D)
    got = np.asarray(sparse_attention_gqa(q, k, v, scale))
    # all keys selected: the textbook formula (torch SDPA, GQA convention)
    ref = _sdpa(q[:, None, :], k.transpose(1, 0, 2), v.transpose(1, 0, 2), scale, gqa=True)[:, 0, :]
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), "k = n must equal dense attention"
    # key order does not matter
    perm = rng.permutation(n)
    got_p = np.asarray(sparse_attention_gqa(q, k[perm], v[perm], scale))
    assert np.allclose(got, got_p, rtol=1e-12, atol=1e-13), "permutation invariance"
    # V == 1 gives O == 1 (softmax rows sum to 1)
    ones = np.ones_like(v)
    assert np.allclose(sparse_attention_gqa(q, k, ones, scale), 1.0, atol=1e-13)
    # one-hot V columns return the attention probabilities themselves
    qq = rng.standard_normal((3, D))
    kk = rng.standard_normal((D, D))
    eye = np.eye(D)
    p = softmax_attention(qq, kk, eye, scale)
    ref_p = torch.softmax(torch.as_tensor(qq @ kk.T * scale), dim=-1).numpy()
    assert np.allclose(p, ref_p, rtol=1e-12, atol=1e-14)
    # extreme logits (the GSA gist case) stay finite and match the textbook path
    big = np.array([[700.0, -700.0, 699.0, 3.0]])
    kx = np.eye(4)
    vx = rng.standard_normal((4, 5))
    got_x = softmax_attention(big, kx, vx, 1.0)
    assert np.all(np.isfinite(got_x))
    ref_x = _sdpa(big[None], kx[None], vx[None], 1.0)[0]
    assert np.allclose(got_x, ref_x, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# driver: sharing, needles, dense equivalence end to end
# --------------------------------------------------------------------------

def small_decode_cfg(**kw):
    from synth import configs as C
    base = C.DecodeConfig("pin_decode", 77, B=2, Lq=3, L=300, n_layers=8, group=4, Hq=8,
                          Hkv=2, D=32, H_idx=2, d_idx=16, topk=24)
    return base.with_(**kw)


def pin_driver_sharing(decode_step, oracle_module):
    """One indexer call per group; every layer of a group sees the same set."""
    import oracle.driver as drv
    cfg = small_decode_cfg()
    calls = []
    real = drv.index_scores

    def counting(*a, **k):
        calls.append(1)
        return real(*a, **k)

    drv.index_scores = counting
    try:
        idx, outs = decode_step(cfg)
    finally:
        drv.index_scores = real
    n_groups = cfg.n_layers // cfg.group
    assert len(calls) == n_groups * cfg.B, (len(calls), n_groups, cfg.B)  # one call per (group, batch row)
    removed = 1.0 - n_groups / cfg.n_layers
    assert abs(removed - golden()["index_sharing"]["indexer_compute_removed_printed"]) < 1e-12
    assert len(idx) == n_groups
    assert not np.array_equal(idx[0], idx[1]), "different groups have different indexer inputs"
    # each layer's output is attention over its group's set
    for l, o in outs.items():
        ref = oracle_module.decode_layers(cfg, l, idx[l // cfg.group])
        assert np.allclose(o, ref, rtol=0, atol=0)


def pin_layer_pattern(layer_owner, decode_step_pattern, decode_step):
    """Free Full/Shared placement: each layer reads the set of the last Full
    layer at or before it (brute force over random patterns); every layer
    Full is per-layer routing; the evenly spaced pattern is the group driver;
    one indexer call per Full layer and batch row."""
    import oracle.driver as drv
    assert layer_owner([1, 0, 0, 0, 1, 0, 0, 0]) == [0, 0, 0, 0, 1, 1, 1, 1]
    assert layer_owner([1] * 6) == list(range(6))
    rng = np.random.default_rng(5)
    for _ in range(200):
        n = int(rng.integers(1, 20))
        full = [1] + [int(x) for x in rng.integers(0, 2, n - 1)]
        got = layer_owner(full)
        for l in range(n):
            last = max(j for j in range(l + 1) if full[j])
            assert got[l] == sum(full[:last]), (full, l)
    try:
        layer_owner([0, 1, 0])
    except ValueError:
        pass
    else:
        raise AssertionError("a leading Shared layer has no index to read")
    cfg = small_decode_cfg()
    idx_u, out_u = decode_step(cfg)
    idx_p, out_p = decode_step_pattern(cfg, [1, 0, 0, 0, 1, 0, 0, 0])
    assert sorted(idx_p) == sorted(idx_u)
    for g in idx_u:
        assert np.array_equal(idx_p[g], idx_u[g])
    for l in out_u:
        assert np.array_equal(out_p[l], out_u[l])
    pattern = [1, 1, 0, 0, 0, 1, 0, 1]
    calls = []
    real = drv.index_scores

    def counting(*a, **k):
        calls.append(1)
        return real(*a, **k)

    drv.index_scores = counting
    try:
        idx, outs = decode_step_pattern(cfg, pattern)
    finally:
        drv.index_scores = real
    assert len(calls) == sum(pattern) * cfg.B
    assert len(idx) == sum(pattern)
    # layers 1-4 read Full layer 1's set, layer 5-6 Full layer 2's, layer 7 its own
    for l, g in ((1, 1), (4, 1), (5, 2), (6, 2), (7, 3)):
        assert np.array_equal(outs[l], drv.decode_layers(cfg, l, drv.decode_group(cfg, g)))
    assert not np.array_equal(idx[1], idx[2])


def pin_dense_when_k_covers(decode_step):
    """k >= L: sparse decode equals dense softmax(QK^T/sqrt(d))V over the whole cache."""
    import synth
    from synth import configs as C
    cfg = small_decode_cfg(L=40, topk=64, n_layers=4)
    idx, outs = decode_step(cfg, layers=[1, 2])
    for g, ix in idx.items():
        want = np.full(cfg.topk, -1)
        want[:cfg.L] = np.arange(cfg.L)
        assert np.all(ix == want), "k >= L must select every position"
    for l in (1, 2):
        q = synth.as_float(synth.BF16N, C.make(cfg, cfg.q_spec(l)))
        k = synth.as_float(synth.BF16N, C.make(cfg, cfg.k_spec(l)))
        v = synth.as_float(synth.BF16N, C.make(cfg, cfg.v_spec(l)))
        for b in range(cfg.B):
            ref = _sdpa(q[b].transpose(1, 0, 2), k[b].transpose(1, 0, 2), v[b].transpose(1, 0, 2),
                        cfg.scale, gqa=True).transpose(1, 0, 2)
            assert np.allclose(outs[l][b], ref, rtol=1e-12, atol=1e-12), "dense equivalence"


def pin_needles(index_scores, select_topk):
    """Keys planted with the closed-form maximum score are always chosen."""
    rng = np.random.default_rng(3)
    L, HD, k = 4096, 64, 32
    qi = rng.integers(-8, 8, size=(1, 1, HD)).astype(np.int8)
    ki = rng.integers(-8, 8, size=(1, L, HD)).astype(np.int8)
    needles = np.sort(rng.choice(L, size=9, replace=False))
    ki[0, needles] = np.where(qi[0, 0] >= 0, 7, -8).astype(np.int8)
    s = index_scores(qi, ki, 1)
    sel = np.asarray(select_topk(np.asarray(s)[0], k, L))[0]
    assert set(needles.tolist()) <= set(sel.tolist()), (needles, sel)
    best = int(np.maximum(7 * qi[0, 0].astype(np.int64), -8 * qi[0, 0].astype(np.int64)).sum())
    assert np.all(np.asarray(s)[0, 0, needles] == best)


def pin_prefill(prefill_index_rows, prefill_attention_rows):
    """Causal prefill: rows below k see every earlier position (dense causal)."""
    import synth
    from synth import configs as C
    cfg = C.DecodeConfig("pin_prefill", 91, B=1, Lq=96, L=96, n_layers=4, group=4, Hq=4, Hkv=2,
                         D=16, H_idx=2, d_idx=8, topk=32, causal=True)
    rows = list(range(0, 96, 5)) + [31, 32, 95]
    idx = np.asarray(prefill_index_rows(cfg, 0, rows))
    for j, r in enumerate(rows):
        sel = idx[j][idx[j] >= 0]
        assert sel.size == min(cfg.topk, r + 1)
        assert np.all(sel <= r), "causal: no position after the query"
        if r < cfg.topk:
            assert np.array_equal(sel, np.arange(r + 1))
    out = np.asarray(prefill_attention_rows(cfg, 2, rows, idx))
    q = synth.as_float(synth.BF16N, C.make(cfg, cfg.q_spec(2)))[0]
    k = synth.as_float(synth.BF16N, C.make(cfg, cfg.k_spec(2)))[0]
    v = synth.as_float(synth.BF16N, C.make(cfg, cfg.v_spec(2)))[0]
    ref = _sdpa(q.transpose(1, 0, 2), k.transpose(1, 0, 2), v.transpose(1, 0, 2), cfg.scale,
                causal=True, gqa=True).transpose(1, 0, 2)
    for j, r in enumerate(rows):
        if r < cfg.topk:
            assert np.allclose(out[j], ref[r], rtol=1e-12, atol=1e-12), r


# --------------------------------------------------------------------------
# GSA
# --------------------------------------------------------------------------

def small_gsa_cfg(**kw):
    from synth import configs as C
    base = C.GsaConfig("pin_gsa", 55, B=2, H=3, D=16, Nc=12, chunk=16, kc=4, tail_len=1)
    return base.with_(**kw)


def _gsa_inputs(cfg):
    import synth
    from synth import configs as C
    f = synth.as_float
    return (f(cfg.q_spec()[0], C.make(cfg, cfg.q_spec())), f(cfg.gk_spec()[0], C.make(cfg, cfg.gk_spec())),
            f(synth.BF16N, C.make(cfg, cfg.gv_spec())), f(synth.BF16N, C.make(cfg, cfg.rk_spec())),
            f(synth.BF16N, C.make(cfg, cfg.rv_spec())))


def pin_gsa_dense(gsa_step):
    """Every chunk chosen: attention over all raw tokens, all gists and the tail."""
    for tail in (0, 1, 5, 15):
        cfg = small_gsa_cfg(kc=12, tail_len=tail)
        q, gk, gv, rk, rv = _gsa_inputs(cfg)
        idx, out = gsa_step(cfg)
        n_raw = cfg.Nc * cfg.chunk + tail
        for i, (b, h) in enumerate([(b, h) for b in range(cfg.B) for h in range(cfg.H)]):
            assert np.array_equal(idx[i], np.arange(cfg.Nc))
            keys = np.concatenate([rk[b, h, :n_raw], gk[b, h]])
            vals = np.concatenate([rv[b, h, :n_raw], gv[b, h]])
            ref = _sdpa(q[b, h][None, None], keys[None], vals[None], cfg.scale)[0, 0]
            assert np.allclose(out[i], ref, rtol=1e-12, atol=1e-12), (tail, b, h)


def pin_gsa_sg_sr(gsa_step):
    """One chunk chosen: its raw tokens + its own gist + the tail, nothing else.

    Query and gist keys are overridden with small ternary values so that
    every gist carries real attention weight (with the workload's [-8, 7]
    integers the chosen gist's logit dwarfs all others and a wrong key set
    would be invisible).  The planted gist equals the query, so its score
    ||q||^2 is the unique maximum.  The expected key list is written out from
    the pages' rule: selected gist and raw tokens kept, unselected gists
    dropped, tail always kept.
    """
    import synth
    cfg = small_gsa_cfg(kc=1, tail_len=3)
    _, _, gv, rk, rv = _gsa_inputs(cfg)
    rng = np.random.default_rng(8)
    q2 = rng.choice([-1.0, 1.0], size=(cfg.B, cfg.H, cfg.D))
    gk2 = rng.choice([-1.0, 0.0, 1.0], size=(cfg.B, cfg.H, cfg.Nc, cfg.D))
    planted = 7
    gk2[:, :, planted] = q2

    import oracle.driver as drv
    real_rows = drv.C.rows
    override = {cfg.q_spec(): q2, cfg.gk_spec(): gk2}

    def rows_patched(c, spec, lead):
        if spec in override:
            idxs = np.broadcast_arrays(*[np.asarray(a) for a in lead])
            return synth.f32_to_bf16_bits(override[spec][tuple(idxs)].astype(np.float32))
        return real_rows(c, spec, lead)

    drv.C.rows = rows_patched
    try:
        idx, out = gsa_step(cfg)
    finally:
        drv.C.rows = real_rows
    for i, (b, h) in enumerate([(b, h) for b in range(cfg.B) for h in range(cfg.H)]):
        assert list(idx[i]) == [planted]
        raw_pos = list(range(planted * 16, planted * 16 + 16)) + [cfg.Nc * 16 + t for t in range(3)]
        keys = np.concatenate([rk[b, h, raw_pos], gk2[b, h, planted][None]])
        vals = np.concatenate([rv[b, h, raw_pos], gv[b, h, planted][None]])
        ref = _sdpa(q2[b, h][None, None], keys[None], vals[None], cfg.scale)[0, 0]
        assert np.allclose(out[i], ref, rtol=1e-12, atol=1e-12), (b, h)


# --------------------------------------------------------------------------
# sizes
# --------------------------------------------------------------------------

def pin_sizes(kv_cache_gib, kv_bytes_per_token, scored_pairs):
    g = golden()
    kv = g["kv_cache_gib"]
    for tok, printed in kv["printed_gib_1dp"].items():
        v = kv_cache_gib(kv["n_layers"], kv["kv_heads"], kv["head_dim"], int(tok), kv["bytes_per"])
        assert f"{v:.1f}" == printed, (tok, v, printed)
    per_tok = kv_bytes_per_token(28, 4, 128, 2)
    assert per_tok == 56 * 1024 and round(per_tok / 1024) == g["kv_per_token_kib"]["printed_kib_approx"]
    # 2**20 tokens with this geometry is exactly 56 GiB
    assert kv_cache_gib(28, 4, 128, 1 << 20) == 56.0
    sp = g["scored_pairs_at_1M"]
    n = sp["n_tok"]
    full = scored_pairs(n)
    assert full == sp["full_pairs_printed"]
    for key in ("sliding_window", "topk"):
        e = sp[key]
        p = scored_pairs(n, e["per_query"])
        assert abs(p - e["pairs_printed"]) / e["pairs_printed"] < 0.01, (key, p)
        assert f"1/{round(full / p)}" == e["fraction_printed"], (key, full / p)
    gc = g["gist_count_at_1M"]
    n_gists = gc["n_tok"] // gc["chunk"]
    assert gc["printed_lower_bound"] <= n_gists <= gc["printed_upper_bound"]


def pin_hgsa_select(hgsa_select, gsa_select):
    """Coarse-to-fine routing: a hand-worked case with ties; brute force by
    rank counting on small integer inputs (many ties, a short last group);
    choosing every group reduces to the flat top-kc over all chunks."""
    # hand-worked: D = 2, q = (1, 0), so a key's score is its first feature.
    # Groups of 2 over 6 chunks: meta scores 5, 9, 9 (groups 1 and 2 tie).
    q = np.array([1.0, 0.0])
    mk = np.array([[5, 0], [9, 0], [9, 0]], dtype=float)
    gk = np.array([[8, 0], [8, 0], [4, 0], [4, 0], [7, 0], [1, 0]], dtype=float)
    assert list(hgsa_select(q, mk, gk, 2, 1, 1)) == [2]           # group 1 (tie -> lower), chunk 2 (tie)
    assert list(hgsa_select(q, mk, gk, 2, 2, 2)) == [2, 4]        # chunks 2..5 score 4 4 7 1
    assert list(hgsa_select(q, mk, gk, 2, 2, 5)) == [2, 3, 4, 5, -1]
    assert list(hgsa_select(q, mk, gk, 2, 3, 2)) == [0, 1]        # every group: the flat choice
    rng = np.random.default_rng(11)
    for trial in range(300):
        nc = int(rng.integers(1, 40))
        group = int(rng.integers(1, 9))
        nm = -(-nc // group)
        km = int(rng.integers(1, nm + 2))
        kc = int(rng.integers(1, 12))
        d = 3
        q = rng.integers(-2, 3, d).astype(float)
        mk = rng.integers(-2, 3, (nm, d)).astype(float)
        gk = rng.integers(-2, 3, (nc, d)).astype(float)
        got = hgsa_select(q, mk, gk, group, km, kc)
        ms, gs = mk @ q, gk @ q
        gsel = [g for g in range(nm)
                if sum(1 for h in range(nm) if ms[h] > ms[g] or (ms[h] == ms[g] and h < g)) < km]
        cand = [c for c in range(nc) if c // group in gsel]
        want = sorted(c for c in cand
                      if sum(1 for e in cand if gs[e] > gs[c] or (gs[e] == gs[c] and e < c)) < kc)
        want = want + [-1] * (kc - len(want))
        assert list(got) == want, (trial, nc, group, km, kc)
        if km >= nm:
            assert list(got) == list(gsa_select(q, gk, kc)), trial


def small_hgsa_cfg(**kw):
    base = small_gsa_cfg(Nc=14, kc=3, group=4, km=2)   # meta-gists 0..3, the last one short
    return base.with_(**kw)


def pin_hgsa_step(hgsa_step, gsa_step):
    """Hierarchical GSA decode step (routing, then the gathers and attention).

    (a) With every meta-gist kept (km = number of groups) the coarse step
    chooses nothing away, so the step equals the flat GSA step, which has its
    own pins (dense equivalence, the SG+SR key set).
    (b) A planted case written out from the pages' rule: query and keys are
    overridden with ternary values; meta-gist ``gp`` and gist ``planted`` (in
    group ``gp``) equal the query, so their scores ||q||^2 are the unique
    maxima; with km = kc = 1 the step must unfold exactly chunk ``planted``:
    its 16 raw rows, its own gist (key and value), and the tail, and nothing
    else (compared with textbook attention over that key list).
    """
    import synth
    for tail in (0, 2):
        cfg = small_hgsa_cfg(km=4, tail_len=tail)
        assert cfg.km >= cfg.Nm
        ih, oh = hgsa_step(cfg)
        ig, og = gsa_step(cfg)
        assert np.array_equal(np.asarray(ih), np.asarray(ig)), "all groups kept: flat selection"
        assert np.allclose(oh, og, rtol=1e-12, atol=1e-12), "all groups kept: flat attention"

    cfg = small_hgsa_cfg(km=1, kc=1, tail_len=3)
    _, _, gv, rk, rv = _gsa_inputs(cfg)
    rng = np.random.default_rng(19)
    q2 = rng.choice([-1.0, 1.0], size=(cfg.B, cfg.H, cfg.D))
    gk2 = rng.choice([-1.0, 0.0, 1.0], size=(cfg.B, cfg.H, cfg.Nc, cfg.D))
    mk2 = rng.choice([-1.0, 0.0, 1.0], size=(cfg.B, cfg.H, cfg.Nm, cfg.D))
    gp, planted = 2, 10                      # chunk 10 lies in group 2 (chunks 8..11)
    assert planted // cfg.group == gp
    mk2[:, :, gp] = q2
    gk2[:, :, planted] = q2
    gk2[:, :, 1] = q2                        # an equal gist outside the chosen group is not seen

    import oracle.driver as drv
    real_rows = drv.C.rows
    override = {cfg.q_spec(): q2, cfg.gk_spec(): gk2, cfg.mk_spec(): mk2}

    def rows_patched(c, spec, lead):
        if spec in override:
            idxs = np.broadcast_arrays(*[np.asarray(a) for a in lead])
            return synth.f32_to_bf16_bits(override[spec][tuple(idxs)].astype(np.float32))
        return real_rows(c, spec, lead)

    drv.C.rows = rows_patched
    try:
        idx, out = hgsa_step(cfg)
    finally:
        drv.C.rows = real_rows
    for i, (b, h) in enumerate([(b, h) for b in range(cfg.B) for h in range(cfg.H)]):
        assert list(idx[i]) == [planted], (b, h, list(idx[i]))
        raw_pos = list(range(planted * 16, planted * 16 + 16)) + [cfg.Nc * 16 + t for t in range(3)]
        keys = np.concatenate([rk[b, h, raw_pos], gk2[b, h, planted][None]])
        vals = np.concatenate([rv[b, h, raw_pos], gv[b, h, planted][None]])
        ref = _sdpa(q2[b, h][None, None], keys[None], vals[None], cfg.scale)[0, 0]
        assert np.allclose(out[i], ref, rtol=1e-12, atol=1e-12), (b, h)


def _softmax_rows(q, k, v, scale):
    """Direct softmax-weighted sum for one query (explicit exponentials)."""
    z = (k @ q) * scale
    w = np.exp(z - z.max())
    return (w / w.sum()) @ v


def pin_gsa_prefill(gsa_prefill, gsa_prefill_visible):
    """The gist mask: one segment is plain causal attention; the gists-first
    key order (the prefill kernel's permutation) gives the same outputs;
    earlier segments' raw tokens and a raw token's own gist are invisible,
    earlier gists visible; anchors are seen by every later token; the
    visible counts per row have closed forms."""
    rng = np.random.default_rng(17)
    D, chunk, nc, scale = 8, 4, 5, 0.3
    qr, kr, vr = (rng.standard_normal((nc * chunk, D)) for _ in range(3))
    qg, kg, vg = (rng.standard_normal((nc, D)) for _ in range(3))
    out_r, out_g = gsa_prefill(qr, qg, kr, vr, kg, vg, chunk, scale)
    # one segment: causal attention over its raw tokens; its gist sees them all and itself
    r1, g1 = gsa_prefill(qr[:chunk], qg[:1], kr[:chunk], vr[:chunk], kg[:1], vg[:1], chunk, scale)
    for i in range(chunk):
        assert np.allclose(r1[i], _softmax_rows(qr[i], kr[:i + 1], vr[:i + 1], scale), atol=1e-12)
    assert np.allclose(g1[0], _softmax_rows(qg[0], np.vstack([kr[:chunk], kg[:1]]),
                                            np.vstack([vr[:chunk], vg[:1]]), scale), atol=1e-12)
    # gists first, then the segment's own raw tokens
    for c in range(nc):
        for i in range(chunk):
            t = c * chunk + i
            keys = np.vstack([kg[:c], kr[c * chunk:t + 1]])
            vals = np.vstack([vg[:c], vr[c * chunk:t + 1]])
            assert np.allclose(out_r[t], _softmax_rows(qr[t], keys, vals, scale), atol=1e-12), (c, i)
        keys = np.vstack([kg[:c + 1], kr[c * chunk:(c + 1) * chunk]])
        vals = np.vstack([vg[:c + 1], vr[c * chunk:(c + 1) * chunk]])
        assert np.allclose(out_g[c], _softmax_rows(qg[c], keys, vals, scale), atol=1e-12), c
    # earlier raw tokens invisible, earlier gists visible, own gist invisible to raw tokens
    vr2 = vr.copy()
    vr2[:chunk] += 1.0
    o2, _ = gsa_prefill(qr, qg, kr, vr2, kg, vg, chunk, scale)
    assert np.allclose(o2[chunk:], out_r[chunk:]) and not np.allclose(o2[:chunk], out_r[:chunk])
    vg2 = vg.copy()
    vg2[2] += 1.0
    o3, _ = gsa_prefill(qr, qg, kr, vr, kg, vg2, chunk, scale)
    assert np.allclose(o3[:3 * chunk], out_r[:3 * chunk]) and not np.allclose(o3[3 * chunk:], out_r[3 * chunk:])
    # anchors: the first two raw positions are seen by every later token, not by earlier ones
    vr3 = vr.copy()
    vr3[1] += 1.0
    o4, _ = gsa_prefill(qr, qg, kr, vr3, kg, vg, chunk, scale, n_sink=2)
    o4b, _ = gsa_prefill(qr, qg, kr, vr, kg, vg, chunk, scale, n_sink=2)
    assert np.allclose(o4[0], o4b[0]) and not np.allclose(o4[3 * chunk], o4b[3 * chunk])
    # the per-row form (visible keys listed row by row) agrees with the mask form, anchors too
    import oracle.gsa as G
    for ns in (0, 3):
        fr, fg = gsa_prefill(qr, qg, kr, vr, kg, vg, chunk, scale, n_sink=ns)
        rr, rg = G.gsa_prefill_rows(qr, qg, kr, vr, kg, vg, chunk, scale, raw_rows=range(nc * chunk),
                                    gist_rows=range(nc), n_sink=ns)
        assert np.allclose(rr, fr, atol=1e-12) and np.allclose(rg, fg, atol=1e-12), ns
    # visible keys per row: raw (c, i) sees c gists and i + 1 raw tokens; gist c sees c + 1 gists and chunk raw
    is_gist, seg, raw_pos, vis = gsa_prefill_visible(nc, chunk)
    for t in range(len(is_gist)):
        c = seg[t]
        want = c + 1 + chunk if is_gist[t] else c + (raw_pos[t] - c * chunk) + 1
        assert vis[t].sum() == want, t
