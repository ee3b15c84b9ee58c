"""Parity at the full workload sizes (MI355X), in the launch configuration the
benchmark times.

Every index set of every workload is compared with the oracle: all
(group, sequence) sets of the decode workloads, all (batch, head) pairs of the
GSA workloads, every row of the 64K causal index.  Attention outputs are
compared on sampled layers and rows (each costs the oracle a float64 softmax
over gathered rows).  Every index set is also checked for properties that hold
at any size (ascending, unique, in range, exactly min(k, valid) entries, one
buffer per group).  Inputs are generated in HBM by the device filler; the
oracle regenerates the rows it reads with the host generator (threads over
independent rows).
"""

import concurrent.futures as cf
import gc

import numpy as np
import pytest
import torch

import long_context_top_amd as lct
import oracle
import synth
import synth.device as sd
from synth import configs as C
from tests.gpu_util import announce, host

pytestmark = pytest.mark.gpu

ATOL = 1e-2


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def _check_index_rows(idx, L, k, valid):
    """Properties of an index row that hold at any size."""
    n = min(k, valid)
    assert np.all(idx[:n] >= 0) and np.all(idx[n:] == -1)
    assert np.all(np.diff(idx[:n]) > 0), "ascending and unique"
    assert idx[n - 1] < valid


def _pool(fn, items, workers=8):
    with cf.ThreadPoolExecutor(workers) as ex:
        return list(ex.map(fn, items))


def _oracle_set(cfg, g, b):
    """The oracle's index set of sequence b in group g (exact int64 scores of
    the one query row, chunks of keys regenerated in parallel)."""
    qi = C.rows(cfg, cfg.qi_spec(g), (np.array([b]), np.array([0])))[0]
    chunk = 1 << 17
    starts = list(range(0, cfg.L, chunk))

    def part(t0):
        t = np.arange(t0, min(cfg.L, t0 + chunk))
        return oracle.index_scores_row(qi, C.rows(cfg, cfg.ki_spec(g), (np.full_like(t, b), t)))

    s = np.concatenate(_pool(part, starts))
    return oracle.select_topk_threshold(s[None], cfg.topk)[0]


def _decode_full(cfg, sample_rows, sample_layers):
    announce(cfg.name)
    ng = cfg.n_groups
    qi = [sd.make(cfg, cfg.qi_spec(g)) for g in range(ng)]
    ki = [sd.make(cfg, cfg.ki_spec(g)) for g in range(ng)]
    q = [sd.make(cfg, cfg.q_spec(l)) for l in range(cfg.n_layers)]
    k = [sd.make(cfg, cfg.k_spec(l)) for l in range(cfg.n_layers)]
    v = [sd.make(cfg, cfg.v_spec(l)) for l in range(cfg.n_layers)]
    out = [torch.empty((cfg.B, cfg.Lq, cfg.Hq, cfg.D), dtype=torch.float32, device="cuda")
           for _ in range(cfg.n_layers)]
    idx_out = [torch.empty((cfg.B, cfg.Lq, cfg.topk), dtype=torch.int32, device="cuda") for _ in range(ng)]
    run = lct.GroupRun(qi, ki, q, k, v, out, cfg.topk, cfg.group, cfg.scale, idx_out=idx_out)
    run()
    torch.cuda.synchronize()
    seen = run.layer_index_addresses()
    for l in range(cfg.n_layers):
        assert seen[l] == idx_out[l // cfg.group].data_ptr(), "a layer read another group's buffer"
    idx = [host(t) for t in idx_out]
    for g in range(ng):
        for b in range(cfg.B):
            _check_index_rows(idx[g][b, 0], cfg.L, cfg.topk, cfg.L)
    sets = [(g, b) for g in range(ng) for b in range(cfg.B)]
    if cfg.L >= (1 << 20):
        wants = [_oracle_set(cfg, g, b) for g, b in sets]       # chunks in parallel inside
    else:
        wants = _pool(lambda gb: _oracle_set(cfg, *gb), sets)
    bad = [gb for gb, w in zip(sets, wants) if not np.array_equal(idx[gb[0]][gb[1], 0], w)]
    assert not bad, f"{len(bad)} of {len(sets)} (group, sequence) index sets differ: {bad[:6]}"
    print(f"  all {len(sets)} (group, sequence) index sets equal the oracle's", flush=True)
    for l in sample_layers:
        g = l // cfg.group
        ref = oracle.decode_layers(cfg, l, idx[g][sample_rows], batch=sample_rows)
        got = host(out[l])[sample_rows]
        err = np.abs(got - ref).max()
        assert err < ATOL, (l, err)
    del qi, ki, q, k, v, out, idx_out, run
    _free()


def test_decode_128k_b8_full_size():
    _decode_full(C.DECODE_128K, sample_rows=[0, 7], sample_layers=[0, 3, 27])


def test_decode_32k_b8_full_size():
    _decode_full(C.DECODE_32K, sample_rows=[3, 5], sample_layers=[9, 10])


def test_decode_1m_b1_full_size():
    _decode_full(C.DECODE_1M, sample_rows=[0], sample_layers=[1, 22])


def _check_all_pairs(cfg, step, got_idx, got):
    """Every (batch, head) pair: chunk set bit-exact, output within ATOL."""
    pairs = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    parts = _pool(lambda ps: step(cfg, ps), [pairs[i::16] for i in range(16)])
    ref_idx = np.zeros((len(pairs), cfg.kc), dtype=np.int64)
    ref_out = np.zeros((len(pairs), cfg.D))
    for i in range(16):
        ref_idx[i::16], ref_out[i::16] = parts[i]
    rows = [b * cfg.H + h for b, h in pairs]
    bad = [p for p, r, w in zip(pairs, rows, ref_idx) if not np.array_equal(got_idx[r], w)]
    assert not bad, f"{len(bad)} of {len(pairs)} chunk sets differ: {bad[:6]}"
    err = np.abs(got[rows] - ref_out).max()
    print(f"  all {len(pairs)} (batch, head) chunk sets equal the oracle's; max |out - oracle| = {err:.2e}",
          flush=True)
    assert err < ATOL


def test_gsa_128k_b16_full_size():
    cfg = C.GSA_128K
    announce(cfg.name)
    BH = cfg.B * cfg.H

    def mk(spec):
        t = sd.make(cfg, spec)
        return t.view((BH,) + tuple(t.shape[2:]))

    qv, gk, gv, rk, rv = (mk(cfg.q_spec()), mk(cfg.gk_spec()), mk(cfg.gv_spec()),
                          mk(cfg.rk_spec()), mk(cfg.rv_spec()))
    out, cidx = lct.gsa_decode(qv, gk, gv, rk, rv, cfg.kc, cfg.tail_len, cfg.scale)
    torch.cuda.synchronize()
    got_idx, got = host(cidx), host(out)
    for i in range(BH):
        _check_index_rows(got_idx[i], cfg.Nc, cfg.kc, cfg.Nc)
    _check_all_pairs(cfg, oracle.driver.gsa_step, got_idx, got)
    del qv, gk, gv, rk, rv, out, cidx
    _free()


def test_causal_prefill_64k_full_size():
    """One group (4 layers) of the 64K causal prefill; every index row against
    the oracle, attention outputs on sampled rows."""
    cfg = C.PREFILL_64K.with_(n_layers=4)
    announce(cfg.name)
    qi = [sd.make(cfg, cfg.qi_spec(0))]
    ki = [sd.make(cfg, cfg.ki_spec(0))]
    q = [sd.make(cfg, cfg.q_spec(l)) for l in range(4)]
    k = [sd.make(cfg, cfg.k_spec(l)) for l in range(4)]
    v = [sd.make(cfg, cfg.v_spec(l)) for l in range(4)]
    out = [torch.empty((1, cfg.L, cfg.Hq, cfg.D), dtype=torch.float32, device="cuda") for _ in range(4)]
    idx_out = [torch.empty((1, cfg.L, cfg.topk), dtype=torch.int32, device="cuda")]
    run = lct.GroupRun(qi, ki, q, k, v, out, cfg.topk, cfg.group, cfg.scale, causal=True,
                       idx_out=idx_out)
    run()
    torch.cuda.synchronize()
    idx = host(idx_out[0])[0]
    for r in range(0, cfg.L, 97):
        _check_index_rows(idx[r], cfg.L, cfg.topk, r + 1)
    below = np.arange(cfg.topk)  # rows whose set is every earlier position
    for r in below[::37]:
        assert np.array_equal(idx[r][: r + 1], np.arange(r + 1))
    # every row against the exact float32-product scorer + partition select
    # (both pinned against the int64 / sort definitions on the CPU)
    qh = C.rows(cfg, cfg.qi_spec(0), (np.array([0]),))[0]
    kh = C.rows(cfg, cfg.ki_spec(0), (np.array([0]),))[0]
    blocks = [np.arange(r0, min(cfg.L, r0 + 512)) for r0 in range(0, cfg.L, 512)]

    def block_bad(rb):
        s = oracle.index_scores_f32(qh[rb], kh[: rb[-1] + 1])
        w = oracle.select_topk_threshold(s, cfg.topk, rb + 1)
        return [int(r) for r, a, b in zip(rb, idx[rb], w) if not np.array_equal(a, b)]

    bad = [r for rs in _pool(block_bad, blocks) for r in rs]
    assert not bad, f"{len(bad)} of {cfg.L} rows differ from the oracle: {bad[:8]}"
    print(f"  all {cfg.L} index rows equal the oracle's", flush=True)
    rows = [2047, 2048, 2049, 33333, 65535]     # the int64 / sort definition on a few rows
    want = oracle.prefill_index_rows(cfg, 0, rows)
    for j, r in enumerate(rows):
        assert np.array_equal(idx[r], want[j]), r
    # every row below 2048 (nested prefixes and fast-growing overlaps: the
    # block-union path) and a spread of long rows (one to four 16384-position
    # segments, merged)
    sample = list(range(0, 2048)) + [2048, 4097, 16383, 16384, 33333, 65535] + list(range(2559, cfg.L, 1021))
    ref = oracle.prefill_attention_rows(cfg, 2, sample, idx[sample])
    assert np.abs(host(out[2])[0, sample] - ref).max() < ATOL
    del qi, ki, q, k, v, out, idx_out, run
    _free()


def test_hgsa_128k_b16_full_size():
    cfg = C.HGSA_128K
    announce(cfg.name)
    BH = cfg.B * cfg.H

    def mk(spec):
        t = sd.make(cfg, spec)
        return t.view((BH,) + tuple(t.shape[2:]))

    qv, mkeys, gk, gv, rk, rv = (mk(cfg.q_spec()), mk(cfg.mk_spec()), mk(cfg.gk_spec()), mk(cfg.gv_spec()),
                                 mk(cfg.rk_spec()), mk(cfg.rv_spec()))
    out, cidx = lct.hgsa_decode(qv, mkeys, gk, gv, rk, rv, cfg.group, cfg.km, cfg.kc, cfg.tail_len,
                                cfg.scale)
    torch.cuda.synchronize()
    got_idx, got = host(cidx), host(out)
    for i in range(BH):
        _check_index_rows(got_idx[i], cfg.Nc, cfg.kc, cfg.Nc)
    _check_all_pairs(cfg, oracle.driver.hgsa_step, got_idx, got)
    del qv, mkeys, gk, gv, rk, rv, out, cidx
    _free()


def test_gsa_prefill_128k_h16_full_size():
    cfg = C.GSA_PREFILL_128K
    announce(cfg.name)
    BH = cfg.B * cfg.H

    def mk(spec):
        t = sd.make(cfg, spec)
        return t.view((BH,) + tuple(t.shape[2:]))

    qr, qg, rk, rv, gk, gv = (mk(cfg.qr_spec()), mk(cfg.qg_spec()), mk(cfg.rk_spec()), mk(cfg.rv_spec()),
                              mk(cfg.gk_spec()), mk(cfg.gv_spec()))
    out_r, out_g = lct.gsa_prefill(qr, qg, rk, rv, gk, gv, cfg.scale)
    torch.cuda.synchronize()
    n_raw = cfg.Nc * cfg.chunk
    raw_rows = [0, 1, 15, 16, 17, 1000, 16383, 16384, 70001, n_raw - 17, n_raw - 1]
    gist_rows = [0, 1, 63, 64, 1000, 4097, cfg.Nc - 1]
    f = synth.as_float
    for h in (0, 9, 15):
        idx = (np.array(0), np.array(h))
        args = [f(spec[0], C.rows(cfg, spec, idx)) for spec in
                (cfg.qr_spec(), cfg.qg_spec(), cfg.rk_spec(), cfg.rv_spec(), cfg.gk_spec(), cfg.gv_spec())]
        args[2], args[3] = args[2][:n_raw], args[3][:n_raw]
        want_r, want_g = oracle.gsa_prefill_rows(*args, cfg.chunk, cfg.scale, raw_rows=raw_rows,
                                                 gist_rows=gist_rows)
        got_r = host(out_r[h, raw_rows])
        got_g = host(out_g[h, gist_rows])
        assert np.abs(got_r - want_r).max() < ATOL, h
        assert np.abs(got_g - want_g).max() < ATOL, h
    del qr, qg, rk, rv, gk, gv, out_r, out_g
    _free()
