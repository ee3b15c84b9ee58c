"""Layer-group driver parity (indexer once per group, shared index, sparse
attention for every layer) against the CPU oracle on small workloads (MI355X)."""

import numpy as np
import pytest
import torch

import long_context_top_amd as lct
import oracle
import synth.device as sd
from synth import configs as C
from tests.gpu_util import announce, dev_i32, host

pytestmark = pytest.mark.gpu

ATOL = 1e-2


def _inputs(cfg):
    ng = cfg.n_groups
    qi = [sd.make(cfg, cfg.qi_spec(g)) for g in range(ng)]
    ki = [sd.make(cfg, cfg.ki_spec(g)) for g in range(ng)]
    q = [sd.make(cfg, cfg.q_spec(l)) for l in range(cfg.n_layers)]
    k = [sd.make(cfg, cfg.k_spec(l)) for l in range(cfg.n_layers)]
    v = [sd.make(cfg, cfg.v_spec(l)) for l in range(cfg.n_layers)]
    return qi, ki, q, k, v


def _run(cfg, valid_len=None):
    qi, ki, q, k, v = _inputs(cfg)
    idx_out = [torch.full((cfg.B, cfg.Lq, cfg.topk), -7, dtype=torch.int32, device="cuda")
               for _ in range(cfg.n_groups)]
    vl = None if valid_len is None else dev_i32(np.asarray(valid_len))
    out, run = lct.group_run(qi, ki, q, k, v, cfg.topk, cfg.group, cfg.scale, causal=cfg.causal,
                             valid_len=vl, idx_out=idx_out)
    torch.cuda.synchronize()
    return [host(t) for t in idx_out], [host(t) for t in out], run


def test_tiny_config_end_to_end():
    cfg = C.TINY
    announce(cfg.name)
    idx, out, run = _run(cfg)
    ref_idx, ref_out = oracle.decode_step(cfg)
    assert np.array_equal(idx[0], ref_idx[0])
    for l in range(cfg.n_layers):
        assert np.abs(out[l] - ref_out[l]).max() < ATOL, l
    seen = run.layer_index_addresses()
    assert len(set(seen)) == 1  # one group: every layer read the same buffer


def test_tiny_config_dense_when_k_is_context():
    """k = L = 2048: every position is chosen, sparse attention is dense attention."""
    cfg = C.TINY.with_(name="tiny_dense", topk=2048)
    announce(cfg.name)
    idx, out, _ = _run(cfg)
    assert np.array_equal(idx[0][0, 0], np.arange(2048))
    _, ref_out = oracle.decode_step(cfg)
    for l in range(cfg.n_layers):
        assert np.abs(out[l] - ref_out[l]).max() < ATOL


@pytest.mark.parametrize("L,valid", [(5000, [5000, 100, 4000]), (40000, [40000, 2047, 33333])])
def test_decode_ragged_valid_len(L, valid):
    cfg = C.DecodeConfig("ragged", 4242, B=3, Lq=2, L=L, n_layers=8, group=4, Hq=16, Hkv=2, D=128,
                         H_idx=4, d_idx=64, topk=512)
    announce(f"{cfg.name} L={L}")
    idx, out, run = _run(cfg, valid)
    for g in range(cfg.n_groups):
        for b in range(cfg.B):
            from synth import configs as CC
            qi = CC.rows(cfg, cfg.qi_spec(g), (np.array([b]),))
            ki = CC.rows(cfg, cfg.ki_spec(g), (np.array([b]),))
            s = oracle.index_scores(qi, ki, cfg.H_idx)[0]
            want = oracle.select_topk(s, cfg.topk, valid[b])
            assert np.array_equal(idx[g][b], want), (g, b)
    for l in (0, 5):
        ref = oracle.decode_layers(cfg, l, idx[l // cfg.group])
        assert np.abs(out[l] - ref).max() < ATOL, l
    seen = run.layer_index_addresses()
    assert seen[0] == seen[3] and seen[4] == seen[7] and seen[0] != seen[4]


def test_causal_prefill_small():
    cfg = C.DecodeConfig("prefill_small", 5151, B=1, Lq=700, L=700, n_layers=4, group=4, Hq=8, Hkv=2,
                         D=128, H_idx=4, d_idx=64, topk=64, causal=True)
    announce(cfg.name)
    idx, out, _ = _run(cfg)
    rows = list(range(cfg.L))
    want = oracle.prefill_index_rows(cfg, 0, rows)
    assert np.array_equal(idx[0][0], want)
    sample = [0, 1, 5, 63, 64, 65, 300, 699]
    ref = oracle.prefill_attention_rows(cfg, 3, sample, want[sample])
    assert np.abs(out[3][0, sample] - ref).max() < ATOL


def test_causal_prefill_graph_capture():
    """Causal group_run (index with rows for the whole-row select, then
    attention) captured in a HIP graph and replayed three times with eager
    work in between; index sets and sampled outputs checked each time."""
    cfg = C.DecodeConfig("prefill_graph", 5353, B=1, Lq=1300, L=1300, n_layers=4, group=4, Hq=8, Hkv=2,
                         D=128, H_idx=4, d_idx=64, topk=64, causal=True)
    announce(cfg.name)
    qi, ki, q, k, v = _inputs(cfg)
    qi[0][0, 3::4] = 0                       # all-zero rows: every score equal
    idx_out = [torch.full((1, cfg.L, cfg.topk), -7, dtype=torch.int32, device="cuda")]
    out = [torch.empty(t.shape, dtype=torch.float32, device="cuda") for t in q]
    run = lct.GroupRun(qi, ki, q, k, v, out, cfg.topk, cfg.group, cfg.scale, causal=True, idx_out=idx_out)
    run()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.current_stream().wait_stream(s)
    qh = host(qi[0])[0]
    kh = host(ki[0])[0]
    sc = oracle.index_scores(qh[None], kh[None], cfg.H_idx)[0]
    want = oracle.select_topk(sc, cfg.topk, np.arange(cfg.L) + 1)
    sample = [0, 3, 63, 64, 67, 700, 1299]
    ref = oracle.prefill_attention_rows(cfg, 2, sample, want[sample])
    for rep in range(3):
        idx_out[0].fill_(-7)
        out[2].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(idx_out[0])[0], want), rep
        assert np.abs(host(out[2])[0, sample] - ref).max() < ATOL, rep


def _run_pattern(cfg, layer_full):
    n_full = sum(layer_full)
    qi = [sd.make(cfg, cfg.qi_spec(g)) for g in range(n_full)]
    ki = [sd.make(cfg, cfg.ki_spec(g)) for g in range(n_full)]
    _, _, q, k, v = _inputs(cfg)
    idx_out = [torch.full((cfg.B, cfg.Lq, cfg.topk), -7, dtype=torch.int32, device="cuda")
               for _ in range(n_full)]
    out, run = lct.group_run(qi, ki, q, k, v, cfg.topk, cfg.group, cfg.scale, causal=cfg.causal,
                             idx_out=idx_out, layer_full=layer_full)
    torch.cuda.synchronize()
    return idx_out, [host(t) for t in idx_out], [host(t) for t in out], run


def test_decode_free_full_shared_pattern():
    """Full layers at uneven places (IndexCache greedy-search patterns): each
    layer attends over the set of the last Full layer at or before it."""
    pattern = [1, 0, 0, 1, 0, 1, 1, 0, 0, 0]
    cfg = C.DecodeConfig("pattern", 6060, B=2, Lq=2, L=5000, n_layers=len(pattern), group=1,
                         Hq=8, Hkv=2, D=128, H_idx=4, d_idx=64, topk=256)
    announce(f"{cfg.name} {pattern}")
    bufs, idx, out, run = _run_pattern(cfg, pattern)
    owner = oracle.layer_owner(pattern)
    for g in range(sum(pattern)):
        assert np.array_equal(idx[g], oracle.decode_group(cfg, g)), g
    for l in range(cfg.n_layers):
        ref = oracle.decode_layers(cfg, l, idx[owner[l]])
        assert np.abs(out[l] - ref).max() < ATOL, l
    seen = run.layer_index_addresses()
    assert seen == [bufs[owner[l]].data_ptr() for l in range(cfg.n_layers)]


def test_causal_prefill_free_pattern():
    pattern = [1, 1, 0]
    cfg = C.DecodeConfig("prefill_pattern", 7171, B=1, Lq=600, L=600, n_layers=3, group=1, Hq=8,
                         Hkv=2, D=128, H_idx=4, d_idx=64, topk=64, causal=True)
    announce(f"{cfg.name} {pattern}")
    _, idx, out, _ = _run_pattern(cfg, pattern)
    rows = list(range(cfg.L))
    for g in range(2):
        assert np.array_equal(idx[g][0], oracle.prefill_index_rows(cfg, g, rows)), g
    sample = [0, 1, 63, 64, 65, 599]
    for l, g in ((1, 1), (2, 1)):
        ref = oracle.prefill_attention_rows(cfg, l, sample, idx[g][0][sample])
        assert np.abs(out[l][0, sample] - ref).max() < ATOL, l


def test_causal_prefill_segmented_attention():
    """33000 positions, 4 KV heads: the prefill attention takes the position-
    segment path; rows inside the first segment and rows spanning several
    are checked against the oracle."""
    cfg = C.DecodeConfig("prefill_seg", 8181, B=1, Lq=33000, L=33000, n_layers=1, group=1, Hq=16,
                         Hkv=4, D=128, H_idx=4, d_idx=64, topk=512, causal=True)
    announce(cfg.name)
    idx, out, _ = _run(cfg)
    # rows below k keep every earlier position (nested prefixes: the block-union
    # path); all of them and every row below 2048, then a spread
    sample = np.array(list(range(0, 2048)) + [4095, 4096, 16383, 16384, 16385, 25000, 32767, 32768, 32999])
    # index sets: the exact float32-product scorer and partition select (both
    # pinned on the CPU against the int64 / sort definitions), then the
    # definition itself on a few rows
    qh = C.rows(cfg, cfg.qi_spec(0), (np.zeros_like(sample), sample))
    kh = C.rows(cfg, cfg.ki_spec(0), (np.array([0]),))[0]
    want = oracle.select_topk_threshold(oracle.index_scores_f32(qh, kh), cfg.topk, sample + 1)
    few = [0, 511, 512, 2047, 32999]
    assert np.array_equal(want[[0, 511, 512, 2047, len(sample) - 1]], oracle.prefill_index_rows(cfg, 0, few))
    assert np.array_equal(idx[0][0][sample], want)
    ref = oracle.prefill_attention_rows(cfg, 0, sample, want)
    assert np.abs(out[0][0, sample] - ref).max() < ATOL


def test_causal_prefill_segmented_groups_reuse_index_work():
    """Causal prefill over 33000 positions with Full layers 0 and 3 of five:
    the Shared layers (1, 2, 4) reuse the segment bounds and block-union
    lists their group's Full layer derived from the index, the second Full
    layer derives them anew from its own index; every layer is checked
    against the oracle on rows of the union blocks and of the per-row path."""
    pattern = [1, 0, 0, 1, 0]
    cfg = C.DecodeConfig("prefill_seg_groups", 8282, B=1, Lq=33000, L=33000, n_layers=len(pattern), group=1,
                         Hq=16, Hkv=4, D=128, H_idx=4, d_idx=64, topk=512, causal=True)
    announce(f"{cfg.name} {pattern}")
    _, idx, out, _ = _run_pattern(cfg, pattern)
    sample = np.array([0, 1, 15, 16, 300, 511, 512, 513, 1000, 2047, 2048, 4095, 4096, 16383, 16384,
                       16385, 25000, 32767, 32768, 32999])
    kh_rows = lambda g: C.rows(cfg, cfg.ki_spec(g), (np.array([0]),))[0]
    for g in range(2):
        qh = C.rows(cfg, cfg.qi_spec(g), (np.zeros_like(sample), sample))
        want = oracle.select_topk_threshold(oracle.index_scores_f32(qh, kh_rows(g)), cfg.topk, sample + 1)
        assert np.array_equal(idx[g][0][sample], want), g
    owner = oracle.layer_owner(pattern)
    for l in range(cfg.n_layers):
        ref = oracle.prefill_attention_rows(cfg, l, sample, idx[owner[l]][0][sample])
        assert np.abs(out[l][0, sample] - ref).max() < ATOL, l


def test_decode_shared_kv_cache():
    """One KV cache for every layer (YOCO / CLSA): the same K/V tensors are
    handed to all layers; each layer still has its own queries."""
    cfg = C.DecodeConfig("shared_kv", 9191, B=2, Lq=2, L=6000, n_layers=8, group=4, Hq=16, Hkv=4,
                         D=128, H_idx=4, d_idx=64, topk=512, shared_kv=True)
    announce(cfg.name)
    qi = [sd.make(cfg, cfg.qi_spec(g)) for g in range(cfg.n_groups)]
    ki = [sd.make(cfg, cfg.ki_spec(g)) for g in range(cfg.n_groups)]
    q = [sd.make(cfg, cfg.q_spec(l)) for l in range(cfg.n_layers)]
    k0, v0 = sd.make(cfg, cfg.k_spec(0)), sd.make(cfg, cfg.v_spec(0))
    idx_out = [torch.empty((cfg.B, cfg.Lq, cfg.topk), dtype=torch.int32, device="cuda")
               for _ in range(cfg.n_groups)]
    out, _ = lct.group_run(qi, ki, q, [k0] * cfg.n_layers, [v0] * cfg.n_layers, cfg.topk, cfg.group,
                           cfg.scale, idx_out=idx_out)
    torch.cuda.synchronize()
    ref_idx, ref_out = oracle.decode_step(cfg)
    for g in range(cfg.n_groups):
        assert np.array_equal(host(idx_out[g]), ref_idx[g]), g
    for l in range(cfg.n_layers):
        assert np.abs(host(out[l]) - ref_out[l]).max() < ATOL, l
