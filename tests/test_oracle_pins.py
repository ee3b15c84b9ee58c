"""The CPU oracle against its pins (closed forms, page values, library routines, brute force)."""

import oracle
from tests import oracle_pins as P


def test_index_scores_closed_forms():
    P.pin_index_scores(oracle.index_scores)


def test_index_scores_row_closed_forms():
    P.pin_index_scores_row(oracle.index_scores_row)


def test_index_scores_f32_exact():
    P.pin_index_scores_f32(oracle.index_scores_f32)


def test_topk_bruteforce_ranks():
    P.pin_topk(oracle.select_topk)


def test_topk_threshold_bruteforce_ranks():
    P.pin_topk(oracle.select_topk_threshold)


def test_attention_textbook_cases():
    P.pin_attention(oracle.softmax_attention, oracle.sparse_attention_gqa)


def test_driver_shares_one_index_per_group():
    P.pin_driver_sharing(oracle.decode_step, oracle)


def test_free_full_shared_pattern():
    P.pin_layer_pattern(oracle.layer_owner, oracle.decode_step_pattern, oracle.decode_step)


def test_decode_dense_when_k_covers_cache():
    P.pin_dense_when_k_covers(oracle.decode_step)


def test_planted_needles_are_selected():
    P.pin_needles(oracle.index_scores, oracle.select_topk)


def test_prefill_causal_rows():
    P.pin_prefill(oracle.prefill_index_rows, oracle.prefill_attention_rows)


def test_gsa_dense_when_all_chunks_chosen():
    P.pin_gsa_dense(oracle.gsa_step)


def test_gsa_keeps_selected_gists_and_raw_only():
    P.pin_gsa_sg_sr(oracle.gsa_step)


def test_sizes_match_printed_values():
    P.pin_sizes(oracle.kv_cache_gib, oracle.kv_bytes_per_token, oracle.scored_pairs)


def test_shared_kv_cache_reads_layer_zero():
    """YOCO / CLSA: with one KV cache every layer attends over layer 0's K/V
    (checked by dense softmax attention over the gathered rows, a different
    routine from the GQA one the driver uses), with its own queries."""
    import numpy as np
    import synth
    from synth import configs as C
    cfg = P.small_decode_cfg(shared_kv=True, n_layers=4)
    assert all(cfg.k_spec(l) == cfg.k_spec(0) and cfg.v_spec(l) == cfg.v_spec(0) for l in range(4))
    idx, outs = oracle.decode_step(cfg, batch=[1], layers=[0, 3])
    sel = idx[0][0, 2]
    sel = sel[sel >= 0]
    G = cfg.Hq // cfg.Hkv
    k = synth.as_float(synth.BF16N, C.make(cfg, cfg.k_spec(0)))[1, sel]
    v = synth.as_float(synth.BF16N, C.make(cfg, cfg.v_spec(0)))[1, sel]
    for l in (0, 3):
        q = synth.as_float(synth.BF16N, C.make(cfg, cfg.q_spec(l)))[1, 2]
        for h in range(cfg.Hq):
            want = oracle.softmax_attention(q[h][None], k[:, h // G], v[:, h // G], cfg.scale)[0]
            assert np.allclose(outs[l][0, 2, h], want, atol=1e-12)
    assert not np.allclose(outs[0], outs[3])  # the queries differ per layer


def test_hgsa_coarse_to_fine_select():
    P.pin_hgsa_select(oracle.hgsa_select, oracle.gsa_select)


def test_gsa_prefill_gist_mask():
    P.pin_gsa_prefill(oracle.gsa_prefill, oracle.gsa_prefill_visible)


def test_hgsa_step_gathers_and_attention():
    P.pin_hgsa_step(oracle.hgsa_step, oracle.gsa_step)
