"""The CPU oracle against its pins (closed forms, page values, library routines, brute force)."""

import oracle
from tests import oracle_pins as P


def test_index_scores_closed_forms():
    P.pin_index_scores(oracle.index_scores)


def test_topk_bruteforce_ranks():
    P.pin_topk(oracle.select_topk)


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
