"""Causal prefill index of one group (fused score filter + exact select)
against the CPU oracle, every row compared, on the MI355X.

Inputs are the seeded int8 generator's (uniform on [-8, 7], the indexer
workload's distribution) plus hand-built score patterns that drive the
select through each of its cases: the bin list, the theta ties, rows that
keep every key, and rows the filter hands to the plain path.
"""

import numpy as np
import pytest
import torch

import long_context_top_amd as lct
import oracle
import synth
from tests.gpu_util import announce, dev_i8, host

pytestmark = pytest.mark.gpu

HD = 256


def _synth_qk(seed, L):
    q = synth.tensor(synth.I8U4, seed, 1, (L, HD))
    k = synth.tensor(synth.I8U4, seed, 2, (L, HD))
    return q, k


def _want(q, k, topk, rows=None):
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    s = oracle.index_scores(q[rows][None], k[None], 4)[0]
    return oracle.select_topk(s, topk, rows + 1)


def _run(q, k, topk):
    stats = {}
    out = lct.prefill_index(dev_i8(q), dev_i8(k), topk, stats=stats)
    torch.cuda.synchronize()
    print(f"  rows on the plain path: {stats['n_fallback']}", flush=True)
    return host(out), stats["n_fallback"]


@pytest.mark.parametrize("L,topk", [(1, 1), (7, 16), (129, 64), (700, 64), (1500, 1),
                                    (1500, 512), (3001, 2048), (4100, 256)])
def test_prefill_index_synthetic_all_rows(L, topk):
    announce(f"prefill_index L={L} k={topk}")
    q, k = _synth_qk(1000 + L + topk, L)
    got, _ = _run(q, k, topk)
    assert np.array_equal(got, _want(q, k, topk))


def test_prefill_index_equal_scores_take_plain_path():
    """Every score equal: a row's candidates crowd one bin, so the long
    rows go through the plain path (in several batches); every row keeps its
    lowest positions."""
    L, topk = 1500, 64
    announce(f"prefill_index equal scores L={L} k={topk}")
    q, _ = _synth_qk(77, L)
    k = np.zeros((L, HD), dtype=np.int8)
    got, nf = _run(q, k, topk)
    assert np.array_equal(got, _want(q, k, topk))
    assert 0 < nf <= L - topk


def test_prefill_index_sample_bias_and_equal_bins():
    """Sampled positions (every 16th) score 100, the rest 99: the threshold
    lands at the samples' score, so the rows whose candidates (the sampled
    positions alone) are fewer than k go through the plain path, longer rows
    settle one bin of equal scores by position, and rows with few samples
    keep every key."""
    L, topk = 2000, 64
    announce(f"prefill_index sample bias L={L} k={topk}")
    q = np.zeros((L, HD), dtype=np.int8)
    q[:, 0] = 1
    k = np.zeros((L, HD), dtype=np.int8)
    k[:, 0] = 99
    k[::16, 0] = 100
    got, nf = _run(q, k, topk)
    assert np.array_equal(got, _want(q, k, topk))
    assert 0 < nf < L - 16 * topk


def test_prefill_index_mixed_rows():
    """Half of the query rows have all-zero scores (plain path), half are
    synthetic: both kinds in one call."""
    L, topk = 2500, 128
    announce(f"prefill_index mixed rows L={L} k={topk}")
    q, k = _synth_qk(4242, L)
    q[1::2] = 0
    got, nf = _run(q, k, topk)
    assert np.array_equal(got, _want(q, k, topk))
    assert (L - topk) // 4 < nf <= (L - topk) // 2 + 1  # long zero rows only


def test_prefill_index_unfused_shape():
    """HD = 128 takes the blocked score + row-select path."""
    L, topk = 900, 100
    announce(f"prefill_index HD=128 L={L} k={topk}")
    q = synth.tensor(synth.I8U4, 9, 1, (L, 128))
    k = synth.tensor(synth.I8U4, 9, 2, (L, 128))
    got, nf = _run(q, k, topk)
    assert nf == 0
    assert np.array_equal(got, _want(q, k, topk))
