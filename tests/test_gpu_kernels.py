"""Per-kernel parity of the HIP path against the CPU oracle (MI355X).

Index sets and integer scores must match bit-exactly; attention outputs
within max-abs 1e-2 of the oracle's float64 result (bf16 inputs, fp32
accumulation and bf16 attention weights in the PV product).
"""

import math

import numpy as np
import pytest
import torch

import long_context_top_amd as lct
import oracle
import synth
from tests.gpu_util import announce, dev_bf16, dev_f32, dev_i8, dev_i32, host

pytestmark = pytest.mark.gpu

ATOL = 1e-2


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------ generator ----

@pytest.mark.parametrize("kind", [synth.I8U4, synth.BF16U4, synth.BF16N])
def test_device_generator_matches_host(kind):
    import synth.device as sd
    announce(f"synth fill kind={kind}")
    n = (1 << 20) + 37
    dtype = torch.int8 if kind == synth.I8U4 else torch.bfloat16
    t = torch.empty(n, dtype=dtype, device="cuda")
    sd.fill_(t, kind, 1234, 77)
    want = synth.values(kind, 1234, 77, np.arange(n))
    if kind == synth.I8U4:
        got = t.cpu().numpy()
    else:
        got = t.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)


# -------------------------------------------------------------- indexer ----

@pytest.mark.parametrize("B,Lq,L,HD", [(2, 1, 3000, 256), (1, 16, 2048, 64), (3, 5, 777, 128),
                                        (1, 3, 1111, 16), (2, 2, 501, 32), (1, 4, 1500, 512),
                                        (8, 1, 65, 256)])
def test_idx_score_stream_exact(B, Lq, L, HD):
    announce(f"idx_score stream B={B} Lq={Lq} L={L} HD={HD}")
    r = _rng(B * 1000 + L)
    qi = r.integers(-128, 128, size=(B, Lq, HD))
    ki = r.integers(-128, 128, size=(B, L, HD))
    got = host(lct.idx_score(dev_i8(qi), dev_i8(ki)))
    want = oracle.index_scores(qi.astype(np.int8), ki.astype(np.int8), 4 if HD >= 64 else 1)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("Lq,L,HD,pos0", [(300, 300, 256, 0), (200, 333, 256, 133), (130, 130, 64, 0),
                                           (64 + 17, 190, 128, 100)])
def test_idx_score_mfma_causal_exact(Lq, L, HD, pos0):
    announce(f"idx_score mfma Lq={Lq} L={L} HD={HD} pos0={pos0}")
    r = _rng(L + HD)
    qi = r.integers(-128, 128, size=(1, Lq, HD))
    ki = r.integers(-128, 128, size=(1, L, HD))
    got = host(lct.idx_score(dev_i8(qi), dev_i8(ki), q_pos0=pos0))
    want = oracle.index_scores(qi.astype(np.int8), ki.astype(np.int8), 1)
    for row in range(Lq):
        vis = pos0 + row + 1
        assert np.array_equal(got[0, row, :vis], want[0, row, :vis]), row


def test_idx_score_mfma_dense_exact():
    announce("idx_score mfma dense")
    r = _rng(5)
    qi = r.integers(-128, 128, size=(2, 40, 256))
    ki = r.integers(-128, 128, size=(2, 250, 256))
    got = host(lct.idx_score(dev_i8(qi), dev_i8(ki)))
    assert np.array_equal(got, oracle.index_scores(qi.astype(np.int8), ki.astype(np.int8), 4))


# ---------------------------------------------------------------- top-k ----

def _check_topk(scores, k, valid_len=None):
    vl_t = None if valid_len is None else dev_i32(np.asarray(valid_len))
    if scores.dtype.kind == "f":
        st = dev_f32(scores)
    else:
        st = dev_i32(scores)
    got = host(lct.topk_select(st, k, valid_len=vl_t))
    want = oracle.select_topk(scores, k, valid_len)
    bad = np.where(~np.all(got == want, axis=1))[0]
    assert bad.size == 0, f"rows {bad[:5]} differ; first: got {got[bad[0]][:8]} want {want[bad[0]][:8]}"


@pytest.mark.parametrize("case", ["narrow", "wide", "allequal", "binary", "valid", "k_ge_n", "float", "tiny_n"])
def test_topk_rows_kernel(case):
    announce(f"topk rows {case}")
    r = _rng(hash(case) % 1000)
    rows, n, k = 100, 5000, 64
    vl = None
    if case == "narrow":
        s = r.integers(-50, 50, size=(rows, n))
    elif case == "wide":
        s = r.integers(-2**31, 2**31 - 1, size=(rows, n), dtype=np.int64)
    elif case == "allequal":
        s = np.full((rows, n), 7)
    elif case == "binary":
        s = r.integers(0, 2, size=(rows, n))
    elif case == "valid":
        s = r.integers(-1000, 1000, size=(rows, n))
        vl = r.integers(0, n + 10, size=rows)
        vl[:5] = [0, 1, 63, 64, 65]
    elif case == "k_ge_n":
        s = r.integers(-5, 5, size=(rows, 50))
        k = 64
    elif case == "float":
        s = r.standard_normal((rows, n)).astype(np.float32)
        s[:, ::7] = 0.0
        s[:, ::11] = -0.0
        s[:, 5] = 1e30
    else:
        s = r.integers(-3, 3, size=(rows, 3))
        k = 2
    _check_topk(s if s.dtype.kind == "f" else s.astype(np.int64), k, vl)


@pytest.mark.parametrize("n", [8192, 8193, 20000, 100000])
@pytest.mark.parametrize("case", ["random", "allequal", "valid"])
def test_topk_rows_kernel_long_rows(n, case):
    """More than 64 rows of up to 100000 keys: the one-workgroup-per-row
    select, its full-bitmap instance above 8192 keys and the rows it reads
    again per pass (above 8192 keys it cannot keep in registers)."""
    announce(f"topk rows long n={n} {case}")
    r = _rng(n + len(case))
    rows, k = 65, 512
    vl = None
    if case == "random":
        s = r.integers(-3000, 3000, size=(rows, n))
    elif case == "allequal":
        s = np.full((rows, n), -11)
    else:
        s = r.integers(-100, 100, size=(rows, n))
        vl = r.integers(0, n + 5, size=rows)
        vl[:6] = [0, 1, 511, 512, 8192, 8193]
    _check_topk(s.astype(np.int64), k, vl)


@pytest.mark.parametrize("case", ["normal", "allequal", "outlier", "valid", "float", "many_rows_long"])
def test_topk_multi_kernel(case):
    announce(f"topk multi {case}")
    r = _rng(len(case))
    rows, n, k = 3, 200003, 2048
    vl = None
    if case == "normal":
        s = np.round(r.standard_normal((rows, n)) * 344 + 64)
    elif case == "allequal":
        s = np.full((rows, 40000), -3)
    elif case == "outlier":
        s = r.integers(-500, 500, size=(rows, n))
        s[:, 17] = 2**31 - 1  # forces a wide window: the threshold bin holds many candidates
        s[:, 99] = -2**31
    elif case == "valid":
        s = r.integers(-300, 300, size=(rows, n))
        vl = [n, 1000, 2048]
    elif case == "float":
        s = (r.standard_normal((rows, n)) * 100).astype(np.float32)
    else:
        rows, n = 70, 300000  # n above the row-kernel limit: multi path in row chunks
        s = r.integers(-2000, 2000, size=(rows, n))
        k = 100
    _check_topk(s if s.dtype.kind == "f" else s.astype(np.int64), k, vl)


# ------------------------------------------------------------ attention ----

def _attn_case(B, Lq, Hq, Hkv, L, kk, seed, pad=0, shuffle=False, ones=False):
    r = _rng(seed)
    q, qh = dev_bf16(r.standard_normal((B, Lq, Hq, 128)))
    k, kh = dev_bf16(r.standard_normal((B, L, Hkv, 128)))
    vv = np.ones((B, L, Hkv, 128)) if ones else r.standard_normal((B, L, Hkv, 128))
    v, vh = dev_bf16(vv)
    idx = np.full((B, Lq, kk), -1, dtype=np.int32)
    for b in range(B):
        for j in range(Lq):
            m = max(0, kk - pad)
            sel = np.sort(r.choice(L, size=min(m, L), replace=False))
            if shuffle:
                r.shuffle(sel)
            idx[b, j, :sel.size] = sel
    scale = 1.0 / math.sqrt(128)
    got = host(lct.sparse_attn_gather(q, k, v, dev_i32(idx), scale))
    want = np.zeros_like(got, dtype=np.float64)
    for b in range(B):
        for j in range(Lq):
            sel = idx[b, j][idx[b, j] >= 0]
            if sel.size:
                want[b, j] = oracle.sparse_attention_gqa(qh[b, j], kh[b, sel], vh[b, sel], scale)
    return got, want


@pytest.mark.parametrize("B,Lq,Hq,Hkv,L,kk", [(2, 3, 8, 2, 1000, 100), (1, 1, 32, 4, 5000, 2048),
                                               (1, 2, 16, 16, 300, 37), (3, 1, 16, 1, 700, 128),
                                               (1, 1, 8, 8, 64, 64), (2, 1, 4, 2, 4000, 1000),
                                               (1, 1, 16, 1, 5000, 2048), (8, 1, 32, 4, 9000, 2048)])
def test_sparse_attn_matches_oracle(B, Lq, Hq, Hkv, L, kk):
    announce(f"attn B={B} Lq={Lq} Hq={Hq} Hkv={Hkv} L={L} kk={kk}")
    got, want = _attn_case(B, Lq, Hq, Hkv, L, kk, seed=L + kk, pad=kk // 7)
    err = np.abs(got - want).max()
    assert err < ATOL, err


def test_sparse_attn_order_invariant_and_ones():
    announce("attn shuffled / V=1")
    got, want = _attn_case(1, 2, 8, 1, 3000, 300, seed=3, shuffle=True)
    assert np.abs(got - want).max() < ATOL
    got1, _ = _attn_case(2, 1, 32, 4, 3000, 2048, seed=4, ones=True)
    assert np.abs(got1 - 1.0).max() < 1e-5


def test_sparse_attn_split_path_repeated_calls():
    """The split path's workgroups count themselves in per (row, KV head) and
    the last one merges; every call must leave the counters ready for the
    next, on one workspace, with a different shape in between."""
    announce("attn split path, repeated calls on one workspace")
    ws = lct.Workspace()
    r = _rng(21)
    for it, (B, kk) in enumerate([(2, 2048), (2, 2048), (1, 700), (3, 2048)]):
        L, Hq, Hkv = 6000, 32, 4
        q, qh = dev_bf16(r.standard_normal((B, 1, Hq, 128)))
        k, kh = dev_bf16(r.standard_normal((B, L, Hkv, 128)))
        v, vh = dev_bf16(r.standard_normal((B, L, Hkv, 128)))
        idx = np.stack([np.sort(r.choice(L, size=kk, replace=False)) for _ in range(B)])[:, None, :]
        idx = idx.astype(np.int32)
        scale = 1.0 / math.sqrt(128)
        got = host(lct.sparse_attn_gather(q, k, v, dev_i32(idx), scale, ws=ws))
        for b in range(B):
            want = oracle.sparse_attention_gqa(qh[b, 0], kh[b, idx[b, 0]], vh[b, idx[b, 0]], scale)
            assert np.abs(got[b, 0] - want).max() < ATOL, (it, b)


def test_sparse_attn_empty_rows_are_zero():
    announce("attn empty rows")
    got, _ = _attn_case(1, 3, 8, 2, 100, 32, seed=9, pad=32)
    assert np.all(got == 0.0)


@pytest.mark.parametrize("Hq", [8, 4])
def test_sparse_attn_segmented_path_row_shapes(Hq):
    """Many rows over a long cache take the position-segment path (16800
    (row, KV head) pairs, 40000 positions: several segments), at 2 and 1
    query heads per KV head.  Rows of every shape: ascending with -1
    padding, inside one segment, skipping a segment, shuffled, with
    duplicates, with -1 in the middle, empty, full."""
    B, Lq, Hkv, L, kk = 2, 2100, 4, 40000, 200
    announce(f"attn segmented B={B} Lq={Lq} Hkv={Hkv} L={L} kk={kk}")
    r = _rng(77)
    q, qh = dev_bf16(r.standard_normal((B, Lq, Hq, 128)))
    k, kh = dev_bf16(r.standard_normal((B, L, Hkv, 128)))
    v, vh = dev_bf16(r.standard_normal((B, L, Hkv, 128)))
    idx = np.full((B, Lq, kk), -1, dtype=np.int32)
    for b in range(B):
        for j in range(Lq):
            kind = (j + b) % 8
            if kind == 0:
                sel = np.sort(r.choice(L, size=kk - 1 - j % 50, replace=False))
            elif kind == 1:
                sel = np.sort(r.choice(np.arange(16384, 16384 + 4096), size=kk, replace=False))
            elif kind == 2:
                sel = r.choice(L, size=kk, replace=False)
            elif kind == 3:
                sel = np.zeros(0, dtype=np.int64)
            elif kind == 4:
                sel = np.sort(r.choice(L, size=kk // 2, replace=True))
                sel = np.sort(np.concatenate([sel, sel[:10]]))
            elif kind == 5:
                pool = np.concatenate([np.arange(0, 4096), np.arange(32768, L)])
                sel = np.sort(r.choice(pool, size=kk // 3, replace=False))
            elif kind == 6:
                sel = np.sort(r.choice(L, size=kk, replace=False))
            else:
                sel = np.sort(r.choice(L, size=kk - 5, replace=False))
                sel = np.concatenate([sel[:40], [-1] * 5, sel[40:]])
            idx[b, j, :sel.size] = sel
    scale = 1.0 / math.sqrt(128)
    got = host(lct.sparse_attn_gather(q, k, v, dev_i32(idx), scale))
    nb = lct._sz()
    lct._check(lct.lib().lct_sparse_attn_workspace_bytes(B, Lq, Hq, Hkv, 128, L, kk, lct._c.byref(nb)))
    assert nb.value >= B * Lq * Hkv * 2 * Hq // Hkv * 130 * 4  # partials, two segments or more
    for b in range(B):
        for j in range(Lq):
            sel = idx[b, j][idx[b, j] >= 0]
            if sel.size == 0:
                assert np.all(got[b, j] == 0.0), (b, j)
                continue
            want = oracle.sparse_attention_gqa(qh[b, j], kh[b, sel], vh[b, sel], scale)
            err = np.abs(got[b, j] - want).max()
            assert err < ATOL, (b, j, (j + b) % 8, err)


# ------------------------------------------------------------------ GSA ----

def _gsa_inputs(cfg, gist_vals=None):
    from synth import configs as C
    f = synth.as_float
    q_bits = C.make(cfg, cfg.q_spec())
    gk_bits = C.make(cfg, cfg.gk_spec())
    if gist_vals is not None:
        q_bits, gk_bits = gist_vals
    return dict(q=q_bits, gk=gk_bits, gv=C.make(cfg, cfg.gv_spec()), rk=C.make(cfg, cfg.rk_spec()),
                rv=C.make(cfg, cfg.rv_spec()))


def _union_sizes(idx):
    """Size of the union of the valid positions of each block of 16 rows."""
    rows = idx.reshape(-1, idx.shape[-1])
    return np.array([np.unique(rows[b:b + 16][rows[b:b + 16] >= 0]).size for b in range(0, rows.shape[0], 16)])


def _union_rule(idx, G, bad_blocks):
    """The block-union decisions the plan must take: a block of valid rows
    (ascending, then -1) takes the path with its union's size as the flag
    when the union holds at most 4096 positions and the rows select each
    union position 6 G / 8 times on average; other blocks get 0."""
    rows = idx.reshape(-1, idx.shape[-1])
    usz = _union_sizes(idx)
    sum_n = np.array([(rows[b:b + 16] >= 0).sum() for b in range(0, rows.shape[0], 16)])
    take = (sum_n > 0) & (usz <= 4096) & (usz * 6 * G <= sum_n * 8)
    want = np.where(take, usz, 0)
    want[bad_blocks] = 0
    return want


def _union_flags(ws, B, Lq, Hq, Hkv, L, kk):
    """The block-union decisions the last call left in its workspace (int32
    per block of 16 rows, after the segment partials and bounds): the union's
    size for a block on the union path, else 0."""
    G = Hq // Hkv
    shift = 14
    while ((L - 1) >> shift) + 1 > 64:
        shift += 1
    nseg = ((L - 1) >> shift) + 1
    rows = B * Lq
    up = lambda x: (x + 255) // 256 * 256
    part = rows * Hkv * nseg * G * 132 * 4
    off = up(up(part) + rows * (nseg + 1) * 4)
    n = rows // 16
    return ws.buf[off:off + 4 * n].view(torch.int32).cpu().numpy()


@pytest.mark.parametrize("Hq,Hkv", [(32, 4), (16, 4), (64, 4)])
def test_sparse_attn_block_union_path(Hq, Hkv):
    """Many rows over a long cache whose neighbours share positions: blocks
    of 16 rows with one common set, with nested prefix sets (the causal
    prefill's short rows), with half-shared sets, with independent random
    sets, with a row that is not ascending, or with an empty row among
    shared ones.  The decisions the call leaves in its workspace match the
    plan's rule block by block (every common-set block takes the union path,
    no block with a row out of order does), and every row is compared with
    the oracle."""
    B, Lq, L, kk = 1, 4096, 40000, 256        # 16384 (row, KV head) pairs: the segment path
    announce(f"attn block union Hq={Hq} Hkv={Hkv} Lq={Lq} L={L} kk={kk}")
    r = _rng(Hq)
    q, qh = dev_bf16(r.standard_normal((B, Lq, Hq, 128)))
    k, kh = dev_bf16(r.standard_normal((B, L, Hkv, 128)))
    v, vh = dev_bf16(r.standard_normal((B, L, Hkv, 128)))
    idx = np.full((B, Lq, kk), -1, dtype=np.int32)
    kinds = []
    for blk in range(Lq // 16):
        kind = blk % 6
        kinds.append(kind)
        common = np.sort(r.choice(L, size=kk, replace=False))
        for i in range(16):
            j = blk * 16 + i
            if kind == 0:                       # one common set
                sel = common
            elif kind == 1:                     # nested prefixes 0..m
                m = (blk * 7 + i * 13) % kk + 1
                sel = np.arange(m)
            elif kind == 2:                     # half shared, half own
                own = r.choice(L, size=kk // 2, replace=False)
                sel = np.unique(np.concatenate([common[: kk // 2], own]))[:kk]
            elif kind == 3:                     # independent random sets
                sel = np.sort(r.choice(L, size=kk - (i % 3), replace=False))
            elif kind == 4:                     # common set, one row not ascending
                sel = common.copy()
                if i == 5:
                    sel = sel[::-1].copy()
            else:                               # common set, one empty row, one short row
                sel = common if i not in (3, 9) else (np.zeros(0, np.int64) if i == 3 else common[:17])
            idx[0, j, :sel.size] = sel
    scale = 1.0 / math.sqrt(128)
    ws = lct.Workspace()
    got = host(lct.sparse_attn_gather(q, k, v, dev_i32(idx), scale, ws=ws))
    flags = _union_flags(ws, B, Lq, Hq, Hkv, L, kk)
    kinds = np.array(kinds)
    want = _union_rule(idx, Hq // Hkv, kinds == 4)   # kind 4: a row that is not ascending
    assert np.array_equal(flags, want)
    assert np.all(flags[kinds == 0] > 0) and np.all(flags[kinds == 4] == 0)
    print(f"  union blocks: {int(flags.sum())} of {flags.size}", flush=True)
    worst = 0.0
    for j in range(Lq):
        sel = idx[0, j][idx[0, j] >= 0]
        if sel.size == 0:
            assert np.all(got[0, j] == 0.0), j
            continue
        want = oracle.sparse_attention_gqa(qh[0, j], kh[0, sel], vh[0, sel], scale)
        err = np.abs(got[0, j] - want).max()
        worst = max(worst, err)
        assert err < ATOL, (j, kinds[j // 16], err)
    print(f"  max |out - oracle| = {worst:.2e}", flush=True)


def test_sparse_attn_block_union_two_batch_entries():
    """Two batch entries of 2056 rows (not a multiple of 16): every block of
    16 rows shares one set, so every block takes the block-union path except
    the one that straddles the two entries (rows 2048..2063); the second
    entry's union blocks gather from its own K/V.  A block whose shared set
    holds a position past the cache (its last entry, seen by one lane of the
    check) and a block with one row holding one pair out of order are
    decided per row, which skips the former entry and takes the latter row
    in any order.  Every row is compared with the oracle."""
    B, Lq, L, kk, Hq, Hkv = 2, 2056, 40000, 256, 32, 4
    announce(f"attn block union B={B} Lq={Lq} L={L} kk={kk}")
    r = _rng(77)
    q, qh = dev_bf16(r.standard_normal((B, Lq, Hq, 128)))
    k, kh = dev_bf16(r.standard_normal((B, L, Hkv, 128)))
    v, vh = dev_bf16(r.standard_normal((B, L, Hkv, 128)))
    rows = B * Lq
    idx = np.full((rows, kk), -1, dtype=np.int32)
    for blk in range(rows // 16 + 1):
        common = np.sort(r.choice(L, size=kk, replace=False)).astype(np.int32)
        if blk == 5:
            common[-1] = L + 3                          # past the cache
        idx[blk * 16:(blk + 1) * 16] = common
        if blk == 9:                                    # one row with one pair out of order
            idx[blk * 16 + 3, 100], idx[blk * 16 + 3, 101] = common[101], common[100]
    idx = idx.reshape(B, Lq, kk)
    scale = 1.0 / math.sqrt(128)
    ws = lct.Workspace()
    got = host(lct.sparse_attn_gather(q, k, v, dev_i32(idx), scale, ws=ws))
    flags = _union_flags(ws, B, Lq, Hq, Hkv, L, kk)
    bad = np.zeros(rows // 16, bool)
    bad[2048 // 16] = True                              # straddles the two entries
    bad[5] = bad[9] = True
    assert np.array_equal(flags, _union_rule(idx, Hq // Hkv, bad))
    assert np.all(flags[~bad] > 0)
    worst = 0.0
    for b in range(B):
        for j in range(Lq):
            sel = idx[b, j]
            sel = sel[(sel >= 0) & (sel < L)]
            want = oracle.sparse_attention_gqa(qh[b, j], kh[b, sel], vh[b, sel], scale)
            err = np.abs(got[b, j] - want).max()
            worst = max(worst, err)
            assert err < ATOL, (b, j, err)
    print(f"  max |out - oracle| = {worst:.2e}", flush=True)


@pytest.mark.parametrize("Hq,Hkv", [(32, 4), (16, 4)])
def test_sparse_attn_block_union_large_unions(Hq, Hkv):
    """Blocks of 16 rows of 2048 positions drawn from a common pool: a pool of
    3000 and one of exactly 4096 (rows 0 and 1 take its even and odd
    positions; 64 chunks, the largest union the block-union path holds) take
    that path; a pool of 5000 shares enough but its union is too large, and
    independent random sets share too little: both are decided per row.
    Rows of every kind are compared with the oracle."""
    B, Lq, L, kk = 1, 4096, 40000, 2048
    announce(f"attn block union large Hq={Hq} Hkv={Hkv} Lq={Lq} L={L} kk={kk}")
    r = _rng(Hq + 7)
    q, qh = dev_bf16(r.standard_normal((B, Lq, Hq, 128)))
    k, kh = dev_bf16(r.standard_normal((B, L, Hkv, 128)))
    v, vh = dev_bf16(r.standard_normal((B, L, Hkv, 128)))
    idx = np.full((B, Lq, kk), -1, dtype=np.int32)
    pools = {0: 3000, 1: 4096, 2: 5000}
    kinds = np.arange(Lq // 16) % 4
    for blk, kind in enumerate(kinds):
        pool = np.sort(r.choice(L, size=pools[kind], replace=False)) if kind in pools else None
        for i in range(16):
            if kind == 1 and i < 2:
                sel = pool[i::2]
            elif pool is not None:
                sel = np.sort(r.choice(pool, size=kk, replace=False))
            else:
                sel = np.sort(r.choice(L, size=kk, replace=False))
            idx[0, blk * 16 + i] = sel
    scale = 1.0 / math.sqrt(128)
    ws = lct.Workspace()
    got = host(lct.sparse_attn_gather(q, k, v, dev_i32(idx), scale, ws=ws))
    flags = _union_flags(ws, B, Lq, Hq, Hkv, L, kk)
    assert np.array_equal(flags, _union_rule(idx, Hq // Hkv, np.zeros(kinds.size, bool)))
    usz = _union_sizes(idx)
    assert np.array_equal(flags[kinds == 0], usz[kinds == 0]) and np.all(flags[kinds == 1] == 4096)
    assert np.all(flags[kinds == 2] == 0) and np.all(flags[kinds == 3] == 0)
    rows = [j for j in range(Lq) if j // 16 < 64 or j % 37 == 0]
    worst = 0.0
    for j in rows:
        sel = idx[0, j]
        want = oracle.sparse_attention_gqa(qh[0, j], kh[0, sel], vh[0, sel], scale)
        err = np.abs(got[0, j] - want).max()
        worst = max(worst, err)
        assert err < ATOL, (j, int(kinds[j // 16]), err)
    print(f"  {len(rows)} rows, max |out - oracle| = {worst:.2e}", flush=True)


def test_sparse_attn_block_union_sixteen_heads_per_kv_head():
    """16 query heads per KV head: the plan's limit is then 16 x 2048 x 8 /
    (6 x 16) = 2730 union positions, so pools of 2400 and 2100 positions take
    the instance for unions above 2048 and a set shared by the whole block the
    one for unions up to 2048; independent sets go per row.  The decisions
    match the rule and the rows match the oracle."""
    B, Lq, L, kk, Hq, Hkv = 1, 4096, 40000, 2048, 64, 4
    announce(f"attn block union G=16 Lq={Lq} L={L} kk={kk}")
    r = _rng(1601)
    q, qh = dev_bf16(r.standard_normal((B, Lq, Hq, 128)))
    k, kh = dev_bf16(r.standard_normal((B, L, Hkv, 128)))
    v, vh = dev_bf16(r.standard_normal((B, L, Hkv, 128)))
    idx = np.full((B, Lq, kk), -1, dtype=np.int32)
    kinds = np.arange(Lq // 16) % 4
    for blk, kind in enumerate(kinds):
        if kind == 3:
            shared = np.sort(r.choice(L, size=kk, replace=False))
        pool = np.sort(r.choice(L, size={0: 2400, 1: 2100}[kind], replace=False)) if kind < 2 else None
        for i in range(16):
            if pool is not None:
                sel = np.sort(r.choice(pool, size=kk, replace=False))
            elif kind == 3:
                sel = shared
            else:
                sel = np.sort(r.choice(L, size=kk, replace=False))
            idx[0, blk * 16 + i] = sel
    scale = 1.0 / math.sqrt(128)
    ws = lct.Workspace()
    got = host(lct.sparse_attn_gather(q, k, v, dev_i32(idx), scale, ws=ws))
    flags = _union_flags(ws, B, Lq, Hq, Hkv, L, kk)
    assert np.array_equal(flags, _union_rule(idx, Hq // Hkv, np.zeros(kinds.size, bool)))
    assert np.all(flags[kinds < 2] > 2048) and np.all(flags[kinds == 3] == 2048) and np.all(flags[kinds == 2] == 0)
    rows = [j for j in range(Lq) if j // 16 < 24 or j % 61 == 0]
    worst = 0.0
    for j in rows:
        sel = idx[0, j]
        want = oracle.sparse_attention_gqa(qh[0, j], kh[0, sel], vh[0, sel], scale)
        err = np.abs(got[0, j] - want).max()
        worst = max(worst, err)
        assert err < ATOL, (j, int(kinds[j // 16]), err)
    print(f"  {len(rows)} rows, max |out - oracle| = {worst:.2e}", flush=True)


@pytest.mark.parametrize("tail", [0, 1, 7, 15, 16])
def test_gist_score_and_gsa_decode(tail):
    from synth import configs as C
    from tests.gpu_util import dev_bf16_bits
    announce(f"gsa decode tail={tail}")
    cfg = C.GsaConfig("t_gsa", 31 + tail, B=2, H=3, D=128, Nc=300, chunk=16, kc=8, tail_len=tail)
    inp = _gsa_inputs(cfg)
    BH = cfg.B * cfg.H
    dv = {k: dev_bf16_bits(v.reshape((BH,) + v.shape[2:])) for k, v in inp.items()}
    gs = host(lct.gist_score(dv["q"], dv["gk"]))
    qf = synth.as_float(synth.BF16U4, inp["q"]).reshape(BH, 128)
    gkf = synth.as_float(synth.BF16U4, inp["gk"]).reshape(BH, cfg.Nc, 128)
    assert np.array_equal(gs, oracle.gist_scores(qf, gkf))  # integer-valued: exact
    out, cidx = lct.gsa_decode(dv["q"], dv["gk"], dv["gv"], dv["rk"], dv["rv"], cfg.kc, tail, cfg.scale)
    ref_idx, ref_out = oracle.driver.gsa_step(cfg)
    assert np.array_equal(host(cidx), ref_idx)
    assert np.abs(host(out) - ref_out).max() < ATOL


def test_gsa_attn_long_and_ragged_chunk_lists():
    """lct_gsa_attn straight from a chunk list: 512 (batch, head) rows of 300
    chunks each (one split per row, so a wave takes 76 items in turn), with
    -1 entries and ids past Nc that are skipped, and a row with no valid
    chunk (the tail alone).  Rows are compared with the
    oracle over exactly the listed valid chunks' raw rows, their gists and the
    tail."""
    BH, Nc, kc, tail, D = 512, 320, 300, 5, 128
    announce(f"gsa attn BH={BH} Nc={Nc} kc={kc} tail={tail}")
    gen = torch.Generator(device="cuda").manual_seed(4242)
    dev = "cuda"
    raw_cap = Nc * 16 + tail
    rk = torch.randn((BH, raw_cap, D), generator=gen, device=dev).to(torch.bfloat16)
    rv = torch.randn((BH, raw_cap, D), generator=gen, device=dev).to(torch.bfloat16)
    gk = torch.randn((BH, Nc, D), generator=gen, device=dev).to(torch.bfloat16)
    gv = torch.randn((BH, Nc, D), generator=gen, device=dev).to(torch.bfloat16)
    q = torch.randn((BH, D), generator=gen, device=dev).to(torch.bfloat16)
    r = _rng(99)
    cid = np.stack([r.permutation(Nc)[:kc] for _ in range(BH)]).astype(np.int32)
    cid[r.random(cid.shape) < 0.05] = -1
    cid[r.random(cid.shape) < 0.03] = Nc + 7          # past Nc: skipped
    cid[7, :] = -1                                     # only the tail
    qh = q.float().cpu().numpy().astype(np.float64)
    gkh = gk.float().cpu().numpy().astype(np.float64)
    gs = np.einsum("bd,bnd->bn", qh, gkh).astype(np.float32)
    scale = 1.0 / math.sqrt(D)
    got = host(lct.gsa_attn(q, rk, rv, gv, dev_f32(gs), dev_i32(cid), tail, scale))
    worst = 0.0
    for b in (0, 7, 100, 257, 511):
        ch = cid[b][(cid[b] >= 0) & (cid[b] < Nc)]
        pos = np.concatenate([(ch[:, None] * 16 + np.arange(16)[None, :]).reshape(-1),
                              Nc * 16 + np.arange(tail)])
        rkb, rvb = rk[b].float().cpu().numpy(), rv[b].float().cpu().numpy()
        gvb = gv[b].float().cpu().numpy()
        want = oracle.gsa_attention(qh[b], rkb[pos], rvb[pos], gkh[b, ch], gvb[ch], scale)
        err = np.abs(got[b] - want).max()
        worst = max(worst, err)
        assert err < ATOL, (b, err)
    print(f"  max |out - oracle| = {worst:.2e}", flush=True)


@pytest.mark.parametrize("Nc,group,km,kc,tail", [(300, 16, 3, 8, 1), (300, 4, 2, 16, 0),
                                                  (1000, 64, 4, 64, 16), (2049, 1, 64, 64, 5),
                                                  (513, 512, 2, 100, 1)])
def test_hgsa_decode(Nc, group, km, kc, tail):
    """Coarse-to-fine routing against the oracle: short last groups, fewer
    candidates than kc (-1 padding), groups of one gist, two groups only."""
    from synth import configs as C
    from tests.gpu_util import dev_bf16_bits
    announce(f"hgsa decode Nc={Nc} group={group} km={km} kc={kc} tail={tail}")
    cfg = C.GsaConfig("t_hgsa", 700 + Nc + group, B=2, H=3, D=128, Nc=Nc, chunk=16, kc=kc,
                      tail_len=tail, group=group, km=km)
    inp = _gsa_inputs(cfg)
    inp["mk"] = C.make(cfg, cfg.mk_spec())
    BH = cfg.B * cfg.H
    dv = {k: dev_bf16_bits(v.reshape((BH,) + v.shape[2:])) for k, v in inp.items()}
    out, cidx = lct.hgsa_decode(dv["q"], dv["mk"], dv["gk"], dv["gv"], dv["rk"], dv["rv"], group, km, kc,
                                tail, cfg.scale)
    ref_idx, ref_out = oracle.driver.hgsa_step(cfg)
    assert np.array_equal(host(cidx), ref_idx)
    assert np.abs(host(out) - ref_out).max() < ATOL


@pytest.mark.parametrize("Nc,BH", [(1, 2), (3, 2), (4, 1), (5, 3), (67, 2), (130, 1)])
def test_gsa_prefill_matches_oracle(Nc, BH):
    """Every raw and gist token's output under the gist mask, against the
    oracle's interleaved-sequence definition (partial workgroups of chunks
    and of gists, one chunk, a few)."""
    announce(f"gsa prefill Nc={Nc} BH={BH}")
    r = _rng(900 + Nc)
    chunk, D = 16, 128
    raw_cap = Nc * chunk + 5  # room past the last chunk, unused
    qr, qrh = dev_bf16(r.standard_normal((BH, Nc * chunk, D)))
    qg, qgh = dev_bf16(r.standard_normal((BH, Nc, D)))
    rk, rkh = dev_bf16(r.standard_normal((BH, raw_cap, D)))
    rv, rvh = dev_bf16(r.standard_normal((BH, raw_cap, D)))
    gk, gkh = dev_bf16(r.standard_normal((BH, Nc, D)))
    gv, gvh = dev_bf16(r.standard_normal((BH, Nc, D)))
    scale = 1.0 / math.sqrt(D)
    out_r, out_g = lct.gsa_prefill(qr, qg, rk, rv, gk, gv, scale)
    out_r, out_g = host(out_r), host(out_g)
    for b in range(BH):
        want_r, want_g = oracle.gsa_prefill(qrh[b], qgh[b], rkh[b, :Nc * chunk], rvh[b, :Nc * chunk], gkh[b],
                                            gvh[b], chunk, scale)
        assert np.abs(out_r[b] - want_r).max() < ATOL, b
        assert np.abs(out_g[b] - want_g).max() < ATOL, b


@pytest.mark.parametrize("scale", [1.0, 4.0])
def test_gsa_prefill_large_logits(scale):
    """Logits of tens to hundreds with key norms growing along the sequence:
    the running softmax reference keeps moving (the output is rescaled on
    many tiles) and a tile's weights reach the 2^8 headroom; outputs stay
    within the bar."""
    announce(f"gsa prefill large logits scale={scale}")
    r = _rng(77)
    BH, Nc, chunk, D = 1, 67, 16, 128
    n_raw = Nc * chunk
    ramp_r = np.linspace(0.2, 2.0, n_raw)[None, :, None]
    ramp_g = np.linspace(0.2, 2.0, Nc)[None, :, None]
    qr, qrh = dev_bf16(r.standard_normal((BH, n_raw, D)))
    qg, qgh = dev_bf16(r.standard_normal((BH, Nc, D)))
    rk, rkh = dev_bf16(r.standard_normal((BH, n_raw, D)) * ramp_r)
    rv, rvh = dev_bf16(r.standard_normal((BH, n_raw, D)))
    gk, gkh = dev_bf16(r.standard_normal((BH, Nc, D)) * ramp_g)
    gv, gvh = dev_bf16(r.standard_normal((BH, Nc, D)))
    out_r, out_g = lct.gsa_prefill(qr, qg, rk, rv, gk, gv, scale)
    out_r, out_g = host(out_r), host(out_g)
    want_r, want_g = oracle.gsa_prefill(qrh[0], qgh[0], rkh[0], rvh[0], gkh[0], gvh[0], chunk, scale)
    assert np.isfinite(out_r).all() and np.isfinite(out_g).all()
    assert np.abs(out_r[0] - want_r).max() < ATOL
    assert np.abs(out_g[0] - want_g).max() < ATOL


@pytest.mark.parametrize("D", [64, 256])
def test_gist_score_other_head_dims(D):
    """The gist scorer's 64- and 256-feature instances (the decode workload
    uses 128): integer-valued bf16 inputs, so every score is exact in fp32;
    Nc ragged against the 512-gist tiles."""
    announce(f"gist score D={D}")
    r = _rng(40 + D)
    BH, Nc = 3, 1500
    q, qh = dev_bf16(r.integers(-8, 8, size=(BH, D)).astype(np.float32))
    gk, gkh = dev_bf16(r.integers(-8, 8, size=(BH, Nc, D)).astype(np.float32))
    got = host(lct.gist_score(q, gk))
    assert np.array_equal(got, oracle.gist_scores(qh, gkh))


def test_gsa_raw_path_sensitivity():
    """Ternary gist keys keep gist logits small so raw tokens carry real weight."""
    from tests.gpu_util import dev_bf16_bits
    announce("gsa ternary gists")
    r = _rng(12)
    BH, Nc, D, kc, tail = 5, 200, 128, 6, 3
    q, qh = dev_bf16(r.choice([-1.0, 0.0, 1.0], size=(BH, D)))
    gk, gkh = dev_bf16(r.choice([-1.0, 0.0, 1.0], size=(BH, Nc, D)))
    gv, gvh = dev_bf16(r.standard_normal((BH, Nc, D)))
    rk, rkh = dev_bf16(r.standard_normal((BH, Nc * 16 + 16, D)))
    rv, rvh = dev_bf16(r.standard_normal((BH, Nc * 16 + 16, D)))
    out, cidx = lct.gsa_decode(q, gk, gv, rk, rv, kc, tail, 1 / math.sqrt(D))
    sc = oracle.gist_scores(qh, gkh)
    ref_idx = oracle.select_topk(sc, kc)
    assert np.array_equal(host(cidx), ref_idx)
    got = host(out)
    for i in range(BH):
        raw, gid = oracle.gsa_key_positions(ref_idx[i], 16, Nc, tail)
        want = oracle.gsa_attention(qh[i], rkh[i, raw], rvh[i, raw], gkh[i, gid], gvh[i, gid], 1 / math.sqrt(D))
        assert np.abs(got[i] - want).max() < ATOL, i
