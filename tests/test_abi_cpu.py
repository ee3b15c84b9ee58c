"""The C-ABI library on the host: it loads, exports every declared symbol and
rejects bad arguments before touching a device (no GPU needed)."""

import ctypes
import os
import re

import pytest
import torch

import long_context_top_amd as lct

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lct.h")

pytestmark = pytest.mark.skipif(not os.path.exists(lct.LIB_PATH),
                                reason="liblct.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lct_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert names == sorted([
        "lct_version", "lct_last_error", "lct_idx_score_i8", "lct_gist_score_bf16",
        "lct_topk_select", "lct_topk_workspace_bytes", "lct_sparse_attn_gather",
        "lct_sparse_attn_workspace_bytes", "lct_gsa_attn", "lct_gsa_attn_workspace_bytes",
        "lct_gsa_decode", "lct_gsa_decode_workspace_bytes", "lct_hgsa_decode",
        "lct_hgsa_decode_workspace_bytes", "lct_gsa_prefill", "lct_group_run",
        "lct_group_workspace_bytes", "lct_group_run_noalloc", "lct_prefill_index_i8",
        "lct_prefill_index_workspace_bytes"]), names
    so = ctypes.CDLL(lct.LIB_PATH)
    for n in names:
        assert hasattr(so, n), f"{n} declared in lct.h but not exported"
    # and the binding knows the signature of each
    assert set(names) <= set(lct._SIGS), set(names) - set(lct._SIGS)


def test_version_and_error_strings():
    assert "gfx950" in lct.version()
    L = lct.lib()
    rc = L.lct_idx_score_i8(None, None, None, 1, 1, 16, 64, -1, None)
    assert rc == lct.LCT_EINVAL
    assert b"null" in L.lct_last_error()


FAKE = ctypes.c_void_p(1 << 20)  # aligned non-null address; never dereferenced by these calls


def test_idx_score_validation():
    L = lct.lib()
    assert L.lct_idx_score_i8(FAKE, FAKE, FAKE, 0, 1, 16, 64, -1, None) == lct.LCT_EINVAL
    assert L.lct_idx_score_i8(FAKE, FAKE, FAKE, 1, 1, 0, 64, -1, None) == lct.LCT_EINVAL
    assert L.lct_idx_score_i8(FAKE, FAKE, FAKE, 1, 1, 16, 48, -1, None) == lct.LCT_EUNSUPPORTED
    assert L.lct_idx_score_i8(FAKE, FAKE, FAKE, 1, 1, 16, 1024, -1, None) == lct.LCT_EUNSUPPORTED
    assert L.lct_idx_score_i8(FAKE, FAKE, FAKE, 1, 64, 16, 32, 0, None) == lct.LCT_EUNSUPPORTED
    mis = ctypes.c_void_p((1 << 20) + 4)
    assert L.lct_idx_score_i8(mis, FAKE, FAKE, 1, 1, 16, 64, -1, None) == lct.LCT_EINVAL
    assert L.lct_idx_score_i8(FAKE, FAKE, FAKE, 1, 1, 1 << 31, 64, -1, None) == lct.LCT_EINVAL


def test_topk_validation_and_workspace_sizes():
    L = lct.lib()
    nb = ctypes.c_size_t()
    assert L.lct_topk_workspace_bytes(8, 131072, 2048, ctypes.byref(nb)) == 0
    assert nb.value > 8 * 131072 // 8  # few long rows: multi-workgroup scratch (bitmap and more)
    assert L.lct_topk_workspace_bytes(65536, 8192, 64, ctypes.byref(nb)) == 0
    assert nb.value == 0  # many rows: one workgroup per row, no scratch
    assert L.lct_topk_select(FAKE, 7, FAKE, 1, 10, 10, 3, None, FAKE, 1 << 21, None) == lct.LCT_EINVAL
    assert L.lct_topk_select(FAKE, 0, FAKE, 1, 10, 9, 3, None, FAKE, 1 << 21, None) == lct.LCT_EINVAL
    assert L.lct_topk_select(FAKE, 0, FAKE, 1, 10, 10, 0, None, FAKE, 1 << 21, None) == lct.LCT_EINVAL
    # multi-workgroup path with too small a workspace
    assert L.lct_topk_select(FAKE, 0, FAKE, 2, 200000, 200000, 64, None, FAKE, 4096, None) \
        == lct.LCT_ENOWORKSPACE


def test_attention_validation():
    L = lct.lib()
    args = [FAKE] * 5
    ws = FAKE
    # D other than 128
    assert L.lct_sparse_attn_gather(*args, 1, 1, 8, 2, 64, 100, 16, 0.1, ws, 1 << 22, None) \
        == lct.LCT_EUNSUPPORTED
    # Hq not a multiple of Hkv
    assert L.lct_sparse_attn_gather(*args, 1, 1, 6, 4, 128, 100, 16, 0.1, ws, 1 << 22, None) \
        == lct.LCT_EINVAL
    # group of 32 query heads per KV head
    assert L.lct_sparse_attn_gather(*args, 1, 1, 32, 1, 128, 100, 16, 0.1, ws, 1 << 22, None) \
        == lct.LCT_EUNSUPPORTED
    # non-finite scale
    assert L.lct_sparse_attn_gather(*args, 1, 1, 8, 1, 128, 100, 16, float("inf"), ws, 1 << 22, None) \
        == lct.LCT_EINVAL
    # too small workspace (2048 positions for one query row are split across workgroups)
    assert L.lct_sparse_attn_gather(*args, 1, 1, 8, 1, 128, 4096, 2048, 0.1, ws, 1024, None) \
        == lct.LCT_ENOWORKSPACE


def test_gsa_validation():
    L = lct.lib()
    p = [FAKE] * 7
    # raw_cap too small for the tail
    assert L.lct_gsa_attn(*p, 4, 128, 100, 1600, 16, 8, 1, 0.1, FAKE, 1 << 22, None) == lct.LCT_EINVAL
    # chunk other than 16
    assert L.lct_gsa_attn(*p, 4, 128, 100, 3300, 32, 8, 1, 0.1, FAKE, 1 << 22, None) == lct.LCT_EUNSUPPORTED
    # tail longer than a chunk
    assert L.lct_gsa_attn(*p, 4, 128, 100, 1700, 16, 8, 17, 0.1, FAKE, 1 << 22, None) == lct.LCT_EINVAL


def _desc(**kw):
    d = lct.GroupDesc()
    d.B, d.Lq, d.L, d.HD, d.Hq, d.Hkv, d.D = 2, 1, 4096, 256, 8, 2, 128
    d.topk, d.n_layers, d.layers_per_group, d.causal, d.scale = 64, 8, 4, 0, 0.088
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_group_validation_and_sizes():
    L = lct.lib()
    nb = ctypes.c_size_t()
    d = _desc()
    # pointer arrays missing
    assert L.lct_group_workspace_bytes(ctypes.byref(d), ctypes.byref(nb)) == lct.LCT_EINVAL
    arr_g = (ctypes.c_void_p * 2)(*([FAKE.value] * 2))
    arr_l = (ctypes.c_void_p * 8)(*([FAKE.value] * 8))
    P = ctypes.POINTER(ctypes.c_void_p)
    d.qi = ctypes.cast(arr_g, P)
    d.ki = ctypes.cast(arr_g, P)
    d.q = d.k = d.v = d.out = ctypes.cast(arr_l, P)
    assert L.lct_group_workspace_bytes(ctypes.byref(d), ctypes.byref(nb)) == 0
    scores = 2 * 1 * 4096 * 4
    assert nb.value >= scores
    bad = _desc(n_layers=6)
    bad.qi, bad.ki, bad.q, bad.k, bad.v, bad.out = d.qi, d.ki, d.q, d.k, d.v, d.out
    assert L.lct_group_workspace_bytes(ctypes.byref(bad), ctypes.byref(nb)) == lct.LCT_EINVAL
    causal_bad = _desc(causal=1)
    causal_bad.qi, causal_bad.ki, causal_bad.q = d.qi, d.ki, d.q
    causal_bad.k, causal_bad.v, causal_bad.out = d.k, d.v, d.out
    assert L.lct_group_workspace_bytes(ctypes.byref(causal_bad), ctypes.byref(nb)) == lct.LCT_EINVAL
    assert L.lct_group_run(ctypes.byref(d), FAKE, 1024, None) == lct.LCT_ENOWORKSPACE
    # a Full/Shared pattern lifts the multiple-of-group rule; its first layer must be Full
    U8 = ctypes.POINTER(ctypes.c_uint8)
    pat = (ctypes.c_uint8 * 6)(1, 0, 1, 1, 0, 0)
    free = _desc(n_layers=6, layers_per_group=0)
    arr_3 = (ctypes.c_void_p * 3)(*([FAKE.value] * 3))  # one indexer tensor per Full layer
    free.qi = free.ki = ctypes.cast(arr_3, P)
    free.q, free.k, free.v, free.out = d.q, d.k, d.v, d.out
    free.layer_full = ctypes.cast(pat, U8)
    assert L.lct_group_workspace_bytes(ctypes.byref(free), ctypes.byref(nb)) == 0
    pat[0] = 0
    assert L.lct_group_workspace_bytes(ctypes.byref(free), ctypes.byref(nb)) == lct.LCT_EINVAL


def test_group_noalloc_limit():
    """The no-allocation driver: the header's limit matches the binding's, the
    decode workloads fit it, and a step that does not fit is refused before
    any device work."""
    text = open(HEADER).read()
    m = re.search(r"#define LCT_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == lct.NOALLOC_SCRATCH_BYTES
    L = lct.lib()
    nb = ctypes.c_size_t()
    P = ctypes.POINTER(ctypes.c_void_p)
    arr = (ctypes.c_void_p * 28)(*([FAKE.value] * 28))
    for Lc, B in ((131072, 8), (32768, 8), (1 << 20, 1)):
        d = _desc(B=B, L=Lc, Hq=32, Hkv=4, topk=2048, n_layers=28)
        d.qi = d.ki = d.q = d.k = d.v = d.out = ctypes.cast(arr, P)
        assert L.lct_group_workspace_bytes(ctypes.byref(d), ctypes.byref(nb)) == 0
        assert nb.value <= lct.NOALLOC_SCRATCH_BYTES, (Lc, B, nb.value)
    big = _desc(B=1, Lq=65536, L=65536, Hq=32, Hkv=4, topk=2048, n_layers=28, causal=1)
    big.qi = big.ki = big.q = big.k = big.v = big.out = ctypes.cast(arr, P)
    assert L.lct_group_workspace_bytes(ctypes.byref(big), ctypes.byref(nb)) == 0
    assert nb.value > lct.NOALLOC_SCRATCH_BYTES
    assert L.lct_group_run_noalloc(ctypes.byref(big), None) == lct.LCT_ENOWORKSPACE
    assert b"scratch" in L.lct_last_error()


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a GPU is present")
def test_no_device_reports_enodev():
    L = lct.lib()
    # valid arguments for the one-workgroup-per-row select, which needs no workspace
    rc = L.lct_topk_select(FAKE, 0, FAKE, 100, 10, 10, 3, None, None, 0, None)
    assert rc == lct.LCT_ENODEV, (rc, L.lct_last_error())


def test_binding_refuses_host_tensors():
    with pytest.raises((ValueError, TypeError)):
        lct.idx_score(torch.zeros((1, 1, 64), dtype=torch.int8), torch.zeros((1, 8, 64), dtype=torch.int8))


def test_prefill_index_validation_and_sizing():
    L = lct.lib()
    nb = ctypes.c_size_t(0)
    # fused shape: the candidate lists (5120 per row) dominate
    assert L.lct_prefill_index_workspace_bytes(65536, 256, 2048, ctypes.byref(nb)) == lct.LCT_OK
    assert nb.value >= 65536 * 5120 * 4
    # other HD: one block of int32 score rows
    assert L.lct_prefill_index_workspace_bytes(4096, 128, 64, ctypes.byref(nb)) == lct.LCT_OK
    assert nb.value >= 128 * 4096 * 4
    assert L.lct_prefill_index_workspace_bytes(4096, 32, 64, ctypes.byref(nb)) == lct.LCT_EUNSUPPORTED
    assert L.lct_prefill_index_workspace_bytes(0, 256, 64, ctypes.byref(nb)) == lct.LCT_EINVAL
    assert L.lct_prefill_index_workspace_bytes((1 << 18) + 1, 256, 64, ctypes.byref(nb)) == lct.LCT_EUNSUPPORTED
    rc = L.lct_prefill_index_i8(None, None, None, 4096, 256, 64, None, 0, None, None)
    assert rc == lct.LCT_EINVAL
    assert "null" in lct.lib().lct_last_error().decode()


def test_sparse_attn_workspace_sizes():
    L = lct.lib()
    nb = ctypes.c_size_t()
    # one decode row per batch entry: split partials only
    assert L.lct_sparse_attn_workspace_bytes(8, 1, 32, 4, 128, 131072, 2048, ctypes.byref(nb)) == 0
    small = nb.value
    assert small <= 8 * 4 * 64 * 16 * 132 * 4
    # 64K causal prefill rows: position-segment partials (O, m, l per row, KV head,
    # query head and segment; at least two segments) and per-row bounds
    assert L.lct_sparse_attn_workspace_bytes(1, 65536, 32, 4, 128, 65536, 2048, ctypes.byref(nb)) == 0
    assert nb.value >= 65536 * 4 * 2 * 8 * 130 * 4 + 65536 * 3 * 4
    # Hq not a multiple of Hkv
    assert L.lct_sparse_attn_workspace_bytes(1, 1, 6, 4, 128, 1000, 16, ctypes.byref(nb)) == lct.LCT_EINVAL


def test_hgsa_validation():
    L = lct.lib()
    p = [FAKE] * 8
    ws = FAKE
    # km above the number of meta-gists (ceil(1000 / 64) = 16)
    assert L.lct_hgsa_decode(*p, 4, 128, 1000, 1000 * 16 + 16, 16, 64, 17, 8, 1, 0.1, ws, 1 << 26,
                             None) == lct.LCT_EINVAL
    # candidates km * group above 4096
    assert L.lct_hgsa_decode(*p, 4, 128, 100000, 100000 * 16 + 16, 16, 128, 40, 8, 1, 0.1, ws, 1 << 30,
                             None) == lct.LCT_EUNSUPPORTED
    # group 0
    assert L.lct_hgsa_decode(*p, 4, 128, 1000, 1000 * 16 + 16, 16, 0, 1, 8, 1, 0.1, ws, 1 << 26,
                             None) == lct.LCT_EINVAL
    nb = ctypes.c_size_t()
    assert L.lct_hgsa_decode_workspace_bytes(16, 128, 8192, 64, 1, ctypes.byref(nb)) == 0
    assert nb.value >= 16 * 8192 * 4 + 16 * 64 * 4


def test_gsa_prefill_validation():
    L = lct.lib()
    p = [FAKE] * 8
    # raw_cap too small
    assert L.lct_gsa_prefill(*p, 2, 128, 100, 1599, 16, 0.1, None) == lct.LCT_EINVAL
    # chunk other than 16, head dim other than 128
    assert L.lct_gsa_prefill(*p, 2, 128, 100, 3200, 32, 0.1, None) == lct.LCT_EUNSUPPORTED
    assert L.lct_gsa_prefill(*p, 2, 64, 100, 1600, 16, 0.1, None) == lct.LCT_EUNSUPPORTED
