"""Python binding of liblct: routed top-k sparse attention with a shared index.

Argument marshalling only: every step of the path runs in the gfx950 kernels
of ``liblct.so`` (C-ABI declared in ``include/lct.h``).  PyTorch supplies
device memory and the current HIP stream.  There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

__all__ = [
    "LctError", "Workspace", "lib", "version", "idx_score", "gist_score", "topk_select",
    "sparse_attn_gather", "gsa_attn", "gsa_decode", "group_run", "GroupRun",
]

LCT_OK, LCT_EINVAL, LCT_EUNSUPPORTED, LCT_ENOWORKSPACE, LCT_ENODEV, LCT_EHIP = range(6)
LCT_I32, LCT_F32 = 0, 1
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblct.so")
NOALLOC_SCRATCH_BYTES = 32 << 20  # LCT_NOALLOC_SCRATCH_BYTES in lct.h

_c = ctypes
_vp, _i32, _i64, _f32, _sz = _c.c_void_p, _c.c_int, _c.c_int64, _c.c_float, _c.c_size_t


class LctError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"lct error {code}: {msg}")
        self.code = code


class GroupDesc(_c.Structure):
    """Mirror of ``lct_group_desc``."""

    _fields_ = [
        ("B", _i32), ("Lq", _i32), ("L", _i64), ("HD", _i32), ("Hq", _i32), ("Hkv", _i32),
        ("D", _i32), ("topk", _i32), ("n_layers", _i32), ("layers_per_group", _i32),
        ("causal", _i32), ("scale", _f32), ("valid_len", _vp), ("qi", _c.POINTER(_vp)),
        ("ki", _c.POINTER(_vp)), ("q", _c.POINTER(_vp)), ("k", _c.POINTER(_vp)),
        ("v", _c.POINTER(_vp)), ("out", _c.POINTER(_vp)), ("idx_out", _c.POINTER(_vp)),
        ("layer_idx_seen", _c.POINTER(_vp)), ("layer_full", _c.POINTER(_c.c_uint8)),
    ]


_SIGS = {
    "lct_version": ([], _c.c_char_p),
    "lct_last_error": ([], _c.c_char_p),
    "lct_idx_score_i8": ([_vp, _vp, _vp, _i32, _i32, _i64, _i32, _i64, _vp], _i32),
    "lct_prefill_index_i8": ([_vp, _vp, _vp, _i64, _i32, _i32, _vp, _sz, _vp, _vp], _i32),
    "lct_prefill_index_workspace_bytes": ([_i64, _i32, _i32, _c.POINTER(_sz)], _i32),
    "lct_gist_score_bf16": ([_vp, _vp, _vp, _i32, _i64, _i32, _vp], _i32),
    "lct_topk_select": ([_vp, _i32, _vp, _i32, _i64, _i64, _i32, _vp, _vp, _sz, _vp], _i32),
    "lct_topk_workspace_bytes": ([_i32, _i64, _i32, _c.POINTER(_sz)], _i32),
    "lct_sparse_attn_gather": ([_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i64, _i32,
                                _f32, _vp, _sz, _vp], _i32),
    "lct_sparse_attn_workspace_bytes": ([_i32, _i32, _i32, _i32, _i32, _i64, _i32, _c.POINTER(_sz)],
                                        _i32),
    "lct_gsa_attn": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i64, _i64, _i32, _i32, _i32,
                      _f32, _vp, _sz, _vp], _i32),
    "lct_gsa_decode": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i64, _i64, _i32, _i32, _i32,
                        _f32, _vp, _sz, _vp], _i32),
    "lct_gsa_decode_workspace_bytes": ([_i32, _i32, _i64, _i32, _c.POINTER(_sz)], _i32),
    "lct_gsa_attn_workspace_bytes": ([_i32, _i32, _i32, _i32, _c.POINTER(_sz)], _i32),
    "lct_hgsa_decode": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i64, _i64, _i32, _i32, _i32,
                         _i32, _i32, _f32, _vp, _sz, _vp], _i32),
    "lct_hgsa_decode_workspace_bytes": ([_i32, _i32, _i64, _i32, _i32, _c.POINTER(_sz)], _i32),
    "lct_gsa_prefill": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i64, _i64, _i32, _f32, _vp], _i32),
    "lct_group_run": ([_c.POINTER(GroupDesc), _vp, _sz, _vp], _i32),
    "lct_group_workspace_bytes": ([_c.POINTER(GroupDesc), _c.POINTER(_sz)], _i32),
    "lct_group_run_noalloc": ([_c.POINTER(GroupDesc), _vp], _i32),
}

_lib = None


def lib():
    """The loaded ``liblct.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        l = _c.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(l, name)
            f.argtypes = args
            f.restype = res
        _lib = l
    return _lib


def version() -> str:
    return lib().lct_version().decode()


def _check(rc: int):
    if rc != LCT_OK:
        raise LctError(rc, lib().lct_last_error().decode())


def _p(t: Optional[torch.Tensor]):
    return None if t is None else _vp(t.data_ptr())


def _stream():
    return _vp(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, dtype, name, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


class Workspace:
    """Caller-owned scratch memory (a device byte buffer) that grows on demand."""

    def __init__(self, device=None):
        self.device = torch.device("cuda") if device is None else torch.device(device)
        self.buf: Optional[torch.Tensor] = None

    def get(self, nbytes: int) -> torch.Tensor:
        nbytes = max(int(nbytes), 256)
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = None
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return self.buf

    @property
    def nbytes(self) -> int:
        return 0 if self.buf is None else self.buf.numel()


_default_ws: dict = {}


def _ws(ws: Optional[Workspace]) -> Workspace:
    if ws is not None:
        return ws
    dev = torch.cuda.current_device()
    if dev not in _default_ws:
        _default_ws[dev] = Workspace(torch.device("cuda", dev))
    return _default_ws[dev]


# ----------------------------------------------------------------- calls ----

def idx_score(q: torch.Tensor, k: torch.Tensor, q_pos0: int = -1,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """int8 q [B, Lq, HD], k [B, L, HD] -> int32 scores [B, Lq, L]."""
    _need(q, torch.int8, "q")
    _need(k, torch.int8, "k")
    B, Lq, HD = q.shape
    L = k.shape[1]
    if out is None:
        out = torch.empty((B, Lq, L), dtype=torch.int32, device=q.device)
    _need(out, torch.int32, "out")
    _check(lib().lct_idx_score_i8(_p(q), _p(k), _p(out), B, Lq, L, HD, q_pos0, _stream()))
    return out


def prefill_index(q: torch.Tensor, k: torch.Tensor, topk: int, out: Optional[torch.Tensor] = None,
                  ws: Optional[Workspace] = None, stats: Optional[dict] = None) -> torch.Tensor:
    """Causal index of one group: int8 q, k [L, HD] -> int32 [L, topk].

    Row i lists the min(topk, i + 1) positions t <= i with the largest
    q[i].k[t] (ties to the lower position), ascending, -1 padded.  With
    ``stats`` given, ``stats["n_fallback"]`` receives the number of rows the
    fused filter left to the whole-row select (read after the stream is done:
    the call itself never waits).
    """
    _need(q, torch.int8, "q")
    _need(k, torch.int8, "k")
    L, HD = q.shape
    if tuple(k.shape) != (L, HD):
        raise ValueError("q and k must both be [L, HD]")
    if out is None:
        out = torch.empty((L, topk), dtype=torch.int32, device=q.device)
    _need(out, torch.int32, "out")
    nb = _sz()
    _check(lib().lct_prefill_index_workspace_bytes(L, HD, topk, _c.byref(nb)))
    buf = _ws(ws).get(nb.value)
    nf = None if stats is None else torch.zeros(1, dtype=torch.int32, device=q.device)
    _check(lib().lct_prefill_index_i8(_p(q), _p(k), _p(out), L, HD, topk, _p(buf), buf.numel(),
                                      _p(nf), _stream()))
    if stats is not None:
        stats["n_fallback"] = int(nf.item())   # waits for the stream (only when asked)
    return out


def gist_score(q: torch.Tensor, gk: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 q [BH, D], gk [BH, Nc, D] -> fp32 [BH, Nc] (unscaled dot products)."""
    _need(q, torch.bfloat16, "q")
    _need(gk, torch.bfloat16, "gk")
    BH, Nc, D = gk.shape
    if out is None:
        out = torch.empty((BH, Nc), dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out")
    _check(lib().lct_gist_score_bf16(_p(q), _p(gk), _p(out), BH, Nc, D, _stream()))
    return out


def topk_select(scores: torch.Tensor, k: int, valid_len: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, ws: Optional[Workspace] = None) -> torch.Tensor:
    """int32/fp32 scores [rows, n] -> int32 [rows, k] ascending positions, -1 padded."""
    if scores.dtype not in (torch.int32, torch.float32):
        raise TypeError("scores must be int32 or float32")
    _need(scores, scores.dtype, "scores")
    rows, n = scores.shape
    if out is None:
        out = torch.empty((rows, k), dtype=torch.int32, device=scores.device)
    _need(out, torch.int32, "out")
    if valid_len is not None:
        _need(valid_len, torch.int32, "valid_len")
    nb = _sz()
    _check(lib().lct_topk_workspace_bytes(rows, n, k, _c.byref(nb)))
    buf = _ws(ws).get(nb.value)
    dt = LCT_I32 if scores.dtype == torch.int32 else LCT_F32
    _check(lib().lct_topk_select(_p(scores), dt, _p(out), rows, n, n, k, _p(valid_len), _p(buf),
                                 buf.numel(), _stream()))
    return out


def sparse_attn_gather(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor,
                       scale: float, out: Optional[torch.Tensor] = None,
                       ws: Optional[Workspace] = None) -> torch.Tensor:
    """bf16 q [B, Lq, Hq, D]; k, v [B, L, Hkv, D]; idx [B, Lq, kk] -> fp32 [B, Lq, Hq, D]."""
    _need(q, torch.bfloat16, "q")
    _need(k, torch.bfloat16, "k")
    _need(v, torch.bfloat16, "v")
    _need(idx, torch.int32, "idx")
    B, Lq, Hq, D = q.shape
    L, Hkv = k.shape[1], k.shape[2]
    kk = idx.shape[-1]
    if out is None:
        out = torch.empty((B, Lq, Hq, D), dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out")
    nb = _sz()
    _check(lib().lct_sparse_attn_workspace_bytes(B, Lq, Hq, Hkv, D, L, kk, _c.byref(nb)))
    buf = _ws(ws).get(nb.value)
    _check(lib().lct_sparse_attn_gather(_p(q), _p(k), _p(v), _p(idx), _p(out), B, Lq, Hq, Hkv, D, L,
                                        kk, scale, _p(buf), buf.numel(), _stream()))
    return out


def gsa_attn(q, rk, rv, gv, gscores, chunk_idx, tail_len: int, scale: float, chunk: int = 16,
             out=None, ws: Optional[Workspace] = None) -> torch.Tensor:
    """One query per (batch x head) row: unfold the chosen chunks (raw + gist) and the tail."""
    for t, n in ((q, "q"), (rk, "rk"), (rv, "rv"), (gv, "gv")):
        _need(t, torch.bfloat16, n)
    _need(gscores, torch.float32, "gscores")
    _need(chunk_idx, torch.int32, "chunk_idx")
    BH, D = q.shape
    Nc = gv.shape[1]
    raw_cap = rk.shape[1]
    kc = chunk_idx.shape[-1]
    if out is None:
        out = torch.empty((BH, D), dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out")
    nb = _sz()
    _check(lib().lct_gsa_attn_workspace_bytes(BH, D, kc, tail_len, _c.byref(nb)))
    buf = _ws(ws).get(nb.value)
    _check(lib().lct_gsa_attn(_p(q), _p(rk), _p(rv), _p(gv), _p(gscores), _p(chunk_idx), _p(out), BH,
                              D, Nc, raw_cap, chunk, kc, tail_len, scale, _p(buf), buf.numel(),
                              _stream()))
    return out


def gsa_decode(q, gk, gv, rk, rv, kc: int, tail_len: int, scale: float, chunk: int = 16,
               idx_out=None, out=None, ws: Optional[Workspace] = None):
    """Gist scores, top-kc chunks, unfold attention.  Returns (out, chunk_idx)."""
    for t, n in ((q, "q"), (gk, "gk"), (gv, "gv"), (rk, "rk"), (rv, "rv")):
        _need(t, torch.bfloat16, n)
    BH, D = q.shape
    Nc = gk.shape[1]
    raw_cap = rk.shape[1]
    if out is None:
        out = torch.empty((BH, D), dtype=torch.float32, device=q.device)
    if idx_out is None:
        idx_out = torch.empty((BH, kc), dtype=torch.int32, device=q.device)
    _need(out, torch.float32, "out")
    _need(idx_out, torch.int32, "idx_out")
    nb = _sz()
    _check(lib().lct_gsa_decode_workspace_bytes(BH, D, Nc, kc, _c.byref(nb)))
    buf = _ws(ws).get(nb.value)
    _check(lib().lct_gsa_decode(_p(q), _p(gk), _p(gv), _p(rk), _p(rv), _p(idx_out), _p(out), BH, D,
                                Nc, raw_cap, chunk, kc, tail_len, scale, _p(buf), buf.numel(),
                                _stream()))
    return out, idx_out


def hgsa_decode(q, mk, gk, gv, rk, rv, group: int, km: int, kc: int, tail_len: int, scale: float,
                chunk: int = 16, idx_out=None, out=None, ws: Optional[Workspace] = None):
    """Coarse-to-fine routing (meta-gists, then gists of the km chosen groups,
    kc chunks), unfold attention.  Returns (out, chunk_idx)."""
    for t, n in ((q, "q"), (mk, "mk"), (gk, "gk"), (gv, "gv"), (rk, "rk"), (rv, "rv")):
        _need(t, torch.bfloat16, n)
    BH, D = q.shape
    Nc = gk.shape[1]
    raw_cap = rk.shape[1]
    if out is None:
        out = torch.empty((BH, D), dtype=torch.float32, device=q.device)
    if idx_out is None:
        idx_out = torch.empty((BH, kc), dtype=torch.int32, device=q.device)
    _need(out, torch.float32, "out")
    _need(idx_out, torch.int32, "idx_out")
    nb = _sz()
    _check(lib().lct_hgsa_decode_workspace_bytes(BH, D, Nc, kc, tail_len, _c.byref(nb)))
    buf = _ws(ws).get(nb.value)
    _check(lib().lct_hgsa_decode(_p(q), _p(mk), _p(gk), _p(gv), _p(rk), _p(rv), _p(idx_out), _p(out), BH,
                                 D, Nc, raw_cap, chunk, group, km, kc, tail_len, scale, _p(buf),
                                 buf.numel(), _stream()))
    return out, idx_out


def gsa_prefill(q_raw, q_gist, rk, rv, gk, gv, scale: float, chunk: int = 16, out_raw=None, out_gist=None):
    """Every raw and gist token's attention under the gist mask.
    q_raw [BH, Nc*chunk, D], q_gist [BH, Nc, D], rk/rv [BH, raw_cap, D], gk/gv [BH, Nc, D]
    -> (out_raw fp32 [BH, Nc*chunk, D], out_gist fp32 [BH, Nc, D])."""
    for t, n in ((q_raw, "q_raw"), (q_gist, "q_gist"), (rk, "rk"), (rv, "rv"), (gk, "gk"), (gv, "gv")):
        _need(t, torch.bfloat16, n)
    BH, Nc, D = gk.shape
    raw_cap = rk.shape[1]
    if q_raw.shape != (BH, Nc * chunk, D) or q_gist.shape != (BH, Nc, D):
        raise ValueError("q_raw must be [BH, Nc*chunk, D] and q_gist [BH, Nc, D]")
    if out_raw is None:
        out_raw = torch.empty((BH, Nc * chunk, D), dtype=torch.float32, device=gk.device)
    if out_gist is None:
        out_gist = torch.empty((BH, Nc, D), dtype=torch.float32, device=gk.device)
    _need(out_raw, torch.float32, "out_raw")
    _need(out_gist, torch.float32, "out_gist")
    _check(lib().lct_gsa_prefill(_p(q_raw), _p(q_gist), _p(rk), _p(rv), _p(gk), _p(gv), _p(out_raw), _p(out_gist),
                                 BH, D, Nc, raw_cap, chunk, scale, _stream()))
    return out_raw, out_gist


class GroupRun:
    """Prepared layer-group driver call (descriptor + workspace), reusable across steps.

    Holding the descriptor lets a caller replay the same step cheaply (and
    capture it in a HIP graph).  All tensors must stay alive while in use.
    """

    def __init__(self, qi: Sequence[torch.Tensor], ki: Sequence[torch.Tensor],
                 q: Sequence[torch.Tensor], k: Sequence[torch.Tensor], v: Sequence[torch.Tensor],
                 out: Sequence[torch.Tensor], topk: int, layers_per_group: int, scale: float,
                 causal: bool = False, valid_len: Optional[torch.Tensor] = None,
                 idx_out: Optional[Sequence[torch.Tensor]] = None, ws: Optional[Workspace] = None,
                 layer_full: Optional[Sequence[int]] = None):
        n_layers = len(q)
        if layer_full is not None:
            if len(layer_full) != n_layers:
                raise ValueError("layer_full needs one flag per layer")
            n_groups = sum(1 for f in layer_full if f)
        else:
            n_groups = n_layers // layers_per_group
        if len(qi) != n_groups or len(ki) != n_groups:
            raise ValueError("need one indexer query/key tensor per group")
        for t in qi:
            _need(t, torch.int8, "qi")
        for t in ki:
            _need(t, torch.int8, "ki")
        for lst, n in ((q, "q"), (k, "k"), (v, "v")):
            for t in lst:
                _need(t, torch.bfloat16, n)
        for t in out:
            _need(t, torch.float32, "out")
        if valid_len is not None:
            _need(valid_len, torch.int32, "valid_len")
        B, Lq, HD = qi[0].shape
        L = ki[0].shape[1]
        Hq, D = q[0].shape[2], q[0].shape[3]
        Hkv = k[0].shape[2]
        self._keep = [qi, ki, q, k, v, out, valid_len, idx_out]

        def arr(ts):
            a = (_vp * len(ts))()
            for i, t in enumerate(ts):
                a[i] = None if t is None else t.data_ptr()
            return a

        self._arrs = [arr(qi), arr(ki), arr(q), arr(k), arr(v), arr(out)]
        self._idx_arr = arr(idx_out) if idx_out is not None else None
        self._seen = (_vp * n_layers)()
        d = GroupDesc()
        d.B, d.Lq, d.L, d.HD, d.Hq, d.Hkv, d.D = B, Lq, L, HD, Hq, Hkv, D
        d.topk, d.n_layers, d.layers_per_group = topk, n_layers, layers_per_group
        d.causal, d.scale = int(causal), scale
        d.valid_len = None if valid_len is None else valid_len.data_ptr()
        d.qi, d.ki, d.q, d.k, d.v, d.out = [_c.cast(a, _c.POINTER(_vp)) for a in self._arrs]
        d.idx_out = None if self._idx_arr is None else _c.cast(self._idx_arr, _c.POINTER(_vp))
        d.layer_idx_seen = _c.cast(self._seen, _c.POINTER(_vp))
        self._full = None
        if layer_full is not None:
            self._full = (_c.c_uint8 * n_layers)(*[1 if f else 0 for f in layer_full])
            d.layer_full = _c.cast(self._full, _c.POINTER(_c.c_uint8))
        self.desc = d
        nb = _sz()
        _check(lib().lct_group_workspace_bytes(_c.byref(d), _c.byref(nb)))
        self.ws_bytes = nb.value
        self.ws = _ws(ws)
        self.buf = self.ws.get(self.ws_bytes)

    def __call__(self):
        _check(lib().lct_group_run(_c.byref(self.desc), _p(self.buf), self.buf.numel(), _stream()))

    def call_noalloc(self):
        """The same step through ``lct_group_run_noalloc`` (the library's own
        fixed scratch array instead of this object's workspace)."""
        _check(lib().lct_group_run_noalloc(_c.byref(self.desc), _stream()))

    def layer_index_addresses(self):
        """Device address of the index set each layer read in the last call."""
        return [self._seen[i] for i in range(len(self._seen))]


def group_run(qi, ki, q, k, v, topk: int, layers_per_group: int, scale: float, causal=False,
              valid_len=None, out=None, idx_out=None, ws: Optional[Workspace] = None,
              layer_full=None):
    """One decode step (or causal prefill) of a stack of layers; returns the outputs.

    ``layer_full`` (one flag per layer, first one set) places the Full layers
    freely; without it every ``layers_per_group``-th layer is Full."""
    if out is None:
        out = [torch.empty(t.shape, dtype=torch.float32, device=t.device) for t in q]
    run = GroupRun(qi, ki, q, k, v, out, topk, layers_per_group, scale, causal, valid_len,
                   idx_out, ws, layer_full)
    run()
    return out, run
