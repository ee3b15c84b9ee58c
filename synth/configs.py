"""Workload shapes and tensor identities for the five synthetic workloads.

Shapes follow the Qwen2-7B geometry the long-context tutorial page uses
for its KV-cache arithmetic (28 layers, 4 KV heads, head dim 128, bf16),
with the indexer and sharing parameters of the DSA / IndexShare pages
(int8 lightning indexer, top-2048, one index per group of 4 layers) and
the gist-chunk layout of the GSA/SSA pages (chunks of 16 raw tokens, each
followed by one gist).  No arithmetic of the method lives here.

Tensor identities (the ``tid`` given to the generator) are
``kind_code << 16 | index`` with the index a group or layer number.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

from . import BF16N, BF16U4, I8U4, tensor, values

# tensor kind codes
T_QI, T_KI, T_Q, T_K, T_V = 1, 2, 3, 4, 5
T_GQ, T_GK, T_GV, T_RK, T_RV = 6, 7, 8, 9, 10
T_MK = 11  # meta-gist keys (hierarchical GSA)
T_QR, T_QG = 12, 13  # prefill queries of raw and gist tokens (GSA)


def tid(kind_code: int, index: int = 0) -> int:
    return (kind_code << 16) | index


@dataclass(frozen=True)
class DecodeConfig:
    """Token-level routed sparse attention with a shared index.

    ``Lq`` query rows per batch entry all attend over the same ``L`` cached
    positions; each row has its own index set.  With ``causal`` set, query
    row ``r`` sits at position ``r`` (``Lq == L``) and may only see
    positions ``<= r`` (causal prefill).  With ``shared_kv`` every layer
    reads the one KV cache of layer 0 (YOCO / CLSA cross-layer KV sharing);
    the queries stay per layer.
    """

    name: str
    seed: int
    B: int
    Lq: int
    L: int
    n_layers: int
    group: int
    Hq: int
    Hkv: int
    D: int
    H_idx: int
    d_idx: int
    topk: int
    causal: bool = False
    shared_kv: bool = False

    @property
    def HD(self) -> int:
        return self.H_idx * self.d_idx

    @property
    def n_groups(self) -> int:
        return self.n_layers // self.group

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    # ---- tensor specs: (kind, shape, tid) ----
    def qi_spec(self, g):
        return I8U4, (self.B, self.Lq, self.HD), tid(T_QI, g)

    def ki_spec(self, g):
        return I8U4, (self.B, self.L, self.HD), tid(T_KI, g)

    def q_spec(self, l):
        return BF16N, (self.B, self.Lq, self.Hq, self.D), tid(T_Q, l)

    def kv_layer(self, l):
        """The layer whose KV cache layer ``l`` reads."""
        return 0 if self.shared_kv else l

    def k_spec(self, l):
        return BF16N, (self.B, self.L, self.Hkv, self.D), tid(T_K, self.kv_layer(l))

    def v_spec(self, l):
        return BF16N, (self.B, self.L, self.Hkv, self.D), tid(T_V, self.kv_layer(l))

    def with_(self, **kw) -> "DecodeConfig":
        return replace(self, **kw)


@dataclass(frozen=True)
class GsaConfig:
    """Gist-chunk select-and-unfold decode (one layer, MHA).

    Raw positions ``[c*chunk, (c+1)*chunk)`` form chunk ``c`` and gist ``c``
    follows it.  The current token opens the unfinished chunk ``Nc``; its
    ``tail_len`` raw positions ``[Nc*chunk, Nc*chunk + tail_len)`` are always
    attended.  The raw arrays hold room for one full unfinished chunk.

    Hierarchical routing (``group`` > 0): meta-gist ``g`` summarises gists
    ``[g*group, (g+1)*group)``; the ``km`` best meta-gists are chosen first
    and the ``kc`` chunks only among their gists.
    """

    name: str
    seed: int
    B: int
    H: int
    D: int
    Nc: int
    chunk: int
    kc: int
    tail_len: int
    gist_kind: int = BF16U4
    group: int = 0
    km: int = 0

    @property
    def Nm(self) -> int:
        return -(-self.Nc // self.group) if self.group else 0

    @property
    def raw_cap(self) -> int:
        return self.Nc * self.chunk + self.chunk

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def q_spec(self):
        return BF16U4, (self.B, self.H, self.D), tid(T_GQ)

    def gk_spec(self):
        return self.gist_kind, (self.B, self.H, self.Nc, self.D), tid(T_GK)

    def gv_spec(self):
        return BF16N, (self.B, self.H, self.Nc, self.D), tid(T_GV)

    def mk_spec(self):
        return self.gist_kind, (self.B, self.H, self.Nm, self.D), tid(T_MK)

    def qr_spec(self):
        """Prefill: the raw tokens' queries."""
        return BF16N, (self.B, self.H, self.Nc * self.chunk, self.D), tid(T_QR)

    def qg_spec(self):
        """Prefill: the gist tokens' queries."""
        return BF16N, (self.B, self.H, self.Nc, self.D), tid(T_QG)

    def rk_spec(self):
        return BF16N, (self.B, self.H, self.raw_cap, self.D), tid(T_RK)

    def rv_spec(self):
        return BF16N, (self.B, self.H, self.raw_cap, self.D), tid(T_RV)

    def with_(self, **kw) -> "GsaConfig":
        return replace(self, **kw)


# The five workloads.
TINY = DecodeConfig("tiny_decode_2k", 1001, B=1, Lq=16, L=2048, n_layers=4, group=4,
                    Hq=8, Hkv=1, D=128, H_idx=1, d_idx=64, topk=128)
DECODE_32K = DecodeConfig("sparse_decode_32k_b8", 1002, B=8, Lq=1, L=32768, n_layers=28,
                          group=4, Hq=32, Hkv=4, D=128, H_idx=4, d_idx=64, topk=2048)
DECODE_128K = DECODE_32K.with_(name="sparse_decode_128k_b8", L=131072)
# the 128K decode with one KV cache for all 28 layers (YOCO / CLSA)
DECODE_128K_SHARED_KV = DECODE_128K.with_(name="sparse_decode_128k_b8_shared_kv", shared_kv=True)
PREFILL_64K = DecodeConfig("causal_prefill_64k", 1003, B=1, Lq=65536, L=65536, n_layers=28,
                           group=4, Hq=32, Hkv=4, D=128, H_idx=4, d_idx=64, topk=2048,
                           causal=True)
GSA_128K = GsaConfig("gsa_decode_128k_b16", 1004, B=16, H=16, D=128, Nc=8192, chunk=16,
                     kc=64, tail_len=1)
# GSA 128K with coarse-to-fine routing: 128 meta-gists of 64 gists each, 4
# groups chosen, then the 64 best of their 256 chunks
HGSA_128K = GSA_128K.with_(name="hgsa_decode_128k_b16", seed=1006, group=64, km=4)
# GSA prefill under the gist mask: 128K raw tokens (8192 chunks + their
# gists) for one sequence, 16 heads (the GSA decode workload's context)
GSA_PREFILL_128K = GsaConfig("gsa_prefill_128k_h16", 1007, B=1, H=16, D=128, Nc=8192, chunk=16, kc=64,
                             tail_len=0)
DECODE_1M = DecodeConfig("sparse_decode_1m_b1", 1005, B=1, Lq=1, L=1048576, n_layers=28,
                         group=4, Hq=32, Hkv=4, D=128, H_idx=4, d_idx=64, topk=2048)

ALL = {c.name: c for c in (TINY, DECODE_32K, DECODE_128K, PREFILL_64K, GSA_128K, DECODE_1M,
                           DECODE_128K_SHARED_KV, HGSA_128K, GSA_PREFILL_128K)}


# ---- host-side generation helpers ----

def raise_if_huge(shape, limit=1 << 28):
    n = int(np.prod(shape))
    if n > limit:
        raise MemoryError(f"refusing to generate {n} elements on the host")


def make(cfg, spec) -> np.ndarray:
    """Generate a whole tensor of ``cfg`` on the host."""
    kind, shape, t = spec
    raise_if_huge(shape)
    return tensor(kind, cfg.seed, t, shape)


def rows(cfg, spec, lead_index: tuple) -> np.ndarray:
    """Regenerate only selected leading-index rows of a tensor.

    ``lead_index`` is a tuple of integer arrays (broadcast together) that
    index the leading ``len(lead_index)`` dimensions; the trailing
    dimensions are returned whole.  Output shape is
    ``broadcast(lead_index).shape + shape[len(lead_index):]``.
    """
    kind, shape, t = spec
    nl = len(lead_index)
    idx = np.broadcast_arrays(*[np.asarray(a, dtype=np.int64) for a in lead_index])
    lead_shape = idx[0].shape
    flat_lead = np.zeros(lead_shape, dtype=np.int64)
    for a, n in zip(idx, shape[:nl]):
        if np.any((a < 0) | (a >= n)):
            raise IndexError("row index out of range")
        flat_lead = flat_lead * n + a
    trail = shape[nl:]
    tn = int(np.prod(trail)) if trail else 1
    flat = flat_lead[..., None] * tn + np.arange(tn, dtype=np.int64)
    out = values(kind, cfg.seed, t, flat.reshape(-1))
    return out.reshape(lead_shape + tuple(trail))
