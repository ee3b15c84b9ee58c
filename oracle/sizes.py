"""Closed-form sizes and work counts printed on the tutorial page.

Source: "长上下文：稀疏注意力 / DSA / IndexShare" tutorial:

* KV-cache volume section: bytes = layers x KV heads x head dim x 2 (K and
  V) x bytes per element x tokens; about 56 KiB per token for the
  Qwen2-7B geometry (28 layers, 4 KV heads, head dim 128, bf16).
* Hands-on section ("动手：算清两堵墙"): the same formula evaluated at
  4096 / 131072 / 1,000,000 tokens, and the number of scored pairs at
  one million tokens for full attention, a sliding window of 8192 and
  top-2048 selection.
"""

from __future__ import annotations


def kv_bytes_per_token(n_layers: int, kv_heads: int, head_dim: int, bytes_per: int = 2) -> int:
    """Cache bytes one token adds: a K row and a V row of every KV head of every layer."""
    one_row = head_dim * bytes_per            # one head's K (or V) vector
    per_layer = 2 * kv_heads * one_row        # K and V for every KV head
    return n_layers * per_layer


def kv_cache_gib(n_layers: int, kv_heads: int, head_dim: int, n_tok: int, bytes_per: int = 2) -> float:
    """Whole cache for ``n_tok`` tokens, in GiB (2**30 bytes)."""
    total = n_tok * kv_bytes_per_token(n_layers, kv_heads, head_dim, bytes_per)
    return total / float(1 << 30)


def scored_pairs(n_tok: int, per_query: int | None = None) -> int:
    """Query-key pairs scored: all pairs (``per_query`` None) or a fixed budget per query."""
    return n_tok * n_tok if per_query is None else n_tok * per_query
