"""CPU oracle for routed top-k sparse attention with a cross-layer shared index.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or run anything here.
The product path (the HIP library and its Python binding) never imports
this package, and this package imports nothing from the product path; the
two share only the seeded input generator in ``synth``.

Everything here is the plain, slow definition of what the method computes:

* indexer scores in exact integer arithmetic (int64),
* top-k selection by a stable sort with the lowest position winning ties,
* softmax attention in float64 with the row sum checked,
* gist-chunk selection and unfolding (GSA/SSA) the same way,
* the layer-group driver that computes one index set per group of layers.

Sources (web pages on long-context sparse attention):

* "You Only Index Once" (CLSA) explainer -- section 1.1 (attention formula),
  sections 2.2-2.3 (indexer / selector / sharer workflow).
* "长上下文：稀疏注意力 / DSA / IndexShare" tutorial -- DSA and IndexShare
  section (lightning indexer, top-k, 4 layers share one index), KV-cache
  volume section and the hands-on arithmetic section.
* SSA article (arXiv 2604.20920) -- sections 2-3 (gist tokens, selective
  unfolding, keep selected chunks' gists with their raw tokens), section 4
  (the gist mask), section 5 (hierarchical gists), section 6 (key-order
  invariance and the permuted prefill, split decode with log-sum-exp merge).
* IndexCache article (arXiv 2603.12201) -- section 2 (Full / Shared layers),
  section 3 (the greedy search keeps Full layers at uneven places),
  section 6 (one conditional plus one temporary index buffer).
* GSA summary page (gist.science) -- section 2.2 (selective unfolding),
  section 2.4 (hierarchical gist-of-gist routing).

Pins (``tests/oracle_pins.py``, run by ``tests/test_oracle_pins.py``; each
pin is also run against copies with planted mistakes in
``tests/test_oracle_mutants.py``, which must fail it):

* ``index_scores``: one-hot keys, per-head block keys, the closed-form
  maximising key, additivity in the key (``pin_index_scores``);
* ``index_scores_row``: one-hot keys, closed-form maximum and minimum at the
  int8 extremes, a pure-Python sum of products (``pin_index_scores_row``);
* ``index_scores_f32``: equal to a pure-Python sum of products on random
  full-range int8 rows and at the int8 extremes, refusing head dims past
  its exactness bound (``pin_index_scores_f32``);
* ``select_topk`` and ``select_topk_threshold``: rank counting by brute
  force over tiny rows with massive ties and short valid lengths
  (``pin_topk``);
* ``softmax_attention`` / ``sparse_attention_gqa``: torch's
  ``scaled_dot_product_attention`` in float64, row sums, V = 1
  (``pin_attention``);
* the driver functions: one index computation per group, the Full/Shared
  pattern, dense equivalence when k covers the cache, planted needles,
  causal prefill rows below k against dense causal attention
  (``pin_driver_sharing``, ``pin_layer_pattern``, ``pin_dense_when_k_covers``,
  ``pin_needles``, ``pin_prefill``);
* the GSA functions: every chunk chosen equals dense attention over the whole
  cache, a planted chunk unfolds exactly its raw tokens, its gist and the
  tail (``pin_gsa_dense``, ``pin_gsa_sg_sr``); ``hgsa_select`` by brute force
  (``pin_hgsa_select``); ``hgsa_step`` equal to the flat step when every
  group is kept and a planted coarse-to-fine case (``pin_hgsa_step``); the
  gist-mask prefill against explicit softmax over the visible keys
  (``pin_gsa_prefill``);
* the sizes: the values printed on the tutorial page (``pin_sizes``).

Every function exported here has such a pin.
"""

from .indexer import index_scores, index_scores_f32, index_scores_row  # noqa: F401
from .topk import select_topk, select_topk_threshold  # noqa: F401
from .attention import softmax_attention, sparse_attention_gqa  # noqa: F401
from .gsa import (gist_scores, gsa_key_positions, gsa_attention, gsa_select, hgsa_select,  # noqa: F401
                  gsa_prefill, gsa_prefill_rows, gsa_prefill_visible)
from .driver import (decode_group, decode_layers, decode_step, decode_step_pattern,  # noqa: F401
                     gsa_step, hgsa_step, layer_owner, prefill_attention_rows, prefill_index_rows)
from .sizes import kv_cache_gib, kv_bytes_per_token, scored_pairs  # noqa: F401
