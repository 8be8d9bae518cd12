"""CPU oracle for the sparse-attention indexer scoring + top-k path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import anything here; the
product library never calls it and shares no code, table or constant with
it.  Everything is plain numpy in float64 (integers exact), slow and meant
to be read against its sources:

* the vLLM DeepSeek-V3.2 indexer backend page (``indexer.py`` overlay):
  per-token decode lengths, the prefill chunk planner and chunk windows;
* the vLLM glm5next ``sparse_indexer`` helper page: padded non-uniform decode
  grids, causal fill, the MXFP4 cache row width;
* the vLLM MiniMax-M3 AMD mono runner page: ``token_rows`` and the int64
  page slots of its caches (the cache write, ``cache_write``).

The score itself, ``logit[t] = scale_t * sum_h w_h * relu(q_h . k_t)``, the
lower-index tie rule and the exact causal fill when a row's length is at most
k are the lightning-indexer definition that the pages name (the
``fp8_fp4_paged_mqa_logits`` scorer and the top-k kernels) without printing.

Every function here is pinned by a test under ``tests/`` against something
other than itself (closed forms, library routines, brute force with exact
rationals, hand-worked examples, the pages' own worked example); see the
module docstrings for which pin covers what.
"""

from . import formats, rows, cache, cache_write, score, topk, pool, planner, pipeline  # noqa: F401
