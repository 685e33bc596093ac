"""CPU oracle for causal sparse attention: TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The library (``long_context_sparse_13_amd``)
never imports it, and this package imports nothing from the library: the two share
no code.  Inputs come from ``sa_synth`` (random draws only).

Everything is computed in float64 with plain numpy, in the order the pages describe
the method; see ``oracle.reference`` for the functions and their citations.
"""

from .reference import (  # noqa: F401
    indexer_scores_row,
    indexer_scores,
    topk_select_row,
    topk_select,
    topk_boundary,
    selected_mask_row,
    sparse_attn,
    graph_offsets,
    graph_neighbours,
    graph_neighbour_count,
    graph_attn,
    block_meanpool,
    decode_select,
    decode_token_mask,
    sparse_decode,
    indexcache_prefill,
)
