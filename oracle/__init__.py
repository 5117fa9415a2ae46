"""Float64 CPU oracle for the Sparse-to-Dense (StD) decoding hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) imports, calls or links anything in this package; only
the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP path.

Source: "Sparse-to-Dense: A Free Lunch for Lossless Acceleration of Video
Understanding in LLMs" (abstract page; technical summary pages in German,
Arabic and French; French lay explanation).  Each function names the passage
it follows.  Every function is written from the definitions in plain numpy
float64, slow and direct, so it can be checked against the pages by eye:

* ``select_topk``   -- prefill-time top-K visual KV selection from the mean
                       text->visual attention score (technical summary,
                       Methodology item 4 "KV cache selection").
* ``static_window_idx`` -- the visual positions a streaming-attention draft
                       keeps (an attention sink plus a recent window), the
                       comparator the pages' Experimental results name.
* ``sparse_decode`` -- the sparse model's single-query attention over the
                       selected visual KV plus all non-visual KV (technical
                       summary, Methodology item 2, sparse model M_s).
* ``dense_verify``  -- the dense model's causal attention for the gamma+1
                       verification queries (Methodology item 2, dense model
                       M; item 3, verification); the same function gives
                       the prefill attention of the text rows.
* ``row_lse``       -- the log softmax normaliser of each of those rows (what
                       a prefill attention returns beside its output for the
                       selection's first step, Methodology item 4).
* ``accept``        -- greedy longest-prefix acceptance plus the bonus token
                       (Methodology item 3, decoding procedure).
* ``toy``           -- a tiny float64 decoder that runs plain greedy decoding
                       and the full StD loop, used to pin losslessness
                       (Key contributions, "lossless acceleration").

Pins (tests/test_oracle_*.py) tie every function to something other than
itself: brute-force sorts, closed forms, hand-worked golden cases, softmax
invariants, the sparse==dense special case, an independent library routine
(torch scaled_dot_product_attention in float64), exhaustive enumeration of
the acceptance rule and the losslessness invariant of the toy loop.
"""

from .attention import dense_verify, sparse_decode, sparse_key_set, attend, row_lse
from .selection import select_topk, selection_scores, rank_topk, static_window_idx
from .acceptance import accept, argmax_margin

__all__ = [
    "dense_verify", "sparse_decode", "sparse_key_set", "attend", "row_lse",
    "select_topk", "selection_scores", "rank_topk", "static_window_idx",
    "accept", "argmax_margin",
]
