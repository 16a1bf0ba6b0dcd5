"""fp64 CPU oracle for MLA tree-verify attention — TEST INFRASTRUCTURE ONLY.

Only the test-suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package. The product path (the HIP library and its Python
binding) never imports, links or calls it, and shares no code with it.

Contents:
  definition  – the plain masked-softmax definition in fp64 (the oracle proper),
                plus the tile-streaming and chunk-combine forms of the same result.
  bruteforce  – pure-Python per-head loops with math.fsum, for tiny inputs.
  compaction  – post-verify KV compaction (accepted draft rows moved to the
                front of the draft region), the plain definition.
  projection  – per-head projections into and out of the latent space.
  topk        – top-k index selection (the sparse path's index lists).

Every function is pinned by tests under -m "not gpu" against brute force,
a textbook attention routine (torch SDPA in float64), closed forms and
invariants; none is "parity unpinned".
"""
from .definition import (  # noqa: F401
    attend,
    attend_chunked,
    attend_streaming,
    dense_visible_positions,
    verify_dense,
    verify_sparse,
)
from .compaction import compact_kv  # noqa: F401
from .projection import head_project  # noqa: F401
from .topk import order_key, select_topk  # noqa: F401
