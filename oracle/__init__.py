"""fp64 CPU oracle for the Gated DeltaNet-2 core (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package; the product path never does.  It shares no code
with the HIP library.  Every function cites the page passage it follows; see
gdn2_oracle.py for the citation keys.
"""

from .gdn2_oracle import (CHUNK, step, recurrence, chunk_factors, chunk_apply,
                          chunk_affine_map, chunked, gates_from_logits, recurrence_bwd, chunk_bwd,
                          chunked_bwd, rel_max_err)
from . import layer_oracle, swa_oracle

__all__ = ["CHUNK", "step", "recurrence", "chunk_factors", "chunk_apply",
           "chunk_affine_map", "chunked", "gates_from_logits", "recurrence_bwd", "chunk_bwd",
           "chunked_bwd",
           "rel_max_err", "layer_oracle", "swa_oracle"]
