"""Plain float64 CPU oracle for layer-packed selective recompute with the
mixed-cache logit bias.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (the HIP library and its Python binding) never
imports it, and this package imports nothing from the product path.  The two
share only the seeded input generators in ``workloads``.

Sources (cited by title and section; no line numbers):
* "Budgeted KV-Cache Repair for Evolving Contexts" (page 1): exact budget
  (section 7.1, Eq. 3), sort-and-coalesce into execution intervals (section
  3.2, Algorithm 1), sequential maximal-interval replay (section 7.1),
  mixed-cache recurrence (section 13.2, Eq. 21-22), reusable tile plan
  (section 13.2, Eq. 23-24).
* The cross-attention reuse specification page (page 4): blocks (section
  6.1), mixed cache, load-time metadata and global positions (section 6.2), the seam set T_tau with the
  asymmetric true-prefix rule (section 6.3), the biased operator F, its
  inference mode without write-back and its degeneration (section 6.4).
* "Budgeted KV-Cache Repair" section 7.1, Eq. 2: the Shift operation
  (positional correction of the retained suffix after a deletion).
* "Budgeted KV-Cache Repair" sections 3.2 and 7.3 (Eq. 1 / 7, Eq. 8,
  Algorithm 1): the numeric core of Semantic-Unit Refresh (token relevance,
  unit scores and ranking, exact-budget fill, forward-envelope window).

Arithmetic is float64 throughout (inputs are widened from their float32 /
bf16 storage), except Semantic-Unit Refresh scoring, which the page fixes
to float32.  Matrix products use numpy's matmul as a library step; there
is no blocking, fusion or reordering beyond the definitions.

Where the pages are silent, the reading taken is stated in the docstring of
the function that takes it; every function here is pinned by tests under
``tests/`` (no function is parity-unpinned).
"""
from .repair_set import (BadBlocks, BadSupport, attn_tile_plan, budget, check_positions,
                         check_support, initial_meta, kv_tile_first_query, runs, seam_set,
                         validate_blocks)
from .layer import (FLAG_LOCAL, FLAG_SINK, attention_bias, biased_attention_row,
                    interval_major, layer_repair, rms_norm, rope, silu, stack_repair,
                    write_back_flags)
from .cache_ops import inference_attention, shift_cache
from . import sur

__all__ = [
    "BadBlocks", "BadSupport", "attn_tile_plan", "budget", "check_positions",
    "check_support", "initial_meta", "kv_tile_first_query", "runs", "seam_set",
    "validate_blocks", "FLAG_LOCAL",
    "FLAG_SINK", "attention_bias", "biased_attention_row", "interval_major", "layer_repair",
    "rms_norm", "rope", "silu", "stack_repair", "write_back_flags", "inference_attention",
    "shift_cache", "sur",
]
