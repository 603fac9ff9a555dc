"""CPU oracle for the tree-verification pass.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package.  The library never calls it and has no CPU fallback.

Plain, slow, obviously-correct numpy code in float64 (float32 where the
block-selection arithmetic is pinned on purpose), following the pages'
statement of each step:

* ``attention``  -- every draft-tree node attends to the committed context plus
  its own ancestors, so the whole tree is verified in one target pass
  (SpecExec page, "Approach"; EasySpec page, "+tree" baseline).
* ``accept``     -- greedy match; standard speculative (rejection) sampling
  extended sibling by sibling (SpecExec page, "Builds on": speculative
  sampling, SpecInfer); and sampling from the target at each node, which stays
  equivalent to sequential sampling and works for deterministic trees
  (SpecExec page, "Approach").
* ``commit``     -- the accepted root path becomes committed context.
* ``topk``       -- keep the top-k KV blocks per query by a cheap relevance
  score (sparse-verification page, "Methodology", attention sparsity), per
  query or shared by a KV group's rows (same section, reuse across draft
  tokens).
* ``expand``     -- one batched step of the draft-tree search: the best
  children by cumulative log-probability (SpecExec page, "Approach").
* ``build``      -- the whole draft-tree search to a budget: sequential
  best-first over cumulative log-probability (same section).

Pins (tests/test_oracle_*.py) tie each function to something other than
itself: torch's scaled_dot_product_attention, closed forms, brute force over
every small tree, chi-square tests of the emitted-token distribution, and a
full sort.  No function here is "parity unpinned".

Readings where the pages are silent are listed per function.
"""
from .tree import ancestor_matrix, children_of, root_path  # noqa: F401
from .attention import attention_dense, attention_by_path  # noqa: F401
from .accept import accept, invcdf  # noqa: F401
from .commit import commit  # noqa: F401
from .topk import (append_block_sums, block_means, block_scores, block_sums,  # noqa: F401
                   means_from_sums, pooled_query, topk_blocks, topk_blocks_shared)
from .expand import expand  # noqa: F401
from .build import build_tree, log_softmax_rows  # noqa: F401
from .codec import decode  # noqa: F401
