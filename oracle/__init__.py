"""CPU oracle for one round of tree-structured speculative verification.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the test suite, the smoke check of the build entry
point and the CPU-baseline leg of the benchmark use it.  It shares no code,
tables or constants with the HIP library; the two meet only through the seeded
inputs of the `workloads` package.

It is written to be read against the pages, not to be fast:

  topk       per-position top-k of the drafter marginals (stable sort)
  tree       greedy best-first draft tree by prefix probability, selected
             exhaustively (full enumeration when small, exact level-by-level
             pruning otherwise), plus ancestor sets
  expand     the same selection over a tree expanded node by node, each
             node branching on its own conditional distribution
  budget     round cost C = C_d + C_v(n; l) and the throughput stop rule
  costfit    the convex, monotone C_v fitted to measured latencies (NNLS)
  global_budget  batch-global admission of tree nodes against an engine
             throughput table, with early stopping
  chains     unfolding of a tree into its root-to-leaf chains
  attention  naive per-node attention in fp64 with explicit ancestor walks
  walk       greedy accept walk over the target's argmax
  commit     copy of the accepted chain into the persistent cache
  round      the four steps chained for a set of requests

Sources (cited by page title and section in each module):
  [review]   "Adapting Tree-Structured Speculative Decoding to DeepSeek-V4 for
             Efficient Inference" (blog review of arXiv 2609.24698)
  [dspark]   "DSpark: Speculative decoding ... LLM inference acceleration" summary
  [caddtree] "Cost-Aware Diffusion Draft Trees for Speculative Decoding"
             (summary of arXiv 2606.01813)

Parity status: every function here is pinned by CPU tests against values the
pages print (the toy example, the DSpark decoding cycle), closed forms,
brute force on tiny inputs and independent library routines (torch SDPA).
The synthetic value distributions themselves are not from the pages and are
parity unpinned.
"""

from .topk import topk_per_position  # noqa: F401
from .budget import adaptive_budget, round_cost, throughput  # noqa: F401
from .tree import ancestor_bits, select_tree, TreeResult  # noqa: F401
from .expand import expand_candidates, expanded_rows, select_tree_expand  # noqa: F401
from .attention import attend_node, attend_request  # noqa: F401
from .costfit import fit_cost  # noqa: F401
from .global_budget import global_budget, global_order  # noqa: F401
from .chains import unfold_chains  # noqa: F401
from .walk import accept_walk, row_argmax  # noqa: F401
from .commit import commit_path  # noqa: F401
from .compress import block_state, chain_entries, compress_chains, refresh_compressed  # noqa: F401
