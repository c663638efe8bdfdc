"""Float64 CPU oracle for draft-tree verification — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything under ``oracle/``. The product path (the HIP
library and its Python binding in ``tree_attention_draft_tv_amd``) never
imports, links or calls it, and the oracle imports nothing from the product
path: the two share no code. Inputs come from the seeded generators in
``workloads/``.

What it computes, and where the method is defined (all on the EmbodiInfer
pull-request page "perf(activevln): grammar-trie speculation and lossless
throughput" unless noted):

* ``tree.build_tree_mask`` — the ancestor-or-self visibility of each draft
  node, found by following parent links (commit "feat(activevln): grammar-trie
  tree speculation with exact acceptance": the N most likely trie nodes are
  verified in one tree-attention forward, so each node may only see its own
  ancestors).
* ``attention.tree_attention`` — the plain softmax-attention definition over
  the committed context plus the node's ancestors, with grouped-query heads
  (commit "perf(activevln): lossless batched replay throughput options",
  item attention_kernel="gqa"), never touching cache slots past the live
  extent (commit "fix(attention): never read KV slots past a row's live
  queries").
* ``accept.accept_greedy`` — keep the argmax path (commit "feat(activevln):
  grammar-trie tree speculation with exact acceptance").
* ``accept.accept_sample`` — SpecInfer-style rejection sampling against the
  draft with a residual resample (same commit; "exact SpecInfer-style
  acceptance" in the page's summary).
* ``block.build_block_mask`` and ``attention.masked_attention`` — draft
  blocks instead of trees: a linear (causal) block, or a block whose rows all
  see one another (the DFlash block attention on the FlashRT page "Alpamayo
  1.5 on Thor: full-request engine with precision presets and FlashDrive
  streaming backend").
* ``linear.linear_rows`` and ``linear.swiglu_rows`` — the few-row
  projections of the verification rows with one output rounding, and the
  rounded SwiGLU of the gate and up projections (commit "perf(activevln):
  batch-invariant Triton GEMMs for decode projections").
* ``attention.tree_attention_packed`` — the same attention over query rows
  packed back to back, located by per-row starts (commit "perf(activevln):
  pack batched prefill turns back to back in CUDA graphs").
* ``budget.adapt_tree_budget`` — the adaptive draft budget (the IluvatarLabs/vllm
  page "Introduce SCV vectorized masking with graph/adaptive modes", its
  adaptive mode) and the packed row starts of the next step.
* ``commit.commit_accepted_kv`` — the accepted path's keys and values become
  contiguous committed context (commit "perf(activevln): lossless batched
  replay throughput options", item incremental_kv_commit; the IluvatarLabs/vllm
  page "Introduce SCV vectorized masking with graph/adaptive modes", its
  commit kernel for accepted drafts).

Every function works in float64 after decoding its inputs exactly from their
stored float32 / bfloat16 values. Every result is pinned by tests against
closed forms, textbook special cases and brute force (tests/test_oracle_*.py).
"""

from .accept import accept_greedy, accept_sample, sample_probs  # noqa: F401
from .attention import ROW_BAD_START, masked_attention, tree_attention  # noqa: F401
from .attention import tree_attention_packed  # noqa: F401
from .budget import adapt_tree_budget  # noqa: F401
from .block import BIDIRECTIONAL, CAUSAL, build_block_mask  # noqa: F401
from .commit import ROW_BAD_PATH, commit_accepted_kv  # noqa: F401
from .linear import linear_rows, round_bf16, silu, swiglu_rows  # noqa: F401
from .decode import decode  # noqa: F401
from .tree import ROW_BAD_PARENT, ROW_BAD_TOKEN, ROW_CTX_BOUND, ROW_NNODES, ROW_OK  # noqa: F401
from .tree import ancestors, build_tree_mask  # noqa: F401
