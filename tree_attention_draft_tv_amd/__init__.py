"""Tree-draft verification for AMD MI355X (gfx950).

Verifies a speculative draft token tree in one forward pass: ancestor masks
(:func:`build_tree_mask`; :func:`build_block_mask` for draft blocks), tree-masked split-KV grouped-query attention
(:func:`tree_attention`; :func:`tree_attention_packed` over packed rows),
exact acceptance (:func:`accept_greedy`, :func:`accept_sample`), the commit of
the accepted path's keys and values (:func:`commit_accepted_kv`) and the
device-side adaptive draft budget (:func:`adapt_tree_budget`), plus the
batch-invariant few-row projections of the verification rows
(:func:`linear_rows`, :func:`linear_swiglu_rows`).
The compute runs in the HIP kernels of the in-tree
``libtv.so`` (C ABI in ``include/tv.h``); this package only marshals
arguments.
"""

from .binding import (  # noqa: F401
    LIB_PATH,
    TV_BF16,
    TV_BLOCK_BIDIRECTIONAL,
    TV_BLOCK_CAUSAL,
    TV_F32,
    TV_MAX_GROUP,
    TV_MAX_TREE,
    TVError,
    accept_greedy,
    accept_greedy_noalloc,
    accept_sample,
    accept_workspace_size,
    adapt_tree_budget,
    attention_workspace_size,
    auto_chunk,
    build_block_mask,
    build_tree_mask,
    commit_accepted_kv,
    linear_rows,
    linear_swiglu_rows,
    load,
    read_probe,
    tree_attention,
    tree_attention_packed,
)
