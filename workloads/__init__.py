"""Seeded synthetic inputs for draft-tree verification.

This package only *draws* inputs (trees, token ids, query/key/value tensors,
target logits, draft distributions, uniforms). It contains none of the
verification arithmetic: no tree masks, no attention, no argmax walk, no
rejection test. Both the float64 oracle (``oracle/``) and the HIP path
(``tree_attention_draft_tv_amd``) consume what it returns; neither is imported
here.
"""

from .gen import (  # noqa: F401
    CONFIG_NAMES,
    Workload,
    bf16_bits_from_f32,
    make_config,
    make_custom,
    random_tree,
)
