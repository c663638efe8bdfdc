"""Draft-tree structure: ancestor sets, visibility masks, depths (oracle).

Test infrastructure only. The tree is the draft trie of the EmbodiInfer page
"perf(activevln): grammar-trie speculation and lossless throughput", commit
"feat(activevln): grammar-trie tree speculation with exact acceptance": row 0
is the root (the last accepted token) and rows 1..n-1 are draft nodes, each
with a parent of smaller index. A node's visible tree keys are its ancestors
and itself.
"""

import numpy as np

# Per-row status values (the verification library reports the same codes).
ROW_OK = 0
ROW_BAD_PARENT = 1
ROW_CTX_BOUND = 2
ROW_NNODES = 3
ROW_BAD_TOKEN = 4


def parents_valid(parent_row: np.ndarray, n: int) -> bool:
    """Every live draft node i in 1..n-1 has 0 <= parent[i] < i."""
    for i in range(1, n):
        p = int(parent_row[i])
        if p < 0 or p >= i:
            return False
    return True


def ancestors(parent_row: np.ndarray, i: int) -> list:
    """anc*(i) = [i, parent(i), parent(parent(i)), ..., 0], by following links."""
    out = [int(i)]
    while out[-1] != 0:
        out.append(int(parent_row[out[-1]]))
    return out


def build_tree_mask(parent: np.ndarray, n_nodes: np.ndarray, T: int):
    """Ancestor-or-self bitmasks, depths and per-row status.

    Returns ``mask`` uint32 [B, T, W] with W = ceil(T / 32) (bit j of word
    j // 32 of ``mask[b, i]`` set iff node j is node i itself or one of its
    ancestors), ``depth`` int32 [B, T] (root 0; -1 on padding rows and on
    rows of a sequence whose status is not OK) and ``row_status`` int32 [B].
    """
    parent = np.asarray(parent)
    B = parent.shape[0]
    W = (T + 31) // 32
    mask = np.zeros((B, T, W), dtype=np.uint32)
    depth = np.full((B, T), -1, dtype=np.int32)
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = int(n_nodes[b])
        if n < 0 or n > T:
            status[b] = ROW_NNODES
            continue
        if not parents_valid(parent[b], n):
            status[b] = ROW_BAD_PARENT
            continue
        for i in range(n):
            anc = ancestors(parent[b], i)
            for j in anc:
                mask[b, i, j // 32] |= np.uint32(1) << np.uint32(j % 32)
            depth[b, i] = len(anc) - 1
    return mask, depth, status
