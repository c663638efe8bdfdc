"""Committing the accepted path's keys and values to the cache (oracle).

Test infrastructure only. During verification the keys and values of the tree
rows sit in the cache slots after the committed context (slot ctx_len + i holds
tree row i). Once acceptance has chosen a path root = path[0], path[1], ...,
path[a], those rows become ordinary context in path order and the rest of the
tree is dropped, so that the next step attends to a contiguous committed
prefix. Sources: the EmbodiInfer page "perf(activevln): grammar-trie
speculation and lossless throughput", commit "perf(activevln): lossless
batched replay throughput options" (item incremental_kv_commit: only the new
turn is copied into the owned KV, not the history), and the IluvatarLabs/vllm
page "Introduce SCV vectorized masking with graph/adaptive modes" (a commit
kernel for accepted drafts over NHD and HND cache layouts).

Reading taken here (the pages give no formula): after the commit, slot
ctx_len + k holds what slot ctx_len + path[k] held before, for k = 0..a; the
committed length becomes ctx_len + a + 1; every other slot is unchanged.
"""

import numpy as np

from .tree import ROW_CTX_BOUND, ROW_NNODES, ROW_OK

ROW_BAD_PATH = 5


def path_valid(path_row: np.ndarray, a: int, n: int) -> bool:
    """path[0] = 0 and 0 < path[1] < path[2] < ... < path[a] < n."""
    if a < 0 or a > n - 1 or int(path_row[0]) != 0:
        return False
    for k in range(1, a + 1):
        if not (int(path_row[k - 1]) < int(path_row[k]) < n):
            return False
    return True


def commit_accepted_kv(k, v, ctx_len, n_nodes, accept_len, path):
    """Return (k_new, v_new, new_ctx_len, status) for caches k, v of shape
    [..., B, Hkv, capacity, D] (any leading layer axes; element values are
    copied unchanged, whatever their type). A padded sequence (n_nodes = 0)
    is left as it is with new_ctx_len = ctx_len; so is a sequence whose n_nodes,
    context bound or path is invalid, which also gets a status code."""
    k = np.asarray(k)
    v = np.asarray(v)
    k_new = k.copy()
    v_new = v.copy()
    B = k.shape[-4]
    cap = k.shape[-2]
    T = path.shape[1]
    new_ctx = np.asarray(ctx_len, dtype=np.int64).copy()
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = int(n_nodes[b])
        L = int(ctx_len[b])
        a = int(accept_len[b])
        if n < 0 or n > T:
            status[b] = ROW_NNODES
            continue
        if n == 0:
            continue
        if L < 0 or L + n > cap:
            status[b] = ROW_CTX_BOUND
            continue
        if not path_valid(path[b], a, n):
            status[b] = ROW_BAD_PATH
            continue
        # Gather from the cache as it was before the commit.
        for kk in range(a + 1):
            src = L + int(path[b][kk])
            k_new[..., b, :, L + kk, :] = k[..., b, :, src, :]
            v_new[..., b, :, L + kk, :] = v[..., b, :, src, :]
        new_ctx[b] = L + a + 1
    return k_new, v_new, new_ctx.astype(np.int32), status
