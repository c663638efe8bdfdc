"""Tree-masked grouped-query attention, plain definition (oracle).

Test infrastructure only. Follows the EmbodiInfer page "perf(activevln):
grammar-trie speculation and lossless throughput":

* commit "feat(activevln): grammar-trie tree speculation with exact
  acceptance" — every draft node of the tree is verified in one attention
  forward; a node sees the committed context and its own ancestors (itself
  included), never its siblings or other branches;
* commit "perf(activevln): lossless batched replay throughput options", item
  attention_kernel="gqa" — query heads that share a KV head read the same
  keys and values; here query head h reads KV head h // (Hq / Hkv);
* commit "fix(attention): never read KV slots past a row's live queries" —
  slots at or past ctx_len + n_nodes are never read (they may hold NaN).

Split-KV with a log-sum-exp combine reaches this same result up to rounding
order, so the oracle is the definition itself: for each live (b, i, h) the
scores s = scale * q . k over the visible keys, o = softmax(s) @ v and
lse = ln sum exp(s) (natural log), evaluated as max + ln sum exp(s - max).

A live row can see no key at all only through an explicit mask
(:func:`masked_attention`) with an empty committed context; the pages never
meet that case. Its sum over no keys is 0, so lse = ln 0 = -inf, and its
output takes the padding value 0 (softmax over an empty set is undefined).
"""

import numpy as np

from .decode import decode
from .tree import ROW_CTX_BOUND, ROW_NNODES, ROW_OK, ancestors, parents_valid


def tree_attention(q, k, v, dtype, ctx_len, n_nodes, parent, scale,
                   max_ctx=None, kv_capacity=None):
    """Exact float64 tree attention.

    q: [B, T, Hq, D] stored values; k, v: [B, Hkv, Lcap, D] stored values;
    ``dtype`` is their storage type ("f32" or "bf16"); ctx_len, n_nodes:
    int [B]; parent: int [B, T]; scale: the float32 softmax scale (used as its
    exact float64 value). ``max_ctx`` and ``kv_capacity`` are the launch
    bounds; a row with ctx_len > max_ctx, ctx_len < 0 or
    ctx_len + n_nodes > kv_capacity is reported as ROW_CTX_BOUND and a row
    with n_nodes outside [0, T] as ROW_NNODES.

    Returns (out float64 [B, T, Hq, D], lse float64 [B, T, Hq], status int32
    [B]). Padding rows (i >= n_nodes[b]) and rows whose status is not OK get
    out = 0 and lse = -inf.
    """
    def tree_keys(b, n):
        # Tree node j lives in slot L + j; node i sees its ancestors-or-self.
        if not parents_valid(parent[b], n):
            raise ValueError("row %d: parent links are not a topologically ordered tree" % b)
        vis = np.zeros((n, n), dtype=bool)
        for i in range(n):
            for j in ancestors(parent[b], i):
                vis[i, j] = True
        return vis

    return _attention(q, k, v, dtype, ctx_len, n_nodes, tree_keys, scale, max_ctx, kv_capacity)


def masked_attention(q, k, v, dtype, ctx_len, n_nodes, mask, scale,
                     max_ctx=None, kv_capacity=None):
    """Exact float64 attention with the draft rows' visibility given as bit
    masks: row i of sequence b sees the whole committed context and block key
    j (slot ctx_len + j, j < n_nodes) iff bit j of word j // 32 of
    mask[b, i] is set. Same arguments and results as :func:`tree_attention`
    otherwise (mask: uint32 [B, T, ceil(T / 32)])."""
    mask = np.asarray(mask, dtype=np.uint32)

    def mask_keys(b, n):
        vis = np.zeros((n, n), dtype=bool)
        for i in range(n):
            for j in range(n):
                vis[i, j] = bool((int(mask[b, i, j // 32]) >> (j % 32)) & 1)
        return vis

    return _attention(q, k, v, dtype, ctx_len, n_nodes, mask_keys, scale, max_ctx, kv_capacity)


ROW_BAD_START = 6


def tree_attention_packed(q, k, v, dtype, ctx_len, n_nodes, parent, row_start, T, scale,
                          max_ctx=None, kv_capacity=None):
    """Exact float64 tree attention over packed query rows (the packed mode of
    the EmbodiInfer page's commit "perf(activevln): pack batched prefill
    turns back to back in CUDA graphs": the rows of the batch sit back to
    back, located by per-row starts, with a query extent equal to the padded
    length T).

    q: [rows, Hq, D] stored values; node i of sequence b is row
    row_start[b] + i. parent: int [B, T] (the tree stays per sequence).
    Statuses, in this order: n outside [0, T] -> ROW_NNODES; n == 0 ->
    padded (OK, no rows); row_start < 0 or row_start + n > rows ->
    ROW_BAD_START; the context bounds of :func:`tree_attention` ->
    ROW_CTX_BOUND (its n rows get out = 0, lse = -inf). Live rows get the
    definition's values. Rows that belong to no written sequence are NaN
    here (the caller's memory, left as it is).

    Returns (out float64 [rows, Hq, D], lse float64 [rows, Hq], status).
    """
    rows, Hq, D = q.shape
    B = len(n_nodes)
    out = np.full((rows, Hq, D), np.nan)
    lse = np.full((rows, Hq), np.nan)
    status = np.zeros(B, dtype=np.int32)
    cap = k.shape[2] if kv_capacity is None else kv_capacity
    mc = cap if max_ctx is None else max_ctx
    for b in range(B):
        n = int(n_nodes[b])
        s0 = int(row_start[b])
        if n < 0 or n > T:
            status[b] = ROW_NNODES
            continue
        if n == 0:
            continue
        if s0 < 0 or s0 + n > rows:
            status[b] = ROW_BAD_START
            continue
        L = int(ctx_len[b])
        if L < 0 or L > mc or L + n > cap:
            status[b] = ROW_CTX_BOUND
            out[s0:s0 + n] = 0.0
            lse[s0:s0 + n] = -np.inf
            continue
        # This sequence alone, in the one-sequence padded layout.
        qb = np.zeros((1, T) + q.shape[1:], dtype=q.dtype)
        qb[0, :n] = q[s0:s0 + n]
        o1, l1, st1 = tree_attention(qb, k[b:b + 1], v[b:b + 1], dtype, ctx_len[b:b + 1],
                                     n_nodes[b:b + 1], parent[b:b + 1], scale, max_ctx=mc,
                                     kv_capacity=cap)
        out[s0:s0 + n] = o1[0, :n]
        lse[s0:s0 + n] = l1[0, :n]
        status[b] = st1[0]
    return out, lse, status


def _attention(q, k, v, dtype, ctx_len, n_nodes, draft_keys, scale, max_ctx, kv_capacity):
    """The definition, with the draft-key visibility of sequence b given by
    draft_keys(b, n) -> bool [n, n]."""
    B, T, Hq, D = q.shape
    Hkv = k.shape[1]
    Lcap = k.shape[2]
    if kv_capacity is None:
        kv_capacity = Lcap
    if max_ctx is None:
        max_ctx = kv_capacity
    G = Hq // Hkv
    sc = np.float64(np.float32(scale))
    out = np.zeros((B, T, Hq, D), dtype=np.float64)
    lse = np.full((B, T, Hq), -np.inf, dtype=np.float64)
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = int(n_nodes[b])
        L = int(ctx_len[b])
        if n < 0 or n > T:
            status[b] = ROW_NNODES
            continue
        if n == 0:
            continue
        if L < 0 or L > max_ctx or L + n > kv_capacity:
            status[b] = ROW_CTX_BOUND
            continue
        # Visible keys of row i: the whole committed context, then the draft
        # keys draft_keys allows (draft row j lives in slot L + j).
        visible = np.zeros((n, L + n), dtype=bool)
        visible[:, :L] = True
        visible[:, L:] = draft_keys(b, n)
        for kv in range(Hkv):
            K = decode(k[b, kv, : L + n], dtype)
            Vv = decode(v[b, kv, : L + n], dtype)
            for g in range(G):
                h = kv * G + g
                qh = decode(q[b, :n, h, :], dtype)
                s = sc * (qh @ K.T)
                s = np.where(visible, s, -np.inf)
                seen = visible.any(axis=1)
                m = np.where(seen, s.max(axis=1), 0.0)[:, None]
                w = np.exp(s - m)  # exactly 0 on invisible keys
                z = w.sum(axis=1)
                zs = np.where(seen, z, 1.0)
                out[b, :n, h, :] = np.where(seen[:, None], (w @ Vv) / zs[:, None], 0.0)
                lse[b, :n, h] = np.where(seen, m[:, 0] + np.log(zs), -np.inf)
        status[b] = ROW_OK
    return out, lse, status
