"""Adaptive draft budget and the next step's packed row table (oracle).

Test infrastructure only. The IluvatarLabs/vllm page "Introduce SCV
vectorized masking with graph/adaptive modes" describes an adaptive mode that
changes the number of speculative tokens from recent acceptance ratios so as
to hold a target ratio; the page gives no formula. The reading taken here
(the plainest one): the acceptance ratio of a verified step is the accepted
draft nodes over the draft nodes verified, a / (n - 1); "recent" is an
exponential moving average with weight alpha; the budget moves by one draft
node per step toward the target (up while the average is above it, down
while below) within [n_min, n_max]. The EmbodiInfer page "perf(activevln):
grammar-trie speculation and lossless throughput", commit "perf(activevln):
pack batched prefill turns back to back in CUDA graphs", locates packed rows
by per-row starts: row_start is the exclusive prefix sum of each sequence's
next row count, budget + 1 (its draft nodes and the root).

The arithmetic is done in float32, one rounded operation at a time in the
order written (ratio, difference, product, sum), because the integer
decision (the budget step) is taken from the float32 average.
"""

import numpy as np

from .tree import ROW_OK

F32 = np.float32


def adapt_tree_budget(accept_len, n_nodes, ratio_ema, budget, target, alpha, n_min, n_max,
                      row_status=None):
    """One controller step for every sequence.

    accept_len, n_nodes: int [B] (the verified step); ratio_ema: float32 [B];
    budget: int [B]; target, alpha: floats (used as their float32 values);
    row_status: int [B] or None. Returns (ratio_ema float32 [B], budget int32
    [B], row_start int32 [B], rows_total int).
    """
    B = len(accept_len)
    ema = np.array(ratio_ema, dtype=np.float32).copy()
    bud = np.array(budget, dtype=np.int64).copy()
    tgt = F32(target)
    a32 = F32(alpha)
    for b in range(B):
        n = int(n_nodes[b])
        a = int(accept_len[b])
        ok = row_status is None or int(row_status[b]) == ROW_OK
        if ok and n >= 2 and 0 <= a <= n - 1:
            ratio = F32(a) / F32(n - 1)
            e = ema[b]
            e = F32(e + F32(a32 * F32(ratio - e)))
            ema[b] = e
            if e > tgt:
                bud[b] += 1
            elif e < tgt:
                bud[b] -= 1
        bud[b] = min(max(int(bud[b]), n_min), n_max)
    rows = bud + 1
    row_start = np.zeros(B, dtype=np.int32)
    acc = 0
    for b in range(B):
        row_start[b] = acc
        acc += int(rows[b])
    return ema, bud.astype(np.int32), row_start, acc
