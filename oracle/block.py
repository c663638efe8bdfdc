"""Draft-block visibility masks (oracle).

Test infrastructure only. Besides trees, a verification forward may carry a
block of draft rows: a linear draft (each row sees the block rows before it
and itself: the causal chain) or a block whose rows all see one another, the
block attention of the DFlash draft on the FlashRT page "Alpamayo 1.5 on
Thor: full-request engine with precision presets and FlashDrive streaming
backend" (attention of the block rows over the context plus the block keys).
The rows see the whole committed context in both modes; the masks use the
bit layout of the tree masks (bit j of word j // 32 of mask[b, i]: block key
j, in slot ctx_len + j).
"""

import numpy as np

from .tree import ROW_NNODES

CAUSAL = 0
BIDIRECTIONAL = 1


def build_block_mask(n_nodes, T: int, mode: int):
    """(mask uint32 [B, T, W], position int32 [B, T], status int32 [B]).
    Causal: row i sees block rows 0..i. Bidirectional: every live row sees
    every live row. position[b, i] = i on live rows (the row's offset after
    the committed context), -1 on padding rows and on sequences whose n_nodes
    is outside [0, T]."""
    if mode not in (CAUSAL, BIDIRECTIONAL):
        raise ValueError("unknown block mode %r" % (mode,))
    n_nodes = np.asarray(n_nodes)
    B = n_nodes.shape[0]
    W = (T + 31) // 32
    mask = np.zeros((B, T, W), dtype=np.uint32)
    pos = np.full((B, T), -1, dtype=np.int32)
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = int(n_nodes[b])
        if n < 0 or n > T:
            status[b] = ROW_NNODES
            continue
        for i in range(n):
            last = i if mode == CAUSAL else n - 1
            for j in range(last + 1):
                mask[b, i, j // 32] |= np.uint32(1) << np.uint32(j % 32)
            pos[b, i] = i
    return mask, pos, status
