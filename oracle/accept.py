"""Exact acceptance of a verified draft tree: greedy and sampling (oracle).

Test infrastructure only. Follows the EmbodiInfer page "perf(activevln):
grammar-trie speculation and lossless throughput", commit "feat(activevln):
grammar-trie tree speculation with exact acceptance": greedy decoding keeps
the argmax path; sampling runs standard (SpecInfer-style) rejection sampling
against the draft so that the output distribution is the target's. The
acceptance mask output mirrors the vectorised accepted-token mask of the
IluvatarLabs/vllm page "Introduce SCV vectorized masking with graph/adaptive
modes".

Outputs per sequence b (padded sequences, n_nodes[b] == 0, and sequences whose
status is not OK keep the padding values):
  accept_len[b]   number of accepted draft nodes (0 on padding)
  path[b, :]      accepted nodes from the root: path[b, 0] = 0, then the
                  accepted nodes in depth order, -1 after (all -1 on padding)
  bonus[b]        the token emitted after the accepted path (-1 on padding)
  accept_mask[b]  1 on the nodes of path[b], 0 elsewhere
  decision[b, :]  sampling only: +1 accepted, 0 rejected, -1 never tested
"""

import numpy as np

from .tree import ROW_BAD_PARENT, ROW_BAD_TOKEN, ROW_NNODES, ROW_OK, parents_valid


def _check_row(parent_row, tok_row, n, T, V):
    if n < 0 or n > T:
        return ROW_NNODES
    if not parents_valid(parent_row, n):
        return ROW_BAD_PARENT
    for i in range(1, n):
        if not (0 <= int(tok_row[i]) < V):
            return ROW_BAD_TOKEN
    return ROW_OK


def _outputs(B, T):
    return (np.zeros(B, np.int32), np.full((B, T), -1, np.int32),
            np.full(B, -1, np.int32), np.zeros((B, T), np.uint8),
            np.zeros(B, np.int32))


def argmax_lowest(row: np.ndarray) -> int:
    """Index of the largest value; the lowest such index on ties.

    Values are compared as numbers, so -0.0 and +0.0 are equal. The row must
    be finite.
    """
    r = np.asarray(row, dtype=np.float64)
    if not np.all(np.isfinite(r)):
        raise ValueError("logits row is not finite")
    best = r.max()
    return int(np.flatnonzero(r == best)[0])


def _children(parent_row, cur, n):
    """Children of ``cur`` among the live nodes, ascending."""
    return [c for c in range(1, n) if int(parent_row[c]) == cur]


def accept_greedy(logits, tokens, parent, n_nodes):
    """Greedy acceptance: follow the argmax path through the draft tree.

    From the root, let a = argmax of the target logits at the current node.
    The walk moves to the lowest-index child whose token equals a; when no
    child matches, a is the bonus token and the walk ends.

    Returns (accept_len, path, bonus, accept_mask, status).
    """
    B, T, V = logits.shape
    accept_len, path, bonus, amask, status = _outputs(B, T)
    for b in range(B):
        n = int(n_nodes[b])
        st = _check_row(parent[b], tokens[b], n, T, V)
        status[b] = st
        if st != ROW_OK or n == 0:
            continue
        cur = 0
        walk = [0]
        while True:
            a = argmax_lowest(logits[b, cur])
            nxt = None
            for c in _children(parent[b], cur, n):
                if int(tokens[b, c]) == a:
                    nxt = c
                    break
            if nxt is None:
                bonus[b] = a
                break
            walk.append(nxt)
            cur = nxt
        accept_len[b] = len(walk) - 1
        path[b, : len(walk)] = walk
        amask[b, walk] = 1
    return accept_len, path, bonus, amask, status


def sample_probs(logit_row, temperature):
    """Target distribution p(x) = exp((l(x) - max l) / tau) / sum, in float64.

    ``tau`` is the float64 value of the float32 temperature.
    """
    tau = np.float64(np.float32(temperature))
    l = np.asarray(logit_row, dtype=np.float32).astype(np.float64)
    e = np.exp((l - l.max()) / tau)
    return e / e.sum()


def _inverse_cdf(r, u0):
    """Smallest x with sum_{y <= x} r(y) > u0 * sum_y r(y).

    The running sum is taken left to right and its last value is the total,
    so an answer exists for every u0 in [0, 1) when the total is positive.
    """
    c = np.cumsum(r)
    idx = np.flatnonzero(c > np.float64(u0) * c[-1])
    return int(idx[0])


def accept_sample(logits, temperature, qdraft, u, tokens, parent, n_nodes):
    """SpecInfer-style multi-step rejection sampling on a token tree.

    With p_j the target distribution at node j and q_c the draft distribution
    child c's token was drawn from (``qdraft[b, c]``):

    1. cur = root, r = p_root.
    2. For each child c of cur in ascending index, with x = tokens[b, c]:
       ratio = r(x) / q_c(x) (ratio = 0 when r(x) = 0; +inf when q_c(x) = 0
       and r(x) > 0). Accept c iff u[b, c] < ratio: c joins the path,
       cur = c, r = p_c, and step 2 restarts at the new cur. Otherwise c is
       rejected and r becomes max(r - q_c, 0) / sum(max(r - q_c, 0)) (kept
       unchanged if that sum is 0, which exact arithmetic never reaches).
    3. When no child of cur is accepted (or cur has none), the bonus token is
       the inverse-CDF draw from r with the single final uniform u[b, 0].

    Returns (accept_len, path, bonus, accept_mask, decision, status).
    """
    B, T, V = logits.shape
    accept_len, path, bonus, amask, status = _outputs(B, T)
    decision = np.full((B, T), -1, np.int8)
    for b in range(B):
        n = int(n_nodes[b])
        st = _check_row(parent[b], tokens[b], n, T, V)
        status[b] = st
        if st != ROW_OK or n == 0:
            continue
        cur = 0
        r = sample_probs(logits[b, 0], temperature)
        walk = [0]
        while True:
            accepted = None
            for c in _children(parent[b], cur, n):
                x = int(tokens[b, c])
                qc = np.asarray(qdraft[b, c], dtype=np.float32).astype(np.float64)
                rx = r[x]
                qx = qc[x]
                if rx == 0.0:
                    ratio = 0.0
                elif qx == 0.0:
                    ratio = np.inf
                else:
                    ratio = rx / qx
                if np.float64(u[b, c]) < ratio:
                    decision[b, c] = 1
                    accepted = c
                    break
                decision[b, c] = 0
                res = np.maximum(r - qc, 0.0)
                s = res.sum()
                if s > 0.0:
                    r = res / s
            if accepted is None:
                bonus[b] = _inverse_cdf(r, u[b, 0])
                break
            walk.append(accepted)
            cur = accepted
            r = sample_probs(logits[b, cur], temperature)
        accept_len[b] = len(walk) - 1
        path[b, : len(walk)] = walk
        amask[b, walk] = 1
    return accept_len, path, bonus, amask, decision, status
