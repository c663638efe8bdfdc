"""Pins for the oracle's packed-row tree attention (CPU only).

The pin is a brute force written with Python loops and math.exp directly on
the packed layout (no numpy attention, no call into the padded oracle),
plus the status cases and the untouched gap rows.
"""

import math

import numpy as np

import oracle


def _brute(q, k, v, ctx_len, n_nodes, parent, row_start, scale):
    rows, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.full((rows, Hq, D), np.nan)
    lse = np.full((rows, Hq), np.nan)
    for b in range(len(n_nodes)):
        n, L, s0 = int(n_nodes[b]), int(ctx_len[b]), int(row_start[b])
        for i in range(n):
            anc = set()
            j = i
            while True:
                anc.add(j)
                if j == 0:
                    break
                j = int(parent[b][j])
            keys = list(range(L)) + [L + j for j in sorted(anc)]
            for h in range(Hq):
                g = h // G
                sc = [float(scale) * sum(float(q[s0 + i, h, d]) * float(k[b, g, s, d])
                                         for d in range(D)) for s in keys]
                m = max(sc)
                w = [math.exp(x - m) for x in sc]
                z = sum(w)
                for d in range(D):
                    out[s0 + i, h, d] = sum(wk * float(v[b, g, s, d])
                                            for wk, s in zip(w, keys)) / z
                lse[s0 + i, h] = m + math.log(z)
    return out, lse


def _case(seed):
    rng = np.random.default_rng(seed)
    B, T, Hq, Hkv, D, cap = 3, 6, 4, 2, 8, 24
    n_nodes = np.array([4, 6, 2], np.int32)
    ctx_len = np.array([5, 0, 11], np.int32)
    row_start = np.array([7, 0, 13], np.int32)  # out of order, gap at rows 6 and 11-12
    rows = 16
    parent = np.full((B, T), -1, np.int32)
    for b in range(B):
        for i in range(1, T):
            parent[b, i] = rng.integers(0, i)
    q = rng.standard_normal((rows, Hq, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, cap, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, cap, D)).astype(np.float32)
    return q, k, v, ctx_len, n_nodes, parent, row_start, T, np.float32(0.35)


def test_packed_matches_brute_force_and_leaves_gaps():
    q, k, v, ctx, n, parent, start, T, scale = _case(3)
    out, lse, st = oracle.tree_attention_packed(q, k, v, "f32", ctx, n, parent, start, T, scale)
    bo, bl = _brute(q, k, v, ctx, n, parent, start, scale)
    assert st.tolist() == [0, 0, 0]
    live = ~np.isnan(bl)
    assert live.sum() == (4 + 6 + 2) * 4
    np.testing.assert_array_equal(np.isnan(lse), ~live)  # gap rows untouched
    np.testing.assert_allclose(out[live], bo[live], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[live], bl[live], rtol=0, atol=1e-12)


def test_packed_statuses():
    q, k, v, ctx, n, parent, start, T, scale = _case(4)
    rows = q.shape[0]
    # b0: start + n past the rows -> bad start, nothing written;
    # b1: n = 7 > T -> bad n_nodes; b2: ctx over max_ctx -> zero rows.
    start2 = np.array([rows - 3, 0, 13], np.int32)
    n2 = np.array([4, 7, 2], np.int32)
    out, lse, st = oracle.tree_attention_packed(q, k, v, "f32", ctx, n2, parent, start2, T,
                                                scale, max_ctx=10)
    assert st.tolist() == [oracle.ROW_BAD_START, oracle.ROW_NNODES, oracle.ROW_CTX_BOUND]
    assert np.all(out[13:15] == 0.0) and np.all(lse[13:15] == -np.inf)
    assert np.all(np.isnan(lse[:13])) and np.all(np.isnan(lse[15:]))
    # A padded sequence (n = 0) writes nothing whatever its start.
    n3 = np.array([0, 6, 2], np.int32)
    start3 = np.array([-5, 0, 13], np.int32)
    out, lse, st = oracle.tree_attention_packed(q, k, v, "f32", ctx, n3, parent, start3, T, scale)
    assert st.tolist() == [0, 0, 0]
    assert np.all(np.isnan(lse[6:13]))
