"""Pins of the accepted-path KV commit oracle (oracle/commit.py), no GPU.

* hand-worked fixtures (tests/golden/kv_commit_hand.json), including a path
  whose later source slot is an earlier destination;
* a chain tree accepted in full leaves the cache as it was;
* the attention outputs of the accepted nodes are preserved: tree attention
  of node path[k] in the verification forward (oracle) equals plain attention
  of the same query over the committed slots [0, ctx_len + k] after the
  commit, computed by torch's CPU scaled_dot_product_attention in float64;
* leading layer axes are committed layer by layer;
* status codes for bad n_nodes, context bounds and paths.
"""

import json
import os

import numpy as np
import torch

import oracle
from oracle.decode import decode
from workloads import make_custom

HERE = os.path.dirname(os.path.abspath(__file__))


def _hand_cache(case):
    B = len(case["ctx_len"])
    cap = case["capacity"]
    k = np.zeros((B, 1, cap, 1), np.float32)
    v = np.zeros((B, 1, cap, 1), np.float32)
    for b in range(B):
        for s in range(cap):
            k[b, 0, s, 0] = 10 * b + s
            v[b, 0, s, 0] = -(100 + 10 * b + s)
    return k, v


def test_hand_fixtures():
    data = json.load(open(os.path.join(HERE, "golden", "kv_commit_hand.json")))
    assert len(data["cases"]) == 4
    for case in data["cases"]:
        k, v = _hand_cache(case)
        kn, vn, ctx, st = oracle.commit_accepted_kv(
            k, v, np.array(case["ctx_len"]), np.array(case["n_nodes"]),
            np.array(case["accept_len"]), np.array(case["path"]))
        assert np.array_equal(kn[:, 0, :, 0], np.array(case["k_after"], np.float32)), case["name"]
        assert np.array_equal(vn[:, 0, :, 0], np.array(case["v_after"], np.float32)), case["name"]
        assert np.array_equal(ctx, case["new_ctx_len"]), case["name"]
        assert np.array_equal(st, case["status"]), case["name"]


def _path_to(parent_row, node):
    return oracle.ancestors(parent_row, node)[::-1]


def test_chain_accepted_in_full_is_identity():
    w = make_custom(3, 2, 4, 2, 64, 50, "bf16", [40, 7], 9, tree="chain", trie_tokens=False)
    T = w.T
    path = np.tile(np.arange(T, dtype=np.int32), (w.B, 1))
    acc = w.n_nodes.astype(np.int32) - 1
    kn, vn, ctx, st = oracle.commit_accepted_kv(w.k, w.v, w.ctx_len, w.n_nodes, acc, path)
    assert np.array_equal(kn.view(np.uint16), np.asarray(w.k).view(np.uint16))
    assert np.array_equal(vn.view(np.uint16), np.asarray(w.v).view(np.uint16))
    assert np.array_equal(ctx, w.ctx_len + w.n_nodes)
    assert not st.any()


def test_accepted_nodes_keep_their_attention():
    w = make_custom(21, 3, 6, 2, 64, 50, "bf16", [37, 0, 64], 12, trie_tokens=False)
    rng = np.random.default_rng(4)
    out_tree, _, _ = oracle.tree_attention(w.q, w.k, w.v, w.dtype, w.ctx_len, w.n_nodes,
                                           w.parent, w.scale)
    T = w.T
    path = np.full((w.B, T), -1, np.int32)
    acc = np.zeros(w.B, np.int32)
    for b in range(w.B):
        n = int(w.n_nodes[b])
        node = int(rng.integers(0, n))
        p = _path_to(w.parent[b], node)
        path[b, :len(p)] = p
        acc[b] = len(p) - 1
    kn, vn, ctx, st = oracle.commit_accepted_kv(w.k, w.v, w.ctx_len, w.n_nodes, acc, path)
    assert not st.any()
    qf, kf, vf = decode(w.q, w.dtype), decode(kn, w.dtype), decode(vn, w.dtype)
    for b in range(w.B):
        L = int(w.ctx_len[b])
        for kk in range(acc[b] + 1):
            node = int(path[b, kk])
            for h in range(w.Hq):
                g = h // w.G
                q = torch.from_numpy(qf[b, node, h][None, None, None, :])
                key = torch.from_numpy(kf[b, g, :L + kk + 1][None, None])
                val = torch.from_numpy(vf[b, g, :L + kk + 1][None, None])
                o = torch.nn.functional.scaled_dot_product_attention(q, key, val,
                                                                     scale=float(w.scale))
                assert np.abs(o.numpy()[0, 0, 0] - out_tree[b, node, h]).max() < 1e-12


def test_layers_committed_one_by_one():
    w = make_custom(8, 2, 4, 2, 64, 50, "bf16", [20, 33], 7, trie_tokens=False)
    k2 = np.stack([w.k, w.k[:, ::-1].copy()])
    v2 = np.stack([w.v, w.v[:, ::-1].copy()])
    path = np.full((w.B, w.T), -1, np.int32)
    acc = np.zeros(w.B, np.int32)
    for b in range(w.B):
        p = _path_to(w.parent[b], int(w.n_nodes[b]) - 1)
        path[b, :len(p)] = p
        acc[b] = len(p) - 1
    kn, vn, ctx, st = oracle.commit_accepted_kv(k2, v2, w.ctx_len, w.n_nodes, acc, path)
    for layer in range(2):
        k1, v1, c1, s1 = oracle.commit_accepted_kv(k2[layer], v2[layer], w.ctx_len, w.n_nodes,
                                                   acc, path)
        assert np.array_equal(kn[layer].view(np.uint16), k1.view(np.uint16))
        assert np.array_equal(vn[layer].view(np.uint16), v1.view(np.uint16))
        assert np.array_equal(c1, ctx) and np.array_equal(s1, st)


def test_status_codes():
    k = np.zeros((4, 1, 10, 1), np.float32)
    ctx = np.array([2, 2, 8, 2])
    n = np.array([9, 3, 3, 3])       # n > T; fine; context bound (8 + 3 > 10); fine
    acc = np.array([0, 3, 0, 1])     # -, accept_len > n - 1, -, bad path
    path = np.array([[0, -1, -1, -1], [0, 1, 2, -1], [0, -1, -1, -1], [1, 2, -1, -1]])
    kn, vn, nc, st = oracle.commit_accepted_kv(k, k, ctx, n, acc, path)
    assert list(st) == [oracle.ROW_NNODES, oracle.ROW_BAD_PATH, oracle.ROW_CTX_BOUND,
                        oracle.ROW_BAD_PATH]
    assert np.array_equal(nc, ctx)
