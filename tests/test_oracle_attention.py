"""Pins for the oracle's tree attention (CPU only).

Nothing here re-types the oracle's formula. The pins are: a hand-worked
example; the two textbook special cases (a chain tree is causal attention, a
root-only tree is plain decode attention), both computed by torch's CPU
scaled_dot_product_attention in float64; closed forms (K = 0, V = const);
and invariances (GQA head mapping, key permutation, batch independence, NaN in
dead slots).
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
from workloads import bf16_bits_from_f32, make_custom


def _ln(x):
    if isinstance(x, str):
        assert x.startswith("ln ")
        return math.log(float(x[3:]))
    return float(x)


def test_golden_tiny_tree(golden_dir):
    with open(os.path.join(golden_dir, "tiny_tree_attention.json")) as f:
        g = json.load(f)
    D = g["D"]
    L = g["ctx_len"]
    T = len(g["parent"])
    q = np.array([[_ln(x) for x in row] for row in g["queries"]], np.float32)
    k = np.array(g["keys"], np.float32)
    v = np.array(g["values"], np.float32)
    out, lse, st = oracle.tree_attention(
        q.reshape(1, T, 1, D), k.reshape(1, 1, L + T, D), v.reshape(1, 1, L + T, D),
        "f32", [L], [T], np.array([g["parent"]]), np.float32(g["scale"]))
    assert st[0] == 0
    np.testing.assert_allclose(out[0, :, 0, :], np.array(g["expected_out"]), rtol=0, atol=2e-6)
    np.testing.assert_allclose(lse[0, :, 0], [_ln(x) for x in g["expected_lse"]], rtol=0, atol=2e-6)


def _rand(rng, shape):
    return rng.standard_normal(shape).astype(np.float32)


@pytest.mark.parametrize("L,T,D", [(0, 5, 8), (37, 9, 16), (100, 33, 32), (3, 65, 8)])
def test_chain_tree_is_causal_attention(L, T, D):
    rng = np.random.default_rng(L * 1000 + T)
    q = _rand(rng, (1, T, 2, D))
    k = _rand(rng, (1, 1, L + T, D))
    v = _rand(rng, (1, 1, L + T, D))
    scale = np.float32(1.0 / math.sqrt(D))
    parent = np.arange(-1, T - 1, dtype=np.int32)[None]
    out, lse, _ = oracle.tree_attention(q, k, v, "f32", [L], [T], parent, scale)
    for h in range(2):
        # Full causal self-attention over L + T positions; the tree rows are
        # the last T queries, so their own queries go at those positions and
        # the first L positions get arbitrary queries.
        qfull = np.concatenate([_rand(rng, (L, D)), q[0, :, h]], axis=0).astype(np.float64)
        kk = torch.from_numpy(k[0, 0].astype(np.float64))[None, None]
        vv = torch.from_numpy(v[0, 0].astype(np.float64))[None, None]
        qq = torch.from_numpy(qfull)[None, None]
        ref = F.scaled_dot_product_attention(qq, kk, vv, is_causal=True,
                                             scale=float(scale))[0, 0, L:].numpy()
        np.testing.assert_allclose(out[0, :, h], ref, rtol=0, atol=1e-12)
        s = (qfull @ k[0, 0].astype(np.float64).T) * np.float64(scale)
        s = np.where(np.tril(np.ones((L + T, L + T), bool)), s, -np.inf)
        np.testing.assert_allclose(lse[0, :, h], scipy.special.logsumexp(s, axis=1)[L:],
                                   rtol=0, atol=1e-12)


@pytest.mark.parametrize("L,D", [(1, 8), (64, 64), (300, 128)])
def test_root_only_tree_is_decode_attention(L, D):
    rng = np.random.default_rng(L + D)
    q = _rand(rng, (1, 1, 4, D))
    k = _rand(rng, (1, 2, L + 1, D))
    v = _rand(rng, (1, 2, L + 1, D))
    scale = np.float32(0.3)
    out, lse, _ = oracle.tree_attention(q, k, v, "f32", [L], [1], np.array([[-1]]), scale)
    for h in range(4):
        kv = h // 2
        qq = torch.from_numpy(q[0, 0, h].astype(np.float64))[None, None, None]
        kk = torch.from_numpy(k[0, kv].astype(np.float64))[None, None]
        vv = torch.from_numpy(v[0, kv].astype(np.float64))[None, None]
        ref = F.scaled_dot_product_attention(qq, kk, vv, scale=float(scale))[0, 0, 0].numpy()
        np.testing.assert_allclose(out[0, 0, h], ref, rtol=0, atol=1e-12)
        s = (k[0, kv].astype(np.float64) @ q[0, 0, h].astype(np.float64)) * np.float64(scale)
        assert abs(lse[0, 0, h] - scipy.special.logsumexp(s)) < 1e-12


def test_zero_keys_closed_form():
    """K = 0: every visible score is 0, so lse = ln(#visible) = ln(L + depth + 1)
    and the output is the plain mean of the visible values."""
    w = make_custom(11, 3, 4, 2, 16, 50, "f32", [10, 0, 77], 12, max_depth=4,
                    trie_tokens=False, n_nodes=[13, 13, 7])
    k = np.where(np.isnan(w.k), np.nan, 0.0).astype(np.float32)
    out, lse, st = oracle.tree_attention(w.q, k, w.v, "f32", w.ctx_len, w.n_nodes,
                                         w.parent, w.scale)
    assert np.all(st == 0)
    _, depth, _ = oracle.build_tree_mask(w.parent, w.n_nodes, w.T)
    for b in range(w.B):
        L = int(w.ctx_len[b])
        for i in range(int(w.n_nodes[b])):
            np.testing.assert_allclose(lse[b, i], math.log(L + depth[b, i] + 1), rtol=0, atol=1e-12)
            # Visible tree slots of node i, written out by walking up by hand.
            slots = list(range(L))
            j = i
            while True:
                slots.append(L + j)
                if j == 0:
                    break
                j = int(w.parent[b, j])
            for h in range(w.Hq):
                mean = w.v[b, h // w.G, slots].astype(np.float64).mean(axis=0)
                np.testing.assert_allclose(out[b, i, h], mean, rtol=0, atol=1e-12)


def test_constant_values_give_constant_output():
    w = make_custom(12, 2, 6, 3, 8, 50, "bf16", [33, 5], 20, trie_tokens=False)
    vbits = bf16_bits_from_f32(np.full(w.v.shape, 1.75, np.float32))
    out, lse, _ = oracle.tree_attention(w.q, w.k, vbits, "bf16", w.ctx_len, w.n_nodes,
                                        w.parent, w.scale)
    assert np.all(np.abs(out - 1.75) < 1e-12)
    assert np.all(np.isfinite(lse))


def test_gqa_mapping_matches_repeated_kv_heads():
    """Query head h reads KV head h // G: repeating each KV head G times
    (one KV head per query head) must not change anything."""
    w = make_custom(13, 2, 12, 3, 16, 50, "f32", [40, 9], 10, trie_tokens=False)
    out, lse, _ = oracle.tree_attention(w.q, w.k, w.v, "f32", w.ctx_len, w.n_nodes,
                                        w.parent, w.scale)
    k_rep = np.repeat(w.k, w.G, axis=1)
    v_rep = np.repeat(w.v, w.G, axis=1)
    out2, lse2, _ = oracle.tree_attention(w.q, k_rep, v_rep, "f32", w.ctx_len, w.n_nodes,
                                          w.parent, w.scale)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)
    # A wrong mapping (h % Hkv) would pair heads with other KV heads:
    assert not np.allclose(out[:, :, 1], out[:, :, 4])


def test_committed_key_permutation_invariance():
    w = make_custom(14, 1, 4, 1, 16, 50, "f32", [64], 6, trie_tokens=False)
    out, lse, _ = oracle.tree_attention(w.q, w.k, w.v, "f32", w.ctx_len, w.n_nodes,
                                        w.parent, w.scale)
    perm = np.random.default_rng(0).permutation(64)
    k = w.k.copy()
    v = w.v.copy()
    k[:, :, :64] = w.k[:, :, perm]
    v[:, :, :64] = w.v[:, :, perm]
    out2, lse2, _ = oracle.tree_attention(w.q, k, v, "f32", w.ctx_len, w.n_nodes,
                                          w.parent, w.scale)
    np.testing.assert_allclose(out, out2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-13)


def test_padding_nan_poison_and_batch_independence():
    w = make_custom(15, 4, 8, 2, 32, 50, "bf16", [100, 7, 64, 250], 16,
                    trie_tokens=False, n_nodes=[17, 0, 5, 17])
    out, lse, st = oracle.tree_attention(w.q, w.k, w.v, "bf16", w.ctx_len, w.n_nodes,
                                         w.parent, w.scale)
    assert np.all(st == 0)
    for b in range(4):
        n = int(w.n_nodes[b])
        assert np.all(np.isfinite(out[b, :n])) and np.all(np.isfinite(lse[b, :n]))
        assert np.all(out[b, n:] == 0) and np.all(lse[b, n:] == -np.inf)
        one = oracle.tree_attention(w.q[b:b + 1], w.k[b:b + 1], w.v[b:b + 1], "bf16",
                                    w.ctx_len[b:b + 1], w.n_nodes[b:b + 1],
                                    w.parent[b:b + 1], w.scale)
        np.testing.assert_array_equal(one[0][0], out[b])
        np.testing.assert_array_equal(one[1][0], lse[b])


def test_context_bound_status():
    w = make_custom(16, 3, 2, 1, 8, 50, "f32", [10, 20, 30], 4, trie_tokens=False,
                    kv_capacity=64, max_ctx=25)
    out, lse, st = oracle.tree_attention(w.q, w.k, w.v, "f32", [10, 20, 30], w.n_nodes,
                                         w.parent, w.scale, max_ctx=25, kv_capacity=64)
    assert st.tolist() == [0, 0, oracle.ROW_CTX_BOUND]
    assert np.all(out[2] == 0) and np.all(lse[2] == -np.inf)
    out, lse, st = oracle.tree_attention(w.q, w.k, w.v, "f32", [10, 61, 3], w.n_nodes,
                                         w.parent, w.scale, kv_capacity=64)
    assert st.tolist() == [0, oracle.ROW_CTX_BOUND, 0]


def test_bf16_decoding_is_exact():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x8000, 0x7FC0], np.uint16)
    d = oracle.decode(bits, "bf16")
    assert d[0] == 1.0 and d[1] == -2.0
    assert d[2] == 2.0 ** -133
    assert d[3] == (2 - 2 ** -7) * 2.0 ** 127
    assert d[4] == 0.0 and math.copysign(1, d[4]) < 0
    assert np.isnan(d[5])
