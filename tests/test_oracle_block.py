"""Pins of the draft-block masks (oracle/block.py) and of the explicit-mask
attention oracle, no GPU.

* hand-derived words for a three-row block (causal: row i sees rows 0..i;
  bidirectional: every live row sees every live row);
* the causal block mask equals the tree mask of a chain tree, built by the
  tree oracle from parent links (another formulation);
* bidirectional block attention equals torch's CPU scaled_dot_product_attention
  in float64 over all ctx_len + n keys with no mask; causal block attention
  equals it with the causal offset mask (row i sees slots < ctx_len + i + 1)
  and equals tree attention of a chain tree;
* status for n_nodes outside [0, T];
* a row that sees no key (explicit mask, empty context): out 0, lse -inf,
  and the other rows equal SDPA over exactly their own visible keys.
"""

import numpy as np
import torch

import oracle
from oracle.decode import decode
from workloads import make_custom


def test_hand_words():
    # T = 5, two sequences with 3 and 0 live rows. Causal: row 0 -> {0} = 1,
    # row 1 -> {0,1} = 3, row 2 -> {0,1,2} = 7. Bidirectional: rows 0..2 ->
    # {0,1,2} = 7. Padding rows 0.
    m, pos, st = oracle.build_block_mask(np.array([3, 0]), 5, oracle.CAUSAL)
    assert m[0, :, 0].tolist() == [1, 3, 7, 0, 0] and not m[1].any()
    assert pos[0].tolist() == [0, 1, 2, -1, -1] and pos[1].tolist() == [-1] * 5
    m, pos, st = oracle.build_block_mask(np.array([3, 0]), 5, oracle.BIDIRECTIONAL)
    assert m[0, :, 0].tolist() == [7, 7, 7, 0, 0] and not m[1].any()
    # T = 40: row 35 of a full causal block covers word 0 and bits 0..3 of word 1.
    m, _, _ = oracle.build_block_mask(np.array([40]), 40, oracle.CAUSAL)
    assert m[0, 35].tolist() == [0xFFFFFFFF, 0xF]
    m, _, _ = oracle.build_block_mask(np.array([37]), 40, oracle.BIDIRECTIONAL)
    assert m[0, 0].tolist() == [0xFFFFFFFF, 0x1F] and not m[0, 37:].any()


def test_causal_equals_chain_tree():
    for T in (1, 9, 33, 64, 100, 128):
        n = np.array([T, T // 2, 0, 1])
        parent = np.tile(np.arange(-1, T - 1, dtype=np.int32), (4, 1))
        m_tree, depth, st_tree = oracle.build_tree_mask(parent, n, T)
        m_blk, pos, st = oracle.build_block_mask(n, T, oracle.CAUSAL)
        assert np.array_equal(m_tree, m_blk) and np.array_equal(depth, pos)
        assert not st.any() and not st_tree.any()


def _sdpa(qv, kv, vv, scale, attn_mask=None):
    q = torch.from_numpy(qv[None, None, None, :])
    k = torch.from_numpy(kv[None, None])
    v = torch.from_numpy(vv[None, None])
    m = None if attn_mask is None else torch.from_numpy(attn_mask[None, None, None, :])
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m,
                                                            scale=scale).numpy()[0, 0, 0]


def test_block_attention_against_sdpa():
    w = make_custom(61, 3, 6, 2, 64, 50, "bf16", [45, 0, 70], 11, tree="chain",
                    trie_tokens=False, padded_rows=[])
    qf, kf, vf = decode(w.q, w.dtype), decode(w.k, w.dtype), decode(w.v, w.dtype)
    for mode in (oracle.CAUSAL, oracle.BIDIRECTIONAL):
        mask, _, _ = oracle.build_block_mask(w.n_nodes, w.T, mode)
        out, lse, st = oracle.masked_attention(w.q, w.k, w.v, w.dtype, w.ctx_len, w.n_nodes,
                                               mask, w.scale)
        assert not st.any()
        for b in range(w.B):
            L, n = int(w.ctx_len[b]), int(w.n_nodes[b])
            for i in range(n):
                keys = L + (i + 1 if mode == oracle.CAUSAL else n)
                for h in range(w.Hq):
                    g = h // w.G
                    ref = _sdpa(qf[b, i, h], kf[b, g, :keys], vf[b, g, :keys], float(w.scale))
                    assert np.abs(out[b, i, h] - ref).max() < 1e-12
        if mode == oracle.CAUSAL:
            out_t, lse_t, _ = oracle.tree_attention(w.q, w.k, w.v, w.dtype, w.ctx_len, w.n_nodes,
                                                    w.parent, w.scale)
            assert np.array_equal(out, out_t) and np.array_equal(lse, lse_t)


def test_status():
    m, pos, st = oracle.build_block_mask(np.array([5, -1, 2]), 4, oracle.BIDIRECTIONAL)
    assert st.tolist() == [oracle.ROW_NNODES, oracle.ROW_NNODES, 0]
    assert not m[:2].any() and (pos[:2] == -1).all()


def test_row_without_visible_keys():
    # Explicit masks over an empty committed context: row 0 sees nothing, row
    # 35 sees only keys 33 and 35 (none of keys 0..31), row 36 sees every key.
    w = make_custom(63, 1, 4, 2, 64, 50, "bf16", [0], 39, tree="chain", trie_tokens=False,
                    padded_rows=[])
    n = int(w.n_nodes[0])
    assert n == 40 and int(w.ctx_len[0]) == 0
    mask, _, _ = oracle.build_block_mask(w.n_nodes, w.T, oracle.CAUSAL)
    mask[0, 0] = 0
    mask[0, 35] = [0, (1 << 1) | (1 << 3)]
    mask[0, 36] = [0xFFFFFFFF, 0xFF]
    out, lse, st = oracle.masked_attention(w.q, w.k, w.v, w.dtype, w.ctx_len, w.n_nodes, mask,
                                           w.scale)
    assert not st.any()
    assert np.all(out[0, 0] == 0.0) and np.all(lse[0, 0] == -np.inf)
    qf, kf, vf = decode(w.q, w.dtype), decode(w.k, w.dtype), decode(w.v, w.dtype)
    for i, keys in ((35, [33, 35]), (36, list(range(40))), (7, list(range(8)))):
        for h in range(w.Hq):
            g = h // w.G
            ref = _sdpa(qf[0, i, h], kf[0, g, keys], vf[0, g, keys], float(w.scale))
            assert np.abs(out[0, i, h] - ref).max() < 1e-12
            s = float(w.scale) * (kf[0, g, keys] @ qf[0, i, h])
            assert abs(lse[0, i, h] - (s.max() + np.log(np.exp(s - s.max()).sum()))) < 1e-12
