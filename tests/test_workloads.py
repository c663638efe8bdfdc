"""The seeded generators produce the measured workloads' shapes and structure."""

import numpy as np
import pytest

from workloads import bf16_bits_from_f32, make_config, make_custom


def _depth(parent_row, n):
    d = [0] * n
    for i in range(1, n):
        d[i] = d[parent_row[i]] + 1
    return d


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20,
                  -2.5, np.inf, np.nan], np.float32)
    bits = bf16_bits_from_f32(x)
    assert bits.tolist()[:6] == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x7F80]
    assert bits[6] == 0x7FC0


@pytest.mark.parametrize("name", ["C1", "C2", "C5"])
def test_config_shapes_and_poison(name):
    w = make_config(name)
    assert w.q.shape == (w.B, w.T, w.Hq, w.D)
    assert w.k.shape == (w.B, w.Hkv, w.kv_capacity, w.D) == w.v.shape
    assert w.logits.shape == (w.B, w.T, w.V)
    assert w.kv_capacity % 64 == 0 and w.kv_capacity >= w.max_ctx + w.T
    isnan = (lambda a: np.isnan(a)) if w.dtype == "f32" else (lambda a: a == 0x7FC0)
    for b in range(w.B):
        n = int(w.n_nodes[b])
        live = int(w.ctx_len[b]) + n
        assert not isnan(w.k[b, :, :live]).any() and isnan(w.k[b, :, live:]).all()
        assert not isnan(w.v[b, :, :live]).any() and isnan(w.v[b, :, live:]).all()
        assert np.all(np.isfinite(w.logits[b, :n])) and np.isnan(w.logits[b, n:]).all()
        d = _depth(w.parent[b], n)
        assert all(w.parent[b, i] < i for i in range(1, n))
        assert max(d) <= {"C1": 4, "C2": 8, "C5": 8}[name]
    if name == "C5":
        assert w.mode == "sample" and w.qdraft.shape == w.logits.shape
        assert np.isnan(w.qdraft[:, 0]).all()
        np.testing.assert_allclose(w.qdraft[:, 1:].astype(np.float64).sum(-1), 1.0, atol=1e-5)
        assert np.all((w.u >= 0) & (w.u < 1))


def test_c1_fixed_sizes():
    w = make_config("C1")
    assert (w.B, w.Hq, w.Hkv, w.D, w.T, w.V, w.dtype) == (1, 8, 2, 64, 9, 512, "f32")
    assert w.ctx_len.tolist() == [256]


def test_trie_siblings_distinct_and_planting():
    w = make_custom(5, 4, 4, 2, 16, 100, "bf16", [16] * 4, 32, plant_depth=4, padded_rows=[2])
    for b in range(4):
        n = int(w.n_nodes[b])
        for p in range(n):
            toks = [int(w.tokens[b, c]) for c in range(1, n) if w.parent[b, c] == p]
            assert len(toks) == len(set(toks))
    assert sorted(w.planted) == [0, 1, 3]
    assert w.n_nodes.tolist() == [33, 33, 0, 33]
    for b, path in w.planted.items():
        assert len(path) == 5 and path[0] == 0
        assert all(w.parent[b, path[j]] == path[j - 1] for j in range(1, 5))


def test_trie_needs_a_token_per_sibling():
    # 20 children of the root and 19 tokens: no trie exists; the generator
    # says so instead of drawing forever.
    with pytest.raises(ValueError, match="more children than vocabulary"):
        make_custom(7, 1, 2, 1, 16, 19, "bf16", [4], 20, tree="star")
    w = make_custom(7, 1, 2, 1, 16, 20, "bf16", [4], 20, tree="star")
    assert sorted(w.tokens[0, 1:].tolist()) == list(range(20))


def test_bushy_tree_limits():
    w = make_custom(6, 1, 4, 2, 16, 100, "bf16", [16], 64, max_depth=12, max_children=6)
    par = w.parent[0]
    counts = np.bincount(par[1:], minlength=65)
    assert counts.max() <= 6
    assert max(_depth(par, 65)) <= 12


def test_generation_is_deterministic():
    a = make_config("C1")
    b = make_config("C1")
    for f in ("q", "k", "v", "logits", "parent", "tokens"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
