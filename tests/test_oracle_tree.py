"""Pins for the oracle's tree masks (CPU only).

Closed forms (chain, star), the hand-worked fixture, and a second formulation
(the recurrence mask[i] = mask[parent[i]] | bit(i)) that the oracle does not
use: it follows parent links instead.
"""

import json
import os

import numpy as np
import pytest

import oracle
from workloads import random_tree


def _bits(mask_row, T):
    return [bool((int(mask_row[j // 32]) >> (j % 32)) & 1) for j in range(T)]


def test_golden_hand_masks(golden_dir):
    with open(os.path.join(golden_dir, "tree_mask_hand.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        T = case["T"]
        if "parent" in case:
            parent = np.array([case["parent"]], np.int32)
        else:
            parent = np.arange(-1, T - 1, dtype=np.int32)[None]
        mask, depth, status = oracle.build_tree_mask(parent, np.array([case["n_nodes"]]), T)
        assert status[0] == oracle.ROW_OK
        if "mask_word0" in case:
            assert mask[0, :, 0].tolist() == case["mask_word0"]
            assert depth[0].tolist() == case["depth"]
        else:
            i = case["row"]
            assert mask[0, i].tolist() == case["mask_words"]
            assert depth[0, i] == case["depth_row"]


@pytest.mark.parametrize("T", [1, 2, 9, 33, 64, 65, 128])
def test_chain_is_lower_triangular(T):
    parent = np.arange(-1, T - 1, dtype=np.int32)[None]
    mask, depth, status = oracle.build_tree_mask(parent, np.array([T]), T)
    assert status[0] == 0
    dense = np.array([_bits(mask[0, i], T) for i in range(T)])
    assert np.array_equal(dense, np.tril(np.ones((T, T), bool)))
    assert depth[0].tolist() == list(range(T))


@pytest.mark.parametrize("T", [2, 9, 33, 100])
def test_star_is_diagonal_plus_root_column(T):
    parent = np.zeros((1, T), np.int32)
    parent[0, 0] = -1
    mask, depth, _ = oracle.build_tree_mask(parent, np.array([T]), T)
    dense = np.array([_bits(mask[0, i], T) for i in range(T)])
    want = np.eye(T, dtype=bool)
    want[:, 0] = True
    assert np.array_equal(dense, want)
    assert depth[0, 0] == 0 and np.all(depth[0, 1:] == 1)


@pytest.mark.parametrize("seed", range(6))
def test_matches_recurrence_and_popcount(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(2, 129))
    if seed % 2:  # bushy: at most 2..6 children, deep enough to hold T nodes
        parent = random_tree(rng, T - 1, max_depth=int(rng.integers(7, 13)),
                             max_children=int(rng.integers(2, 7)))
    else:
        parent = random_tree(rng, T - 1, max_depth=int(rng.integers(1, 13)))
    mask, depth, status = oracle.build_tree_mask(parent[None], np.array([T]), T)
    assert status[0] == 0
    W = (T + 31) // 32
    # Second formulation: a node's mask is its parent's mask plus its own bit.
    rec = np.zeros((T, W), np.uint64)
    rec[0, 0] = 1
    for i in range(1, T):
        rec[i] = rec[parent[i]]
        rec[i, i // 32] |= np.uint64(1) << np.uint64(i % 32)
    assert np.array_equal(mask[0].astype(np.uint64), rec)
    pop = [sum(bin(int(w)).count("1") for w in mask[0, i]) for i in range(T)]
    assert pop == (depth[0] + 1).tolist()


def test_status_and_padding():
    T = 5
    parent = np.array([[-1, 0, 0, 1, 2],       # fine
                       [-1, 0, 2, 1, 0],       # parent[2] = 2 is not < 2
                       [-1, 0, 0, 1, 2],       # n_nodes = 0
                       [-1, 0, 0, 1, 2],       # n_nodes = 6 > T
                       [-1, 0, -1, 7, 9]], np.int32)  # only 2 live rows: fine
    n = np.array([5, 5, 0, 6, 2])
    mask, depth, status = oracle.build_tree_mask(parent, n, T)
    assert status.tolist() == [oracle.ROW_OK, oracle.ROW_BAD_PARENT, oracle.ROW_OK,
                               oracle.ROW_NNODES, oracle.ROW_OK]
    for b in (1, 2, 3):
        assert not mask[b].any() and np.all(depth[b] == -1)
    assert mask[4, :, 0].tolist() == [1, 3, 0, 0, 0]
    assert depth[4].tolist() == [0, 1, -1, -1, -1]
