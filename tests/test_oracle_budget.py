"""Pins for the oracle's adaptive draft budget (CPU only).

The pins: a three-step trajectory worked by hand with exact dyadic ratios
(every clamp, the dead band at the target and every skipped-sequence case
appear in it); the closed form of an exponential average under a constant
ratio; the closed loop of a known acceptance curve, whose fixed point is
known; and the prefix-sum row table checked against a direct count.
"""

import json
import os

import numpy as np

import oracle


def test_golden_hand_trajectory(golden_dir):
    with open(os.path.join(golden_dir, "budget_hand.json")) as f:
        g = json.load(f)
    ema = np.array(g["ema0"], np.float32)
    bud = np.array(g["budget0"], np.int32)
    for step in g["steps"]:
        ema, bud, start, total = oracle.adapt_tree_budget(
            step["accept_len"], step["n_nodes"], ema, bud, g["target"], g["alpha"],
            g["n_min"], g["n_max"], row_status=step["row_status"])
        assert ema.tolist() == step["ema"], step["why"]
        assert bud.tolist() == step["budget"], step["why"]
        assert start.tolist() == step["row_start"], step["why"]
        assert total == step["rows_total"], step["why"]


def test_constant_ratio_closed_form():
    # ratio 1/3 every step: e_k = r + (1 - alpha)^k (e_0 - r), to float32
    # rounding accumulated over k steps.
    alpha, e0, r = 0.3, 0.9, 1.0 / 3.0
    ema = np.array([e0], np.float32)
    bud = np.array([10], np.int32)
    for k in range(1, 61):
        ema, bud, _, _ = oracle.adapt_tree_budget([1], [4], ema, bud, 0.0, alpha, 1, 127)
        exact = r + (1 - alpha) ** k * (np.float32(e0) - r)
        assert abs(float(ema[0]) - exact) <= 4e-7 * k, k
        # target 0 and a positive average: the budget only grows, one per step.
        assert bud[0] == min(10 + k, 127)


def test_closed_loop_fixed_point():
    # Acceptance curve a(N) = min(N, c): ratio c / N for N >= c. With
    # alpha = 1 the average is the last ratio, so for target 1/2 the budget
    # climbs or falls to N = 2c, where the ratio equals the target, and stays.
    for c in (1, 3, 7, 20):
        for start in (1, 2 * c + 9, 60):
            ema = np.array([0.5], np.float32)
            bud = np.array([start], np.int32)
            hist = []
            for _ in range(80):
                N = int(bud[0])
                ema, bud, _, _ = oracle.adapt_tree_budget([min(N, c)], [N + 1], ema, bud, 0.5,
                                                          1.0, 1, 100)
                hist.append(int(bud[0]))
            assert hist[-20:] == [2 * c] * 20, (c, start, hist[-20:])


def test_budget_moves_toward_target_monotonically():
    # Acceptance ratio always 1 (every draft accepted) with target 0.75: the
    # budget rises each step until n_max; ratio 0 with target 0.25: falls to
    # n_min. The average never leaves [0, 1].
    ema = np.array([0.5, 0.5], np.float32)
    bud = np.array([5, 5], np.int32)
    for k in range(1, 12):
        n = [int(bud[0]) + 1, int(bud[1]) + 1]
        ema, bud, _, _ = oracle.adapt_tree_budget([n[0] - 1, 0], n, ema, bud, 0.5, 0.25, 2, 12)
        assert 0.0 <= ema.min() and ema.max() <= 1.0
        assert bud[0] == min(5 + k, 12) and bud[1] == max(5 - k, 2)


def test_row_table_counts_rows():
    rng = np.random.default_rng(7)
    B = 300
    bud = rng.integers(1, 64, B).astype(np.int32)
    n = np.zeros(B, np.int32)  # no updates: only the table
    ema, bud2, start, total = oracle.adapt_tree_budget(np.zeros(B, np.int32), n,
                                                       np.zeros(B, np.float32), bud, 0.5, 0.5,
                                                       1, 127)
    assert np.array_equal(bud2, bud)
    owner = np.full(total, -1)
    for b in range(B):
        assert np.all(owner[start[b]:start[b] + bud[b] + 1] == -1)
        owner[start[b]:start[b] + bud[b] + 1] = b
    assert np.all(owner >= 0)  # the rows tile [0, total) exactly
    assert total == int(bud.sum()) + B
