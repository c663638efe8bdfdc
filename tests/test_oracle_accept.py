"""Pins for the oracle's greedy and sampling acceptance (CPU only).

Greedy: hand-worked fixtures, planted workloads (accept_len = 4 by
construction), a chain-tree cumulative-product formulation and a second,
data-parallel formulation of the accepted path on many random trees.

Sampling: hand-worked fixtures; brute force over every draft tuple of a
4-token vocabulary showing that the rule as specified emits p exactly (so a
wrong residual, ratio or order fails); a chi-square test of the oracle's own
draws against p and against p_c after accepting c; closed forms for one-hot
drafts (sampling without replacement) and for drafts equal to the target.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
from workloads import make_custom


def _f(x):
    return float(x) if not isinstance(x, str) else float(x)


# ---------------------------------------------------------------- greedy ---

def test_golden_greedy(golden_dir):
    with open(os.path.join(golden_dir, "greedy_hand.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        T = len(c["parent"])
        logits = np.array([[_f(x) for x in row] for row in c["logits"]], np.float32)[None]
        al, path, bonus, am, st = oracle.accept_greedy(
            logits, np.array([c["tokens"]]), np.array([c["parent"]]), np.array([T]))
        assert st[0] == 0, c["name"]
        assert al[0] == c["accept_len"], c["name"]
        assert path[0].tolist() == c["path"], c["name"]
        assert bonus[0] == c["bonus"], c["name"]
        assert am[0].tolist() == c["accept_mask"], c["name"]


def test_signed_zero_fixture_really_holds_negative_zero(golden_dir):
    with open(os.path.join(golden_dir, "greedy_hand.json")) as f:
        c = json.load(f)["cases"][1]
    v = np.float32(_f(c["logits"][2][0]))
    assert v == 0 and math.copysign(1.0, float(v)) < 0


@pytest.mark.parametrize("seed", [21, 22, 23])
def test_planted_path_is_accepted(seed):
    w = make_custom(seed, 3, 4, 2, 16, 3000, "bf16", [8, 8, 8], 32, max_depth=8,
                    plant_depth=4, padded_rows=[1])
    al, path, bonus, am, st = oracle.accept_greedy(w.logits, w.tokens, w.parent, w.n_nodes)
    assert np.all(st == 0)
    for b, planted in w.planted.items():
        assert al[b] == 4
        assert path[b, :5].tolist() == planted
        assert bonus[b] == int(np.argmax(w.logits[b, planted[-1]]))
    assert al[1] == 0 and bonus[1] == -1 and np.all(path[1] == -1) and not am[1].any()


@pytest.mark.parametrize("seed", range(5))
def test_chain_tree_cumprod_form(seed):
    """On a chain the accepted length is sum(cumprod(tok[k] == argmax(l[k-1])))."""
    rng = np.random.default_rng(seed)
    T, V = 12, 3
    logits = rng.standard_normal((1, T, V)).astype(np.float32)
    tokens = rng.integers(0, V, size=(1, T)).astype(np.int32)
    parent = np.arange(-1, T - 1, dtype=np.int32)[None]
    al, path, bonus, am, _ = oracle.accept_greedy(logits, tokens, parent, np.array([T]))
    match = tokens[0, 1:] == np.argmax(logits[0, :-1], axis=1)
    n_acc = int(np.cumprod(match).sum())
    assert al[0] == n_acc
    assert bonus[0] == int(np.argmax(logits[0, n_acc]))
    assert path[0].tolist() == list(range(n_acc + 1)) + [-1] * (T - n_acc - 1)


@pytest.mark.parametrize("seed", range(40))
def test_greedy_second_formulation(seed):
    """Data-parallel form: a node is on the path iff every node from it up to
    (not including) the root matches its parent's argmax and is the
    lowest-index matching child among its siblings."""
    rng = np.random.default_rng(100 + seed)
    T = int(rng.integers(1, 40))
    V = int(rng.integers(2, 5))
    parent = np.full(T, -1, np.int32)
    for i in range(1, T):
        parent[i] = rng.integers(0, i)
    tokens = rng.integers(0, V, size=T).astype(np.int32)
    # small integers make ties frequent; argmax ties break to the lowest index
    logits = rng.integers(-2, 3, size=(T, V)).astype(np.float32)
    arg = np.argmax(logits, axis=1)  # numpy: first occurrence of the maximum
    match = np.zeros(T, bool)
    match[1:] = tokens[1:] == arg[parent[1:]]
    first = np.zeros(T, bool)
    for c in range(1, T):
        sib = [s for s in range(1, c) if parent[s] == parent[c] and match[s]]
        first[c] = match[c] and not sib
    on_path = np.zeros(T, bool)
    on_path[0] = True
    for c in range(1, T):
        on_path[c] = first[c] and on_path[parent[c]]
    al, path, bonus, am, st = oracle.accept_greedy(logits[None], tokens[None], parent[None],
                                                   np.array([T]))
    assert st[0] == 0
    assert am[0].astype(bool).tolist() == on_path.tolist()
    assert al[0] == on_path.sum() - 1
    deepest = int(np.flatnonzero(on_path).max())  # indices grow along any root path
    assert bonus[0] == arg[deepest]


def test_greedy_status_codes():
    T, V = 4, 10
    logits = np.zeros((4, T, V), np.float32)
    parent = np.array([[-1, 0, 1, 1], [-1, 0, 3, 1], [-1, 0, 0, 0], [-1, 0, 0, 0]], np.int32)
    tokens = np.array([[0, 1, 2, 3], [0, 1, 2, 3], [0, 1, 10, 3], [0, 1, 2, 3]], np.int32)
    al, path, bonus, am, st = oracle.accept_greedy(logits, tokens, parent, np.array([4, 4, 4, 5]))
    assert st.tolist() == [oracle.ROW_OK, oracle.ROW_BAD_PARENT, oracle.ROW_BAD_TOKEN,
                           oracle.ROW_NNODES]
    for b in (1, 2, 3):
        assert al[b] == 0 and bonus[b] == -1 and np.all(path[b] == -1) and not am[b].any()


# -------------------------------------------------------------- sampling ---

def test_sample_probs_is_tempered_softmax():
    rng = np.random.default_rng(3)
    l = (3 * rng.standard_normal(1000)).astype(np.float32)
    for t in (0.7, 1.0, 1.3):
        tau = np.float64(np.float32(t))
        np.testing.assert_allclose(oracle.sample_probs(l, np.float32(t)),
                                   scipy.special.softmax(l.astype(np.float64) / tau),
                                   rtol=1e-12, atol=0)


def test_golden_sampling(golden_dir):
    with open(os.path.join(golden_dir, "sample_hand.json")) as f:
        g = json.load(f)
    V = g["V"]
    T = len(g["parent"])
    logits = np.log(np.array(g["p_rows"], np.float64)).astype(np.float32)[None]
    q = np.full((1, T, V), np.nan, np.float32)
    for i, row in enumerate(g["q_rows"]):
        if row is not None:
            q[0, i] = row
    for c in g["cases"]:
        res = oracle.accept_sample(logits, np.float32(g["temperature"]), q,
                                   np.array([c["u"]], np.float32), np.array([g["tokens"]]),
                                   np.array([g["parent"]]), np.array([T]))
        al, path, bonus, am, dec, st = res
        assert st[0] == 0
        assert al[0] == c["accept_len"], c["name"]
        assert path[0].tolist() == c["path"], c["name"]
        assert bonus[0] == c["bonus"], c["name"]
        assert dec[0].tolist() == c["decision"], c["name"]


def _analytic_first_token_law(p, qs):
    """Law of the first emitted token when a root with children 1..k (tested
    in order, child c's token drawn from qs[c]) is verified against p. Sums
    over every draft tuple; acceptance of a child happens with probability
    min(1, r(x)/q(x)); the bonus is drawn from the final residual."""
    V = p.shape[0]
    law = np.zeros(V)
    for xs in itertools.product(range(V), repeat=len(qs)):
        weight = np.prod([qs[c][xs[c]] for c in range(len(qs))])
        if weight == 0:
            continue
        r = p.copy()
        reach = 1.0
        for c, x in enumerate(xs):
            if r[x] == 0:
                a = 0.0
            elif qs[c][x] == 0:
                a = 1.0
            else:
                a = min(1.0, r[x] / qs[c][x])
            law[x] += weight * reach * a
            reach *= 1.0 - a
            res = np.maximum(r - qs[c], 0.0)
            if res.sum() > 0:
                r = res / res.sum()
        law += weight * reach * r
    return law


@pytest.mark.parametrize("k", [1, 2, 3])
@pytest.mark.parametrize("seed", range(4))
def test_rule_is_exact_by_brute_force(k, seed):
    rng = np.random.default_rng(seed * 10 + k)
    p = rng.dirichlet(np.ones(4))
    qs = [rng.dirichlet(np.ones(4) * 0.7) for _ in range(k)]
    law = _analytic_first_token_law(p, qs)
    np.testing.assert_allclose(law, p, rtol=0, atol=1e-12)


def _draw_rows(rng, nrows, p_root_logits, p_child_logits, qs, V, depth2):
    """A batch of independent verification rows sharing one tree shape."""
    k = len(qs)
    T = 1 + k + (k if depth2 else 0)
    parent = np.full(T, -1, np.int32)
    parent[1:k + 1] = 0
    if depth2:
        parent[k + 1:] = np.arange(1, k + 1)  # one grandchild under each child
    logits = np.empty((nrows, T, V), np.float32)
    logits[:, 0] = p_root_logits
    for c in range(1, T):
        logits[:, c] = p_child_logits[c]
    q = np.full((nrows, T, V), np.nan, np.float32)
    tokens = np.zeros((nrows, T), np.int32)
    for c in range(1, T):
        qc = qs[(c - 1) % k]
        q[:, c] = qc
        qq = q[0, c].astype(np.float64)
        tokens[:, c] = rng.choice(V, size=nrows, p=qq / qq.sum())
    u = rng.random((nrows, T), dtype=np.float32)
    return (logits, q, u, tokens, np.repeat(parent[None], nrows, 0),
            np.full(nrows, T, np.int32))


def test_oracle_draws_follow_target_chi_square():
    rng = np.random.default_rng(77)
    V, k, nrows = 4, 3, 30000
    root = np.log(rng.dirichlet(np.ones(V))).astype(np.float32)
    child = {c: np.log(rng.dirichlet(np.ones(V))).astype(np.float32) for c in range(1, 2 * k + 1)}
    qs = [rng.dirichlet(np.ones(V)).astype(np.float32) for _ in range(k)]
    logits, q, u, tokens, parent, n = _draw_rows(rng, nrows, root, child, qs, V, True)
    tau = np.float32(1.0)
    al, path, bonus, am, dec, st = oracle.accept_sample(logits, tau, q, u, tokens, parent, n)
    assert np.all(st == 0)
    first = np.where(al >= 1, tokens[np.arange(nrows), path[:, 1]], bonus)
    p_root = oracle.sample_probs(root, tau)
    counts = np.bincount(first, minlength=V)
    pval = scipy.stats.chisquare(counts, p_root * nrows).pvalue
    assert pval > 1e-3, (counts, p_root * nrows)
    # After accepting child c, the next emitted token follows p_c.
    for c in range(1, k + 1):
        sel = (al >= 1) & (path[:, 1] == c)
        nxt = np.where(al[sel] >= 2, tokens[np.flatnonzero(sel), path[sel, 2]], bonus[sel])
        counts = np.bincount(nxt, minlength=V)
        p_c = oracle.sample_probs(child[c], tau)
        pval = scipy.stats.chisquare(counts, p_c * counts.sum()).pvalue
        assert pval > 1e-3, (c, counts, p_c * counts.sum())


def test_one_hot_drafts_sample_without_replacement():
    """q_c = one-hot(x_c): the j-th child (distinct tokens) is accepted iff
    u_j < p(x_j) / (1 - sum_{i<j} p(x_i))."""
    V = 6
    p = np.array([0.05, 0.3, 0.1, 0.25, 0.2, 0.1])
    xs = [1, 3, 4]
    thr = [p[x] / (1 - sum(p[y] for y in xs[:j])) for j, x in enumerate(xs)]
    logits = np.log(p).astype(np.float32)[None, None].repeat(4, 1)
    T = 4
    parent = np.array([[-1, 0, 0, 0]])
    tokens = np.array([[0] + xs])
    q = np.zeros((1, T, V), np.float32)
    for j, x in enumerate(xs):
        q[0, j + 1, x] = 1.0
    for m in range(3):  # accept child m+1 after rejecting the earlier ones
        u = np.zeros((1, T), np.float32)
        for j in range(m):
            u[0, j + 1] = thr[j] * (1 + 1e-5)
        u[0, m + 1] = thr[m] * (1 - 1e-5)
        al, path, bonus, am, dec, st = oracle.accept_sample(
            logits, np.float32(1.0), q, u, tokens, parent, np.array([T]))
        assert dec[0, 1:m + 2].tolist() == [0] * m + [1]
        assert path[0, 1] == m + 1
    # Rejecting all three leaves p restricted to the other tokens.
    u = np.array([[0.5] + [t * (1 + 1e-5) for t in thr]], np.float32)
    al, path, bonus, am, dec, st = oracle.accept_sample(
        logits, np.float32(1.0), q, u, tokens, parent, np.array([T]))
    rest = p.copy()
    rest[xs] = 0
    rest /= rest.sum()
    assert al[0] == 0 and bonus[0] == int(np.searchsorted(np.cumsum(rest), 0.5, side="right"))


def test_duplicate_token_after_one_hot_rejection_is_rejected():
    """After rejecting x with a one-hot draft, r(x) = 0, so a sibling carrying
    the same token is rejected even with u = 0; q(x) = 0 < r(x) accepts."""
    V = 3
    p = np.array([0.5, 0.3, 0.2])
    logits = np.log(p).astype(np.float32)[None, None].repeat(4, 1)
    q = np.zeros((1, 4, V), np.float32)
    q[0, 1] = [1, 0, 0]
    q[0, 2] = [1, 0, 0]
    q[0, 3] = [0.5, 0.5, 0.0]
    tokens = np.array([[0, 0, 0, 2]])
    parent = np.array([[-1, 0, 0, 0]])
    u = np.array([[0.1, 0.9, 0.0, 0.999]], np.float32)
    al, path, bonus, am, dec, st = oracle.accept_sample(
        logits, np.float32(1.0), q, u, tokens, parent, np.array([4]))
    assert dec[0].tolist() == [-1, 0, 0, 1]
    assert path[0, :2].tolist() == [0, 3]


@pytest.mark.parametrize("seed", range(5))
def test_draft_equal_to_target_follows_first_children(seed):
    """q_c = p_parent(c): ratio 1 > u for every first child, so the walk takes
    the first child at every level down to a leaf and draws the bonus from
    p_leaf by inverse CDF."""
    rng = np.random.default_rng(seed)
    T, V = 12, 7
    parent = np.full(T, -1, np.int32)
    for i in range(1, T):
        parent[i] = rng.integers(0, i)
    logits = (2 * rng.standard_normal((T, V))).astype(np.float32)
    tau = np.float32(0.7)
    q = np.full((T, V), np.nan, np.float32)
    for i in range(1, T):
        q[i] = oracle.sample_probs(logits[parent[i]], tau)
    tokens = rng.integers(0, V, size=T).astype(np.int32)
    # q stored as float32 perturbs the ratio by ~1e-7; keep u clear of 1.
    u = (0.999 * rng.random(T)).astype(np.float32)
    al, path, bonus, am, dec, st = oracle.accept_sample(
        logits[None], tau, q[None], u[None], tokens[None], parent[None], np.array([T]))
    cur = 0
    want = [0]
    while True:
        kids = [c for c in range(1, T) if parent[c] == cur]
        if not kids:
            break
        cur = kids[0]
        want.append(cur)
    assert path[0, :len(want)].tolist() == want and al[0] == len(want) - 1
    p_leaf = oracle.sample_probs(logits[cur], tau)
    c = np.cumsum(p_leaf)
    assert bonus[0] == int(np.searchsorted(c, np.float64(u[0]) * c[-1], side="right"))
