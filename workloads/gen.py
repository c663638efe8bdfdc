"""Seeded synthetic workloads for draft-tree verification.

The shapes and value distributions follow the five workloads the verification
path is measured on (a 1-row fp32 case, three bf16 greedy cases of growing
context, and one bf16 sampling case). The pages these workloads stand in for
measured on R2R/RxR replays that are not available here; every input is drawn
from NumPy's PCG64 generator with a fixed seed instead.

Conventions shared by every consumer:

* A tree has ``T = N + 1`` rows per sequence. Row 0 is the root (the last
  accepted token); rows ``1..N`` are draft nodes with ``parent[i] < i``.
  ``n_nodes[b]`` counts the live rows of sequence ``b`` (root included);
  ``n_nodes[b] == 0`` marks a fully padded sequence.
* Query heads ``h`` read KV head ``h // (Hq // Hkv)``.
* The KV cache is ``[B][Hkv][kv_capacity][D]``; the committed context of row
  ``b`` is slots ``[0, ctx_len[b])`` and the tree's own keys/values sit in
  slots ``[ctx_len[b], ctx_len[b] + n_nodes[b])``.
* Everything a correct consumer must never read is poisoned with NaN: cache
  slots past the live extent, every slot of a padded sequence, query rows,
  logits rows and draft-probability rows of padding nodes, the unused draft
  row 0 and the uniforms of padding nodes.
* bf16 tensors are stored as their raw 16-bit patterns (``uint16``), rounded
  to nearest-even from float32.

Nothing in this module evaluates the method itself: it builds trees, draws
numbers, and (for the greedy workloads) raises a few logits so that a known
root-to-leaf path is the argmax path by construction.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

CONFIG_NAMES = ("C1", "C2", "C3", "C4", "C5")


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    nan = np.isnan(x)
    u = x.view(np.uint32).copy()
    u[nan] = 0
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF) + lsb
    out = (u >> np.uint32(16)).astype(np.uint16)
    out[nan] = np.uint16(0x7FC0)
    return out


@dataclass
class Workload:
    name: str
    seed: int
    B: int
    T: int
    Hq: int
    Hkv: int
    D: int
    V: int
    dtype: str  # storage type of q/k/v: "f32" or "bf16"
    scale: np.float32
    ctx_len: np.ndarray  # int32 [B]
    n_nodes: np.ndarray  # int32 [B]
    max_ctx: int
    kv_capacity: int
    parent: np.ndarray  # int32 [B, T]; -1 at the root and at padding rows
    tokens: np.ndarray  # int32 [B, T]; -1 at padding rows
    q: np.ndarray  # [B, T, Hq, D] float32, or uint16 bf16 bits
    k: np.ndarray  # [B, Hkv, kv_capacity, D]
    v: np.ndarray  # [B, Hkv, kv_capacity, D]
    logits: np.ndarray  # float32 [B, T, V]
    mode: str  # "greedy" or "sample"
    temperature: Optional[np.float32] = None
    qdraft: Optional[np.ndarray] = None  # float32 [B, T, V]; row 0 unused
    u: Optional[np.ndarray] = None  # float32 [B, T]; u[b, 0] is the final draw
    planted: Dict[int, List[int]] = field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def live_rows(self) -> int:
        return int(np.count_nonzero(self.n_nodes))

    @property
    def draft_nodes(self) -> int:
        """Draft nodes to verify (live rows minus their roots)."""
        n = self.n_nodes.astype(np.int64)
        return int(np.sum(np.maximum(n - 1, 0)))


def random_tree(
    rng: np.random.Generator,
    n_draft: int,
    max_depth: int,
    max_children: Optional[int] = None,
) -> np.ndarray:
    """Topologically ordered random tree of ``n_draft + 1`` nodes.

    Node ``i >= 1`` picks its parent uniformly among the earlier nodes whose
    depth is below ``max_depth`` (and, if given, that have fewer than
    ``max_children`` children). The root is node 0 with parent -1.
    """
    T = n_draft + 1
    parent = np.full(T, -1, dtype=np.int32)
    depth = np.zeros(T, dtype=np.int64)
    nchild = np.zeros(T, dtype=np.int64)
    for i in range(1, T):
        ok = depth[:i] < max_depth
        if max_children is not None:
            ok &= nchild[:i] < max_children
        cand = np.flatnonzero(ok)
        if cand.size == 0:
            raise ValueError("tree constraints leave no parent for node %d" % i)
        j = int(cand[rng.integers(cand.size)])
        parent[i] = j
        depth[i] = depth[j] + 1
        nchild[j] += 1
    return parent


def _depths(parent: np.ndarray) -> np.ndarray:
    depth = np.zeros(parent.shape[0], dtype=np.int64)
    for i in range(1, parent.shape[0]):
        depth[i] = depth[parent[i]] + 1
    return depth


def _children(parent: np.ndarray, node: int) -> np.ndarray:
    return np.flatnonzero(parent == node)


def _draw_trie_tokens(rng, parent, V):
    """Tokens with distinct values among siblings (a trie). A node with more
    children than vocabulary entries has no such tokens: ValueError."""
    T = parent.shape[0]
    tok = np.empty(T, dtype=np.int32)
    tok[0] = rng.integers(V)
    for i in range(1, T):
        taken = {int(tok[c]) for c in range(1, i) if parent[c] == parent[i]}
        if len(taken) >= V:
            raise ValueError("a node has more children than vocabulary entries: no trie tokens")
        while True:
            t = int(rng.integers(V))
            if t not in taken:
                break
        tok[i] = t
    return tok


def _normal_f32(rng, shape, sigma=1.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def _plant_path(rng, parent, tok, logits_row_block, depth_goal):
    """Raise logits so a random root-to-leaf path is the greedy path to depth_goal.

    Picks a uniformly random leaf of depth >= depth_goal (returns None when the
    tree has none). With n_0 = root and n_1..n_k its ancestors at depths 1..k,
    row n_{j-1} gets ``max(row) + 1`` at token ``tok[n_j]``; row n_k gets every
    child token pushed to ``min(row) - 1`` so that no child of n_k can match
    its argmax. Sibling tokens must be distinct (a trie), so each planted
    argmax selects exactly one child.
    """
    T = parent.shape[0]
    depth = _depths(parent)
    is_leaf = np.ones(T, dtype=bool)
    is_leaf[parent[1:]] = False
    cand = np.flatnonzero(is_leaf & (depth >= depth_goal))
    if cand.size == 0:
        return None
    leaf = int(cand[rng.integers(cand.size)])
    chain = [leaf]
    while chain[-1] != 0:
        chain.append(int(parent[chain[-1]]))
    chain = chain[::-1]  # root .. leaf, chain[d] has depth d
    path = chain[: depth_goal + 1]
    for j in range(1, depth_goal + 1):
        row = logits_row_block[path[j - 1]]
        row[tok[path[j]]] = row.max() + np.float32(1.0)
    last = logits_row_block[path[depth_goal]]
    low = last.min() - np.float32(1.0)
    for c in _children(parent, path[depth_goal]):
        last[tok[c]] = low
    return path


def make_custom(
    seed: int,
    B: int,
    Hq: int,
    Hkv: int,
    D: int,
    V: int,
    dtype: str,
    ctx_len: Sequence[int],
    n_draft: int,
    *,
    name: str = "custom",
    tree: str = "random",
    parents: Optional[Sequence[Sequence[int]]] = None,
    max_depth: int = 8,
    max_children: Optional[int] = None,
    trie_tokens: bool = True,
    logit_sigma: float = 3.0,
    plant_depth: int = 0,
    padded_rows: Sequence[int] = (),
    n_nodes: Optional[Sequence[int]] = None,
    mode: str = "greedy",
    temperature: float = 0.7,
    kv_capacity: Optional[int] = None,
    max_ctx: Optional[int] = None,
    nan_poison: bool = True,
) -> Workload:
    """Draw one workload.

    ``tree`` is "random" (see :func:`random_tree`), "chain" (node i's parent is
    i-1), "star" (every draft node hangs off the root) or "explicit" (take
    ``parents``, one parent array of length ``n_draft + 1`` per row).
    ``n_nodes`` overrides the live row count per sequence (default: the full
    tree, ``n_draft + 1``); ``padded_rows`` lists sequences set to zero live
    rows after everything has been drawn.
    """
    rng = np.random.default_rng(seed)
    T = n_draft + 1
    ctx = np.asarray(ctx_len, dtype=np.int32).reshape(B)
    if dtype not in ("f32", "bf16"):
        raise ValueError(dtype)
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")

    parent = np.full((B, T), -1, dtype=np.int32)
    tokens = np.full((B, T), -1, dtype=np.int32)
    logits = None
    qdraft = None
    planted: Dict[int, List[int]] = {}

    if mode == "greedy":
        logits = np.empty((B, T, V), dtype=np.float32)
    for b in range(B):
        while True:
            if tree == "random":
                par = random_tree(rng, n_draft, max_depth, max_children)
            elif tree == "chain":
                par = np.arange(-1, T - 1, dtype=np.int32)
            elif tree == "star":
                par = np.zeros(T, dtype=np.int32)
                par[0] = -1
            elif tree == "explicit":
                par = np.asarray(parents[b], dtype=np.int32).copy()
            else:
                raise ValueError(tree)
            if mode == "greedy":
                if trie_tokens:
                    tok = _draw_trie_tokens(rng, par, V)
                else:
                    tok = rng.integers(0, V, size=T).astype(np.int32)
                block = _normal_f32(rng, (T, V), logit_sigma)
                if plant_depth > 0:
                    path = _plant_path(rng, par, tok, block, plant_depth)
                    if path is None:
                        if tree != "random":
                            raise ValueError("tree has no leaf deep enough to plant")
                        continue
                    planted[b] = path
                logits[b] = block
            else:
                tok = None
            parent[b] = par
            if tok is not None:
                tokens[b] = tok
            break

    temp = None
    u = None
    if mode == "sample":
        temp = np.float32(temperature)
        tau = np.float64(temp)
        logits = _normal_f32(rng, (B, T, V), logit_sigma)
        qdraft = np.full((B, T, V), np.nan, dtype=np.float32)
        for b in range(B):
            tokens[b, 0] = rng.integers(V)
            for i in range(1, T):
                eps = rng.standard_normal(V)
                z = (logits[b, parent[b, i]].astype(np.float64) + eps) / tau
                z -= z.max()
                e = np.exp(z)
                qi = e / e.sum()
                qdraft[b, i] = qi.astype(np.float32)
                qs = qdraft[b, i].astype(np.float64)
                tokens[b, i] = rng.choice(V, p=qs / qs.sum())
        u = rng.random((B, T), dtype=np.float32)
    elif mode != "greedy":
        raise ValueError(mode)

    nn = np.full(B, T, dtype=np.int32) if n_nodes is None else np.asarray(n_nodes, np.int32).copy()
    for b in padded_rows:
        nn[b] = 0
    if max_ctx is None:
        max_ctx = int(ctx.max()) if B else 0
    if kv_capacity is None:
        kv_capacity = ((max_ctx + T + 63) // 64) * 64

    qf = _normal_f32(rng, (B, T, Hq, D))
    kf = _normal_f32(rng, (B, Hkv, kv_capacity, D))
    vf = _normal_f32(rng, (B, Hkv, kv_capacity, D))

    if nan_poison:
        for b in range(B):
            n = int(nn[b])
            live = int(ctx[b]) + n if n > 0 else 0
            kf[b, :, live:, :] = np.nan
            vf[b, :, live:, :] = np.nan
            qf[b, n:] = np.nan
            logits[b, n:] = np.nan
            if qdraft is not None:
                qdraft[b, 0] = np.nan
                qdraft[b, n:] = np.nan
            if u is not None and n == 0:
                u[b, :] = np.nan
            elif u is not None:
                u[b, n:] = np.nan
    for b in range(B):
        n = int(nn[b])
        parent[b, max(n, 1):] = -1
        if n == 0:
            parent[b, :] = -1
        tokens[b, n:] = -1

    if dtype == "bf16":
        q = bf16_bits_from_f32(qf)
        k = bf16_bits_from_f32(kf)
        v = bf16_bits_from_f32(vf)
    else:
        q, k, v = qf, kf, vf

    return Workload(
        name=name,
        seed=seed,
        B=B,
        T=T,
        Hq=Hq,
        Hkv=Hkv,
        D=D,
        V=V,
        dtype=dtype,
        scale=np.float32(1.0 / np.sqrt(D)),
        ctx_len=ctx,
        n_nodes=nn,
        max_ctx=int(max_ctx),
        kv_capacity=int(kv_capacity),
        parent=parent,
        tokens=tokens,
        q=q,
        k=k,
        v=v,
        logits=logits,
        mode=mode,
        temperature=temp,
        qdraft=qdraft,
        u=u,
        planted={b: p for b, p in planted.items() if nn[b] > 0},
    )


def make_config(name: str, seed: Optional[int] = None) -> Workload:
    """The five measured workloads; the seed defaults to the config number."""
    if name not in CONFIG_NAMES:
        raise ValueError("unknown config %r" % (name,))
    if seed is None:
        seed = int(name[1:])
    rng = np.random.default_rng(seed + 1000)
    if name == "C1":
        # 1 sequence, 8/2 heads, D=64, fp32, context 256, 8 draft nodes of
        # depth <= 4, tokens uniform in a 512-word vocabulary, logits N(0, 2).
        return make_custom(seed, 1, 8, 2, 64, 512, "f32", [256], 8, name=name,
                           max_depth=4, trie_tokens=False, logit_sigma=2.0)
    if name == "C2":
        ctx = rng.integers(1024, 2048, size=4, endpoint=True)
        return make_custom(seed, 4, 28, 4, 128, 152064, "bf16", ctx, 32, name=name,
                           max_depth=8, logit_sigma=3.0, plant_depth=4)
    if name == "C3":
        ctx = rng.integers(4096, 8192, size=8, endpoint=True)
        padded = sorted(rng.choice(8, size=2, replace=False).tolist())
        return make_custom(seed, 8, 28, 4, 128, 152064, "bf16", ctx, 32, name=name,
                           max_depth=8, logit_sigma=3.0, plant_depth=4,
                           padded_rows=padded)
    if name == "C4":
        return make_custom(seed, 1, 28, 4, 128, 152064, "bf16", [32768], 64, name=name,
                           max_depth=12, max_children=6, logit_sigma=3.0, plant_depth=4)
    # C5: sampling.
    ctx = rng.integers(2048, 4096, size=8, endpoint=True)
    return make_custom(seed, 8, 28, 4, 128, 32000, "bf16", ctx, 32, name=name,
                       max_depth=8, logit_sigma=3.0, mode="sample", temperature=0.7)
